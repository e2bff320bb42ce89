"""Device-resident loop step (dflash_step_resident) against the oracle's loop
cycle (needs an MI355X).

Each step verifies the current drafts against target logits planted so that
a planned number of drafts is accepted, appends the anchor and the accepted
drafts from the block's target features at lengths held on the device,
advances those lengths and drafts the next block from the bonus token.  The
oracle runs the same cycle (verify_append_draft) on the same inputs.

The block the target scores in step s is the oracle's draft of step s - 1,
given to both sides (the drafts are an input of the verify): a near-tie
draft that the two sides break differently then cannot change later steps.

Bars: accept counts, bonus tokens (the next anchors) and device lengths
bit-exact; the step's draft ids as in gpu_util.draft_compare (bit-exact
where the oracle's top-2 logit gap clears a fixed gate derived from the
oracle's bf16 noise floor, a near-argmax elsewhere), with the GPU logits and final hidden
states of the same state taken from a debug dflash_draft_block run; cache
rows within 1e-4 (float32) or 2e-2 (bf16) max relative error per tensor.
"""
import numpy as np
import pytest

import oracle as O
from block_diffusion_drafter_concat_amd import configs, synth
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import (dev, draft_compare, rel_err, small_bf16_shape, synthetic_cache, tol,
                      upload_cache)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def torch():
    import torch
    L.load()
    return torch


def _shape(which):
    return configs.TINY_F32 if which == "tiny_f32" else small_bf16_shape()


def _setup(torch, shape, wid, lens, steps, B):
    w = configs.make_weights(shape, wid)
    dr = L.Drafter(shape, w)
    caches = synthetic_cache(shape, wid, lens)
    len_max = max(lens) + steps * B
    cache = L.KVCache(shape, [len_max + B for _ in lens])
    upload_cache(cache, caches)
    return w, dr, caches, cache, len_max


def _i32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _step_inputs(shape, wid, step, drafts, accept_plan, B):
    """Planted target logits (drafts accepted up to accept_plan) and the
    block's target features, as numpy arrays of the workload's dtype."""
    N = drafts.shape[0]
    lg = synth.plant_target_logits(
        synth.values((N, B, shape.vocab), shape.dtype, wid, synth.STREAM_LOGITS, f"rs_lg{step}"),
        drafts, accept_plan, shape.dtype, workload=wid)
    feats = [synth.values((N * B, shape.hidden), shape.dtype, wid, synth.STREAM_FEATURES,
                          f"rs_f{step}.{i}") for i in range(shape.n_feat)]
    return lg, feats


@pytest.mark.parametrize("which,lens,B", [("tiny_f32", [0, 37], 8),
                                          ("small_bf16", [45, 0, 300], 16),
                                          ("small_bf16", [3, 120, 0, 64, 9, 200, 31, 5, 77], 16)])
def test_resident_steps_match_oracle(torch, which, lens, B):
    """Four device-resident steps from ragged contexts (one empty).  The last
    case has 9 x 16 = 144 block rows: fusion and injection then run on the
    LDS-tiled GEMM and the draft's layer GEMMs on the batched path."""
    _resident_steps(torch, _shape(which), 61 + len(lens), lens, B, 4, which)


def test_resident_steps_full_size(torch):
    """The loop as measured: the Qwen3-8B-shaped bf16 drafter, one sequence at
    context 2048, B = 16, three resident steps (verify, append, draft) against
    the oracle's cycle."""
    _resident_steps(torch, configs.QWEN3_8B_LIKE, 2, [2048], 16, 3, "qwen3-8b-shaped")


def _resident_steps(torch, shape, wid, lens, B, steps, which):
    N = len(lens)
    w, dr, caches, cache, len_max = _setup(torch, shape, wid, lens, steps, B)
    anchors = configs.make_anchors(shape, wid, N)
    first = O.draft_block(w, shape, caches, anchors, B)
    drafts = first["draft_ids"]
    plan = synth.integers((steps, N), 0, B - 1, wid, synth.STREAM_INDICES, "rs_plan")

    ws = dr.workspace(N, B, 1)
    dev_len = _i32(torch, lens)
    d_draft = _i32(torch, drafts)
    d_anchor = _i32(torch, anchors)
    d_acc = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids2 = torch.empty((N, B - 1), dtype=torch.int32, device="cuda")
    hid = torch.empty((N * B, shape.hidden), dtype=torch.float32, device="cuda")
    z = torch.empty((N * B, shape.vocab), dtype=torch.float32, device="cuda")
    for s in range(steps):
        d_draft.copy_(_i32(torch, drafts))
        lg, feats = _step_inputs(shape, wid, s, drafts, plan[s], B)
        d_lg = dev(lg.reshape(N * B, -1), shape.dtype).reshape(N, B, -1)
        d_feats = [dev(f, shape.dtype) for f in feats]
        print(f"{which} N={N} B={B} step {s}: plan {plan[s].tolist()}", flush=True)
        dr.step_resident(cache, B, dev_len, len_max, d_lg, d_feats, d_draft, d_anchor, d_acc,
                         d_status, ws)
        torch.cuda.synchronize()
        st = O.verify_append_draft(w, shape, caches, lg, drafts, feats, B)
        np.testing.assert_array_equal(st["accept"], plan[s])
        np.testing.assert_array_equal(d_acc.cpu().numpy(), st["accept"])
        np.testing.assert_array_equal(d_anchor.cpu().numpy(), st["bonus"])
        want_len = [c[0][0].shape[0] for c in st["caches"]]
        np.testing.assert_array_equal(dev_len.cpu().numpy(), want_len)
        assert int(d_status.item()) == 0
        ids = d_draft.cpu().numpy()
        # GPU logits and hidden states of the same state: a debug draft with
        # the host lengths set to the device ones (it rewrites only the
        # block rows past them, which every step rewrites before reading)
        cache.seq_len[:] = want_len
        dr.draft_block(cache, B, d_anchor, ids2, ws, dbg_hidden=hid, dbg_logits=z)
        torch.cuda.synchronize()
        cache.seq_len[:] = lens
        draft_compare(shape, st, ids, hid.cpu().numpy(), z.cpu().numpy(), f"  step {s}")
        caches, drafts = st["caches"], st["draft_ids"]
    # committed cache rows, every layer and sequence
    worst = 0.0
    for b in range(N):
        n = caches[b][0][0].shape[0]
        o = int(cache.offs[b])
        for l, (k, v) in enumerate(caches[b]):
            if n == 0:
                continue
            kg = cache.k[l][:, o:o + n, :].permute(1, 0, 2).float().cpu().numpy()
            vg = cache.v[l][:, :, o:o + n].permute(2, 0, 1).float().cpu().numpy()
            worst = max(worst, rel_err(kg, k), rel_err(vg, v))
    print(f"  cache rel err {worst:.2e} over {steps} steps", flush=True)
    assert worst <= tol(shape)
    # the host lengths are the caller's: untouched
    np.testing.assert_array_equal(cache.seq_len, lens)


def test_resident_length_bound_saturates(torch):
    """A step whose lengths would pass len_max leaves them unchanged and sets
    the status word; sequences below the bound advance."""
    shape = small_bf16_shape()
    wid, B = 71, 16
    lens = [100, 20]
    w, dr, caches, cache, _ = _setup(torch, shape, wid, lens, 1, B)
    len_max = 102           # sequence 0 may grow by 2 rows at most
    N = len(lens)
    anchors = configs.make_anchors(shape, wid, N)
    drafts = O.draft_block(w, shape, caches, anchors, B)["draft_ids"]
    plan = np.array([4, 4])
    lg, feats = _step_inputs(shape, wid, 0, drafts, plan, B)
    ws = dr.workspace(N, B, 1)
    dev_len = _i32(torch, lens)
    d_acc = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dr.step_resident(cache, B, dev_len, len_max,
                     dev(lg.reshape(N * B, -1), "bf16").reshape(N, B, -1),
                     [dev(f, "bf16") for f in feats], _i32(torch, drafts), _i32(torch, anchors),
                     d_acc, d_status, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_acc.cpu().numpy(), plan)
    assert int(d_status.item()) == 1
    np.testing.assert_array_equal(dev_len.cpu().numpy(), [100, 25])


def test_resident_step_graph_replays_match_eager(torch):
    """One step captured in a HIP graph and replayed four times reproduces
    four eager steps bit for bit, lengths growing on the device throughout."""
    shape = small_bf16_shape()
    wid, B, steps = 73, 16, 4
    lens = [300, 45]
    N = len(lens)
    w, dr, caches, cache, len_max = _setup(torch, shape, wid, lens, steps + 1, B)
    anchors = configs.make_anchors(shape, wid, N)
    drafts = O.draft_block(w, shape, caches, anchors, B)["draft_ids"]
    lg, feats = _step_inputs(shape, wid, 0, drafts, np.array([5, 2]), B)
    d_lg = dev(lg.reshape(N * B, -1), "bf16").reshape(N, B, -1)
    d_feats = [dev(f, "bf16") for f in feats]
    ws = dr.workspace(N, B, 1)
    dev_len = _i32(torch, lens)
    d_draft = _i32(torch, drafts)
    d_anchor = _i32(torch, anchors)
    d_acc = torch.full((N,), -1, dtype=torch.int32, device="cuda")
    d_status = torch.zeros(1, dtype=torch.int32, device="cuda")
    state = [dev_len, d_draft, d_anchor] + cache.k + cache.v
    init = [t.clone() for t in state]

    def step():
        dr.step_resident(cache, B, dev_len, len_max, d_lg, d_feats, d_draft, d_anchor, d_acc,
                         d_status, ws)

    eager = []
    for _ in range(steps):
        step()
        torch.cuda.synchronize()
        eager.append([t.clone() for t in (d_acc, d_anchor, dev_len, d_draft)])
    assert int(d_status.item()) == 0
    lens_seen = [e[2].cpu().numpy().tolist() for e in eager]
    print(f"eager lengths {lens_seen}", flush=True)

    for t, v in zip(state, init):
        t.copy_(v)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    # capture ran nothing: the state is still the initial one
    assert dev_len.cpu().numpy().tolist() == lens
    for r in range(steps):
        d_acc.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("accept", "anchor", "len", "drafts"),
                                   (d_acc, d_anchor, dev_len, d_draft), eager[r]):
            assert torch.equal(got, want), (r, name, got, want)
    assert int(d_status.item()) == 0
