"""HIP path against the CPU oracle on the same seeded inputs (needs an MI355X).

Bars: floating-point outputs within max relative error 1e-4 (float32
workloads) or 2e-2 (bf16 workloads), per tensor; verify outputs bit-exact;
draft ids bit-exact wherever the oracle's top-2 logit gap is at least 1e-2
(float32) or max(1e-2, 2 x the drafter family's bf16 noise floor) (bf16; the
floor comes from the oracle alone, tests/golden/bf16_noise_floor.txt), and a
near-argmax of the oracle's logits elsewhere (see gpu_util.draft_compare).
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
from block_diffusion_drafter_concat_amd import configs, synth
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import (dev, draft_compare, feats_dev, rel_err, small_bf16_shape, synthetic_cache,
                      to_np, tol, upload_cache)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def torch():
    import torch
    L.load()
    return torch


def _i32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


# ------------------------------------------------------------------ verify

def _verify_case(torch, logits_np, drafts, dtype):
    N, B, V = logits_np.shape
    lg = dev(logits_np.reshape(N * B, V), dtype).reshape(N, B, V)
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    bon = torch.empty(N, dtype=torch.int32, device="cuda")
    ws = torch.empty(L.verify_workspace_size(N, B, V), dtype=torch.uint8, device="cuda")
    L.verify_greedy(lg, _i32(torch, drafts), acc, bon, ws)
    torch.cuda.synchronize()
    a_o, b_o = O.verify_greedy(logits_np, drafts)
    np.testing.assert_array_equal(acc.cpu().numpy(), a_o)
    np.testing.assert_array_equal(bon.cpu().numpy(), b_o)
    return a_o


def test_verify_tiny_f32_planted(torch):
    """64 seeded cases of the tiny workload: B = 8, V = 1024, k uniform on 0..8."""
    N, B, V = 64, 8, 1024
    k = synth.integers((N,), 0, 8, 1, synth.STREAM_LOGITS, "k")
    a = np.minimum(k, B - 1)
    drafts = synth.integers((N, B - 1), 0, V - 2, 1, synth.STREAM_LOGITS, "drafts")
    lg = synth.plant_target_logits(synth.values((N, B, V), "f32", 1, synth.STREAM_LOGITS, "lg"),
                                   drafts, a, "f32", workload=1)
    got = _verify_case(torch, lg, drafts, "f32")
    assert set(got.tolist()) == set(range(B))


def test_verify_batch16_bf16_full_vocab_with_ties(torch):
    """batch 16, B = 16, V = 151936 bf16; accept ~ Geometric(0.15) capped; planted exact ties."""
    N, B, V = 16, 16, 151936
    tau = synth.geometric_capped(N, 0.15, B, 3, synth.STREAM_LOGITS, "tau")
    drafts = synth.integers((N, B - 1), 0, V - 2, 3, synth.STREAM_LOGITS, "drafts")
    ties = synth.rng(3, synth.STREAM_LOGITS, "tie").random(N) < 0.125
    ties[0] = True
    lg = synth.plant_target_logits(synth.values((N, B, V), "bf16", 3, synth.STREAM_LOGITS, "lg"),
                                   drafts, tau - 1, "bf16", tie_rows=ties, workload=3)
    _verify_case(torch, lg, drafts, "bf16")


@pytest.mark.parametrize("V,B,dtype", [(1001, 2, "bf16"), (9, 3, "f32"), (8193, 16, "bf16")])
def test_verify_ragged_and_degenerate(torch, V, B, dtype):
    N = 5
    g = np.random.default_rng(V)
    drafts = g.integers(0, V, size=(N, B - 1))
    # coarse values: many exact ties inside every row
    lg = np.round(g.standard_normal((N, B, V)) * 2).astype(np.float32)
    for n in range(N):                 # make some prefixes match
        for j in range(min(n, B - 1)):
            drafts[n, j] = int(np.argmax(lg[n, j]))
    _verify_case(torch, lg, drafts, dtype)


def test_verify_many_rows_one_chunk_per_row(torch):
    """2560 target rows (batch 160, B = 16): the first stage then takes every
    row as a single chunk; V = 4096 (vector loads) with coarse values (ties)."""
    N, B, V = 160, 16, 4096
    g = np.random.default_rng(4096)
    lg = np.round(g.standard_normal((N, B, V)) * 2).astype(np.float32)
    drafts = g.integers(0, V, size=(N, B - 1))
    for n in range(N):                 # matching prefixes of every length 0..15
        for j in range(n % B):
            drafts[n, j] = int(np.argmax(lg[n, j]))
    got = _verify_case(torch, lg, drafts, "bf16")
    assert set(got.tolist()) == set(range(B))


# ------------------------------------------------------------------ fuse + inject

def _fuse(torch, dr, shape, feats_np):
    T = feats_np[0].shape[0]
    out = torch.empty((T, shape.hidden), dtype=L.torch_dtype(shape.dtype), device="cuda")
    ws = dr.workspace(1, 16, T)
    dr.fuse_context(feats_dev(feats_np, shape.dtype), out, ws)
    torch.cuda.synchronize()
    return to_np(out)


@pytest.mark.parametrize("which,T", [("tiny", 128), ("small", 37), ("small", 300)])
def test_fuse_context(torch, which, T):
    shape = configs.TINY_F32 if which == "tiny" else small_bf16_shape()
    wid = 11 if which == "tiny" else 12
    w = configs.make_weights(shape, wid)
    dr = L.Drafter(shape, w)
    feats = configs.make_features(shape, wid, T)
    got = _fuse(torch, dr, shape, feats)
    want = O.fuse_context(feats, w["fc"], w["fc_norm"], shape.rms_eps, shape.dtype == "bf16")
    e = rel_err(got, want)
    print(f"fuse {which} T={T}: rel {e:.2e}")
    assert e <= tol(shape)


def _inject_and_compare(torch, shape, w, dr, lens_list, wid, pos_start=None, prefill=None):
    """Inject per-sequence feature rows; compare every committed K/V row."""
    caps = [max(l, 1) + 64 for l in lens_list]
    cache = L.KVCache(shape, caps, fill=0)
    ws = dr.workspace(len(lens_list), 16, sum(lens_list))
    feats = [configs.make_features(shape, wid, n, name=f"inj{b}") for b, n in enumerate(lens_list)]
    cat = [np.concatenate([f[i] for f in feats]) for i in range(shape.n_feat)]
    T = cat[0].shape[0]
    ctx = torch.empty((T, shape.hidden), dtype=L.torch_dtype(shape.dtype), device="cuda")
    dr.fuse_context(feats_dev(cat, shape.dtype), ctx, ws)
    dr.inject_kv(ctx, lens_list, cache, ws)
    torch.cuda.synchronize()
    want = O.prefill(w, shape, feats)
    worst = 0.0
    for b in range(len(lens_list)):
        assert cache.seq_len[b] == lens_list[b]
        for l in range(shape.n_layers):
            if lens_list[b] == 0:
                continue
            worst = max(worst, rel_err(to_np(cache.keys(l, b)), want[b][l][0]),
                        rel_err(to_np(cache.values(l, b)), want[b][l][1]))
    return cache, want, worst, ws


@pytest.mark.parametrize("which", ["tiny", "small"])
def test_inject_kv(torch, which):
    shape = configs.TINY_F32 if which == "tiny" else small_bf16_shape()
    wid = 21 if which == "tiny" else 22
    w = configs.make_weights(shape, wid)
    dr = L.Drafter(shape, w)
    lens = [128] if which == "tiny" else [37, 0, 150]
    _, _, worst, _ = _inject_and_compare(torch, shape, w, dr, lens, wid)
    print(f"inject {which}: rel {worst:.2e}")
    assert worst <= tol(shape)


def test_inject_append_and_rewind(torch):
    """Appending in pieces equals one-shot; a rewind overwrites from pos_start."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 23)
    dr = L.Drafter(shape, w)
    T = 45
    feats = configs.make_features(shape, 23, T)
    want = O.prefill(w, shape, [feats])[0]
    cache = L.KVCache(shape, [T + 64], fill=0)
    ws = dr.workspace(1, 16, T)
    ctx = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device="cuda")
    dr.fuse_context(feats_dev(feats, "bf16"), ctx, ws)
    # garbage first, then rewind to 0 and inject in pieces of 1..16 rows
    dr.inject_kv(ctx[:20], [20], cache, ws)
    t, pieces = 0, [1, 16, 7, 3, 16, 2]
    for n in pieces:
        dr.inject_kv(ctx[t:t + n], [n], cache, ws, pos_start=[t])
        t += n
    torch.cuda.synchronize()
    assert cache.seq_len[0] == T
    for l in range(shape.n_layers):
        assert rel_err(to_np(cache.keys(l, 0)), want[l][0]) <= 2e-2
        assert rel_err(to_np(cache.values(l, 0)), want[l][1]) <= 2e-2


# ------------------------------------------------------------------ draft block

def _draft(torch, dr, shape, cache, B, anchors, ws):
    N = cache.batch
    ids = torch.full((N, B - 1), -1, dtype=torch.int32, device="cuda")
    hid = torch.empty((N * B, shape.hidden), dtype=torch.float32, device="cuda")
    z = torch.empty((N * B, shape.vocab), dtype=torch.float32, device="cuda")
    dr.draft_block(cache, B, _i32(torch, anchors), ids, ws, dbg_hidden=hid, dbg_logits=z)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), hid.cpu().numpy(), z.cpu().numpy()


def test_tiny_f32_end_to_end(torch):
    """The tiny workload: fuse 128 context rows, inject, draft B = 8, verify."""
    shape = configs.TINY_F32
    w = configs.make_weights(shape, 1)
    dr = L.Drafter(shape, w)
    cache, want_cache, worst, ws = _inject_and_compare(torch, shape, w, dr, [128], 1)
    assert worst <= 1e-4
    anchors = configs.make_anchors(shape, 1, 1)
    ws = dr.workspace(1, 8, 128)
    ids, hid, z = _draft(torch, dr, shape, cache, 8, anchors, ws)
    res = O.draft_block(w, shape, want_cache, anchors, 8)
    draft_compare(shape, res, ids, hid, z, "tiny-f32")


@pytest.mark.parametrize("B", [16, 5, 2])
def test_small_bf16_ragged_batch_end_to_end(torch, B):
    """bf16, 2 layers, 3 sequences with contexts 0, 45 and 300 rows."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 31)
    dr = L.Drafter(shape, w)
    lens = [0, 45, 300]
    cache, want_cache, worst, _ = _inject_and_compare(torch, shape, w, dr, lens, 31)
    assert worst <= 2e-2
    anchors = configs.make_anchors(shape, 31, len(lens))
    ws = dr.workspace(len(lens), B, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, B, anchors, ws)
    # the oracle drafts from its own cache (the GPU from the one it injected)
    oc = [[(k, v) for k, v in per] if per[0][0].shape[0] else
          [(np.zeros((0, shape.n_kv_heads, shape.head_dim)),) * 2 for _ in per]
          for per in want_cache]
    res = O.draft_block(w, shape, oc, anchors, B)
    draft_compare(shape, res, ids, hid, z, f"small-bf16 B={B}")


@pytest.mark.parametrize("nb,B", [(4, 16), (13, 5), (5, 16), (9, 16), (16, 16)])
def test_small_bf16_batch_of_blocks(torch, nb, B):
    """Batches of M = nb * B >= 64 block rows (64, 65, 80, 144, 256): the
    layer GEMMs and the LM head run on the LDS-tiled MFMA GEMM with row tiles
    of 64, 128 and 256, ragged M, split-K partials, and a vocabulary (5003)
    that ends inside a tile."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 51)
    dr = L.Drafter(shape, w)
    lens = [int(v) for v in synth.integers((nb,), 0, 400, 51, synth.STREAM_INDICES,
                                           f"mid_lens{nb}")]
    lens[0] = 0
    caches = synthetic_cache(shape, 51, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 51, nb)
    ws = dr.workspace(nb, B, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, B, anchors, ws)
    res = O.draft_block(w, shape, caches, anchors, B)
    draft_compare(shape, res, ids, hid, z, f"small-bf16 batch {nb} x B{B}")


def test_small_bf16_batch_lm_head_split(torch):
    """144 block rows against a 76900-token vocabulary: the LM head's 301
    column tiles of 256 overflow one round of the 256 compute units, so the
    vocabulary rows past the first 256 tiles run as a second launch, here on
    128 x 256 tiles (two row tiles, the second with 16 rows; a partial last
    column tile of 100 rows), with the argmax partials of both launches meeting
    in one finalize."""
    shape = dataclasses.replace(small_bf16_shape(), vocab=76900)
    w = configs.make_weights(shape, 52)
    dr = L.Drafter(shape, w)
    nb, B = 9, 16
    lens = [int(v) for v in synth.integers((nb,), 0, 300, 52, synth.STREAM_INDICES, "split_lens")]
    caches = synthetic_cache(shape, 52, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 52, nb)
    ws = dr.workspace(nb, B, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, B, anchors, ws)
    res = O.draft_block(w, shape, caches, anchors, B)
    draft_compare(shape, res, ids, hid, z, f"small-bf16 V=76900 batch {nb} x B{B}")


def test_small_bf16_ragged_batch_attention_order_near_capacity(torch):
    """48 sequences with contexts 54..2477 and B = 4 (M = 192 block rows): the
    longest-first attention order is planned with chunks as small as 256 keys,
    where the order table holds up to 254 of its 256 (sequence, chunk) entries."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 53)
    dr = L.Drafter(shape, w)
    nb, B = 48, 4
    lens = [int(v) for v in synth.integers((nb,), 0, 2500, 53, synth.STREAM_INDICES, "order_lens")]
    caches = synthetic_cache(shape, 53, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 53, nb)
    ws = dr.workspace(nb, B, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, B, anchors, ws)
    res = O.draft_block(w, shape, caches, anchors, B)
    draft_compare(shape, res, ids, hid, z, f"small-bf16 ragged {nb} x B{B}")


@pytest.mark.parametrize("which", ["small", "qwen"])
def test_autoregressive_stand_in_steps(torch, which):
    """The autoregressive stand-in used for the draft-latency comparison: a
    1-layer drafter run as 2-slot passes, each pass's draft anchoring the
    next, the anchor's K/V row (written by the pass at the first free row)
    kept by advancing the committed length.  The oracle gets the same
    anchors and a cache extended with the anchor's layer-0 K/V, formed from
    its own pieces (bf16 RMSNorm of the embedding row, projection, RoPE at the
    anchor's position).  "qwen": the width and context bench.py times it at
    (the Qwen3-8B-shaped layer, context 2048)."""
    if which == "small":
        shape, wid, n0 = configs.scaled(small_bf16_shape(), n_layers=1), 61, 40
    else:
        shape, wid, n0 = configs.scaled(configs.QWEN3_8B_LIKE, n_layers=1), 3, 2048
    w = configs.make_weights(shape, wid)
    dr = L.Drafter(shape, w)
    caches = synthetic_cache(shape, wid, [n0])
    cache = L.KVCache(shape, [n0 + 32])
    upload_cache(cache, caches)
    ws = dr.workspace(1, 2, 1)
    kc, vc = caches[0][0]
    kc, vc = np.asarray(kc, np.float64), np.asarray(vc, np.float64)
    lw = w["layers"][0]
    anchor = configs.make_anchors(shape, wid, 1)
    for step in range(3):
        ids, hid, z = _draft(torch, dr, shape, cache, 2, anchor, ws)
        res = O.draft_block(w, shape, [[(kc, vc)]], anchor, 2)
        draft_compare(shape, res, ids, hid, z, f"autoregressive step {step}")
        # keep the anchor's K/V: the GPU by advancing the committed length,
        # the oracle by appending the same row
        pos = n0 + step
        u = O.bf16_round(O.rmsnorm(np.asarray(w["embed"][int(anchor[0])], np.float64)[None],
                                   lw["attn_norm"], shape.rms_eps))
        k = (u @ np.asarray(lw["wk"], np.float64).T).reshape(1, shape.n_kv_heads, shape.head_dim)
        v = (u @ np.asarray(lw["wv"], np.float64).T).reshape(1, shape.n_kv_heads, shape.head_dim)
        kc = np.concatenate([kc, O.bf16_round(O.rope(k, [pos], shape.rope_theta))])
        vc = np.concatenate([vc, O.bf16_round(v)])
        cache.seq_len[0] += 1
        anchor = ids[:, 0].astype(np.int32)


def test_draft_is_deterministic(torch):
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 32)
    dr = L.Drafter(shape, w)
    lens = [700, 33]
    cache = L.KVCache(shape, [l + 32 for l in lens])
    upload_cache(cache, synthetic_cache(shape, 32, lens))
    anchors = configs.make_anchors(shape, 32, 2)
    ws = dr.workspace(2, 16, 1)
    a = _draft(torch, dr, shape, cache, 16, anchors, ws)
    b = _draft(torch, dr, shape, cache, 16, anchors, ws)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("nb", [3, 4])
def test_out_of_range_anchor_refused(torch, nb):
    """A block whose anchor is outside [0, V) gets draft ids -1; the other
    blocks' drafts are unchanged bit for bit (3 blocks: weight-streaming
    GEMMs, 48 rows; 4 blocks: the tiled path, 64 rows)."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 33)
    dr = L.Drafter(shape, w)
    lens = [50, 120, 7, 300][:nb]
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, synthetic_cache(shape, 33, lens))
    good = configs.make_anchors(shape, 33, nb)
    bad = good.copy()
    bad[0], bad[1] = -3, shape.vocab
    ws = dr.workspace(nb, 16, 1)
    ids_good = _draft(torch, dr, shape, cache, 16, good, ws)[0]
    ids_bad = _draft(torch, dr, shape, cache, 16, bad, ws)[0]
    assert (ids_good >= 0).all()
    assert (ids_bad[:2] == -1).all()
    np.testing.assert_array_equal(ids_bad[2:], ids_good[2:])


@pytest.fixture(scope="module")
def qwen_like(torch):
    shape = configs.QWEN3_8B_LIKE
    w = configs.make_weights(shape, 2)
    dr = L.Drafter(shape, w)
    return shape, w, dr


def test_headline_shape_draft_block_full_size(torch, qwen_like):
    """Qwen3-8B-shaped drafter, batch 1, ctx 2048, B = 16, at full size.

    The 2048-row context cache is drawn directly (N(0, 1.28^2), the spread an
    injected K/V has under these weights) so the oracle needs only the pass.
    """
    shape, w, dr = qwen_like
    lens = [2048]
    caches = synthetic_cache(shape, 2, lens)
    cache = L.KVCache(shape, [2048 + 64])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 2, 1)
    ws = dr.workspace(1, 16, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, 16, anchors, ws)
    res = O.draft_block(w, shape, caches, anchors, 16)
    draft_compare(shape, res, ids, hid, z, "qwen3-8b-shaped ctx2048")


def test_batch16_ragged_full_size_sampled(torch, qwen_like):
    """Qwen3-8B-shaped drafter, batch 16, contexts 512..8192 (the ragged
    batch workload), B = 16: M = 256 block rows on the tiled path.  Three
    sequences take their context from the shared generator and are checked
    against the oracle; the other thirteen get device draws (sequences never
    exchange anything, so they only have to exist)."""
    shape, w, dr = qwen_like
    wl = configs.qwen3_8b_b16_ragged()
    lens = list(wl.ctx)
    sample = [0, 7, 15]
    cache = L.KVCache(shape, [n + 64 for n in lens])
    g = torch.Generator(device="cuda")
    g.manual_seed(3003)
    for t in cache.k + cache.v:
        t.copy_(torch.randn(t.shape, generator=g, device="cuda") * 1.28)
    cache.seq_len[:] = np.asarray(lens, dtype=np.int32)
    sub = synthetic_cache(shape, wl.wid, [lens[b] for b in sample])
    upload_cache(cache, sub, seqs=sample)
    anchors = configs.make_anchors(shape, wl.wid, wl.batch)
    ws = dr.workspace(wl.batch, 16, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, 16, anchors, ws)
    rows = np.concatenate([np.arange(b * 16, b * 16 + 16) for b in sample])
    res = O.draft_block(w, shape, sub, anchors[sample], 16)
    draft_compare(shape, res, ids[sample], hid[rows], z[rows], "batch-16 ragged, sampled")


def test_headline_shape_float32_full_size(torch):
    """The headline drafter shape with float32 storage, full size, ctx 2048.

    Without bf16 storage points the two sides agree to ~1e-6, so every draft
    id whose oracle top-2 gap is >= 1e-2 must match bit-exactly over the full
    151936-token vocabulary.
    """
    shape = configs.scaled(configs.QWEN3_8B_LIKE, dtype="f32")
    w = configs.make_weights(shape, 6)
    dr = L.Drafter(shape, w)
    caches = synthetic_cache(shape, 6, [2048])
    cache = L.KVCache(shape, [2048 + 64])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 6, 1)
    ws = dr.workspace(1, 16, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, 16, anchors, ws)
    res = O.draft_block(w, shape, caches, anchors, 16)
    draft_compare(shape, res, ids, hid, z, "qwen3-8b-shaped float32 ctx2048")
    del dr, cache


def test_headline_shape_fuse_inject_sampled_rows(torch, qwen_like):
    """Full-size fusion of 2048 rows and injection; oracle on sampled rows."""
    shape, w, dr = qwen_like
    T = 2048
    feats = configs.make_features(shape, 2, T)
    cache = L.KVCache(shape, [T + 64])
    ws = dr.workspace(1, 16, T)
    ctx = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device="cuda")
    dr.fuse_context(feats_dev(feats, "bf16"), ctx, ws)
    dr.inject_kv(ctx, [T], cache, ws)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 1000, 2047])
    c_want = O.fuse_context([f[rows] for f in feats], w["fc"], w["fc_norm"], shape.rms_eps, True)
    c_got = to_np(ctx)[rows]
    assert rel_err(c_got, c_want) <= 2e-2
    kv_want = O.inject_kv(c_want, rows, w["layers"], shape, True)
    for l in range(shape.n_layers):
        k = to_np(cache.k[l][:, rows, :]).transpose(1, 0, 2)
        v = to_np(cache.v[l][:, :, rows]).transpose(2, 0, 1)
        assert rel_err(k, kv_want[l][0]) <= 2e-2
        assert rel_err(v, kv_want[l][1]) <= 2e-2
