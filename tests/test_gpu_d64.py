"""HIP path against the oracle at head dim 64 in bf16 (needs an MI355X).

configs.SMALL_D64_BF16: 6 q heads and 2 kv heads of 64 (three q heads per kv
head, so 48 query rows per kv head in a 16-slot block), six fused target
layers.  These take code the other bf16 shapes do not: the bf16 attention
kernels at head dim 64 with three 16-query tiles, the RoPE pair tiles of a
64-wide head (two per head) in the QKV and injection epilogues, the fused
feature input as six slabs (weight-streaming and LDS-tiled fusion), and the
QKV finishing kernel at head dim 64.  Bars as in test_gpu_parity; the draft-id
gate of this family comes from tests/golden/bf16_noise_floor.txt.
"""
import numpy as np
import pytest

import oracle as O
from block_diffusion_drafter_concat_amd import configs, synth
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import draft_compare, feats_dev, rel_err, synthetic_cache, to_np, tol, upload_cache

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

SHAPE = configs.SMALL_D64_BF16


@pytest.fixture(scope="module")
def torch():
    import torch
    L.load()
    return torch


def _i32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("T", [37, 300])
def test_d64_fuse_context(torch, T):
    """Six feature slabs: T = 37 on the weight-streaming GEMM (slab pick per
    32-column step), T = 300 on the LDS-tiled GEMM (slab per stage)."""
    w = configs.make_weights(SHAPE, 83)
    dr = L.Drafter(SHAPE, w)
    feats = configs.make_features(SHAPE, 83, T)
    out = torch.empty((T, SHAPE.hidden), dtype=torch.bfloat16, device="cuda")
    dr.fuse_context(feats_dev(feats, "bf16"), out, dr.workspace(1, 16, T))
    torch.cuda.synchronize()
    want = O.fuse_context(feats, w["fc"], w["fc_norm"], SHAPE.rms_eps, True)
    e = rel_err(to_np(out), want)
    print(f"d64 fuse T={T}: rel {e:.2e}", flush=True)
    assert e <= tol(SHAPE)


@pytest.mark.parametrize("lens", [[20], [37, 0, 150]])
def test_d64_inject_kv(torch, lens):
    """K (RoPE on two 32-wide pair tiles per head) and V of every layer, on the
    weight-streaming path (20 rows) and the LDS-tiled one (187 rows)."""
    w = configs.make_weights(SHAPE, 84)
    dr = L.Drafter(SHAPE, w)
    caps = [max(n, 1) + 64 for n in lens]
    cache = L.KVCache(SHAPE, caps, fill=0)
    ws = dr.workspace(len(lens), 16, sum(lens))
    feats = [configs.make_features(SHAPE, 84, n, name=f"inj{b}") for b, n in enumerate(lens)]
    cat = [np.concatenate([f[i] for f in feats]) for i in range(SHAPE.n_feat)]
    ctx = torch.empty((sum(lens), SHAPE.hidden), dtype=torch.bfloat16, device="cuda")
    dr.fuse_context(feats_dev(cat, "bf16"), ctx, ws)
    dr.inject_kv(ctx, lens, cache, ws)
    torch.cuda.synchronize()
    want = O.prefill(w, SHAPE, feats)
    worst = 0.0
    for b, n in enumerate(lens):
        assert cache.seq_len[b] == n
        if n == 0:
            continue
        for l in range(SHAPE.n_layers):
            worst = max(worst, rel_err(to_np(cache.keys(l, b)), want[b][l][0]),
                        rel_err(to_np(cache.values(l, b)), want[b][l][1]))
    print(f"d64 inject {lens}: rel {worst:.2e}", flush=True)
    assert worst <= tol(SHAPE)


def _draft(torch, dr, cache, B, anchors, ws):
    N = cache.batch
    ids = torch.full((N, B - 1), -7, dtype=torch.int32, device="cuda")
    hid = torch.empty((N * B, SHAPE.hidden), dtype=torch.float32, device="cuda")
    z = torch.empty((N * B, SHAPE.vocab), dtype=torch.float32, device="cuda")
    dr.draft_block(cache, B, _i32(torch, anchors), ids, ws, dbg_hidden=hid, dbg_logits=z)
    torch.cuda.synchronize()
    return ids, hid, z


def _blocks_case(torch, wid, lens, B=16):
    w = configs.make_weights(SHAPE, wid)
    dr = L.Drafter(SHAPE, w)
    caches = synthetic_cache(SHAPE, wid, lens)
    cache = L.KVCache(SHAPE, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(SHAPE, wid, len(lens))
    return w, dr, caches, cache, anchors, dr.workspace(len(lens), B, 1)


def test_d64_draft_three_sequences(torch):
    """Contexts 0 / 45 / 300, B = 16: 48 block rows on the weight-streaming
    GEMMs, attention with three 16-query tiles per kv head."""
    w, dr, caches, cache, anchors, ws = _blocks_case(torch, 81, [0, 45, 300])
    ids, hid, z = _draft(torch, dr, cache, 16, anchors, ws)
    res = O.draft_block(w, SHAPE, caches, anchors, 16)
    draft_compare(SHAPE, res, ids.cpu().numpy(), hid.cpu().numpy(), z.cpu().numpy(),
                  "d64 contexts 0/45/300")


def test_d64_batch_of_blocks_and_packed(torch):
    """Five contexts below 400, B = 16: 80 block rows on the LDS-tiled GEMMs
    (QKV parts + the finishing kernel at head dim 64), against the oracle; then
    the same draft on packed weights, bit for bit."""
    lens = [int(v) for v in synth.integers((5,), 0, 400, 82, synth.STREAM_INDICES, "d64_lens")]
    w, dr, caches, cache, anchors, ws = _blocks_case(torch, 82, lens)
    ids, hid, z = _draft(torch, dr, cache, 16, anchors, ws)
    res = O.draft_block(w, SHAPE, caches, anchors, 16)
    draft_compare(SHAPE, res, ids.cpu().numpy(), hid.cpu().numpy(), z.cpu().numpy(),
                  f"d64 batch of 5 blocks {lens}")
    buf = torch.empty(dr.packed_weights_size(), dtype=torch.uint8, device="cuda")
    dr.pack_weights(buf)
    ids2, hid2, z2 = _draft(torch, dr, cache, 16, anchors, ws)
    assert torch.equal(ids, ids2) and torch.equal(hid, hid2) and torch.equal(z, z2)
