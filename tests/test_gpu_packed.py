"""Packed (fragment-major) weights on the LDS-tiled GEMMs (needs an MI355X).

Packing changes where the tiled GEMM loads each 16-row x 32-column operand
block from, not what lands in LDS nor the order of the MFMAs, so every output
must be bit-identical to the run on the row-major weights -- which the other
GPU tests hold to the oracle.  One small case is also compared with the oracle
directly, and the packed buffer's contents with a host-side repacking of the
weights.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
from block_diffusion_drafter_concat_amd import configs, synth
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import draft_compare, small_bf16_shape, synthetic_cache, upload_cache

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def torch():
    import torch
    L.load()
    return torch


def _i32(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _pack(torch, dr):
    buf = torch.empty(dr.packed_weights_size(), dtype=torch.uint8, device="cuda")
    dr.pack_weights(buf)
    torch.cuda.synchronize()
    return buf


def _draft(torch, dr, shape, cache, B, anchors, ws):
    N = cache.batch
    ids = torch.full((N, B - 1), -7, dtype=torch.int32, device="cuda")
    hid = torch.full((N * B, shape.hidden), float("nan"), dtype=torch.float32, device="cuda")
    z = torch.full((N * B, shape.vocab), float("nan"), dtype=torch.float32, device="cuda")
    dr.draft_block(cache, B, anchors, ids, ws, dbg_hidden=hid, dbg_logits=z)
    torch.cuda.synchronize()
    return ids, hid, z


def _same(torch, a, b, what):
    for x, y, n in zip(a, b, ("draft ids", "final hidden", "logits")):
        assert torch.equal(x, y), f"{what}: {n} differ between packed and row-major weights"


def _device_weights(torch, shape, seed):
    """Device-drawn bf16 weights (N(0, 0.02^2) matrices, gains near 1): the
    packed and row-major runs only have to agree with each other."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    H, F = shape.hidden, shape.ffn

    def mat(r, c):
        return (torch.randn((r, c), generator=g, device="cuda") * 0.02).to(torch.bfloat16)

    def gain():
        return (1 + torch.randn((H,), generator=g, device="cuda") * 0.02).to(torch.bfloat16)

    w = {"fc": mat(H, shape.n_feat * H), "fc_norm": gain(), "final_norm": gain(),
         "embed": mat(shape.vocab, H), "lm_head": mat(shape.vocab, H), "layers": []}
    for _ in range(shape.n_layers):
        w["layers"].append({"attn_norm": gain(), "wq": mat(shape.q_dim, H),
                            "wk": mat(shape.kv_dim, H), "wv": mat(shape.kv_dim, H),
                            "wo": mat(H, shape.q_dim), "ffn_norm": gain(), "wg": mat(F, H),
                            "wu": mat(F, H), "wd": mat(H, F)})
    return w


def _frag_major_host(a: np.ndarray) -> np.ndarray:
    """Row-major [N, K] -> fragment-major [ceil(N/16)*16 * K]: 16-row groups,
    each as K/32 consecutive blocks of 16 rows x 32 columns (zero rows past N)."""
    N, K = a.shape
    n16 = -(-N // 16) * 16
    p = np.zeros((n16, K), dtype=a.dtype)
    p[:N] = a
    return p.reshape(n16 // 16, 16, K // 32, 32).transpose(0, 2, 1, 3).reshape(-1)


def test_packed_buffer_layout(torch):
    """The packed copy of each matrix is the host repacking of the weights,
    bit for bit, with the LM head's last row group (V = 5003) padded with zeros."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 71)
    dr = L.Drafter(shape, w)
    buf = _pack(torch, dr)
    bits = buf.view(torch.int16).cpu().numpy()
    off = 0

    def check(name, a):
        nonlocal off
        want = _frag_major_host(dr_bits(a))
        got = bits[off // 2: off // 2 + want.size]
        np.testing.assert_array_equal(got, want, err_msg=name)
        off += -(-want.size * 2 // 256) * 256

    def dr_bits(a):
        t = a if hasattr(a, "data_ptr") else L.to_device(a, shape.dtype)
        return t.view(torch.int16).cpu().numpy()

    for l, lw in enumerate(dr.w["layers"]):
        for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
            check(f"layer {l} {n}", lw[n])
    check("fc", dr.w["fc"])
    check("lm_head", dr.w["lm_head"])
    assert off == buf.numel()


@pytest.mark.parametrize("nb,B", [(4, 16), (13, 5), (16, 16)])
def test_packed_batch_of_blocks_bit_identical(torch, nb, B):
    """M = 64, 65 (a ragged last row group) and 256 block rows, V = 5003:
    packed and row-major weights give the same draft ids, final hidden state
    and logits bit for bit; unbinding returns to the row-major weights."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 72)
    dr = L.Drafter(shape, w)
    lens = [int(v) for v in synth.integers((nb,), 0, 400, 72, synth.STREAM_INDICES,
                                           f"pk_lens{nb}")]
    caches = synthetic_cache(shape, 72, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = _i32(torch, configs.make_anchors(shape, 72, nb))
    ws = dr.workspace(nb, B, 1)
    base = _draft(torch, dr, shape, cache, B, anchors, ws)
    buf = _pack(torch, dr)
    packed = _draft(torch, dr, shape, cache, B, anchors, ws)
    _same(torch, base, packed, f"batch {nb} x B{B}")
    dr.pack_weights(None)
    again = _draft(torch, dr, shape, cache, B, anchors, ws)
    _same(torch, base, again, f"batch {nb} x B{B} after unbinding")
    del buf


def test_packed_against_the_oracle(torch):
    """A packed run held to the oracle directly (9 x B16 = 144 rows)."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 73)
    dr = L.Drafter(shape, w)
    nb, B = 9, 16
    lens = [int(v) for v in synth.integers((nb,), 0, 300, 73, synth.STREAM_INDICES, "pk_or")]
    caches = synthetic_cache(shape, 73, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 73, nb)
    ws = dr.workspace(nb, B, 1)
    buf = _pack(torch, dr)
    ids, hid, z = _draft(torch, dr, shape, cache, B, _i32(torch, anchors), ws)
    res = O.draft_block(w, shape, caches, anchors, B)
    draft_compare(shape, res, ids.cpu().numpy(), hid.cpu().numpy(), z.cpu().numpy(),
                  f"packed small-bf16 batch {nb} x B{B}")
    del buf


def test_packed_lm_head_split_bit_identical(torch):
    """V = 76900 (not a multiple of 16): both LM-head launches (256 x 256
    tiles, then the tail on 128 x 256 tiles) read the zero-padded last row
    group."""
    shape = dataclasses.replace(small_bf16_shape(), vocab=76900)
    w = configs.make_weights(shape, 74)
    dr = L.Drafter(shape, w)
    nb, B = 9, 16
    lens = [int(v) for v in synth.integers((nb,), 0, 300, 74, synth.STREAM_INDICES, "pk_split")]
    caches = synthetic_cache(shape, 74, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = _i32(torch, configs.make_anchors(shape, 74, nb))
    ws = dr.workspace(nb, B, 1)
    base = _draft(torch, dr, shape, cache, B, anchors, ws)
    buf = _pack(torch, dr)
    _same(torch, base, _draft(torch, dr, shape, cache, B, anchors, ws), "V=76900")
    del buf


def test_packed_training_layout_bit_identical(torch):
    """The training-layout forward (144 block rows, tiled QKV parts, SwiGLU and
    cross-entropy epilogues): losses and logits bit for bit."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 75)
    dr = L.Drafter(shape, w)
    lens, B = [300, 0, 77], 16
    caches = synthetic_cache(shape, 75, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens], fill=0)
    upload_cache(cache, caches)
    tokens, bseq, apos = configs.make_training_layout(shape, 75, lens, 4, B)
    n = len(bseq)
    anchor_ids = _i32(torch, [tokens[s][a] for s, a in zip(bseq, apos)])
    labels = _i32(torch, np.stack([tokens[s][a + 1:a + B] for s, a in zip(bseq, apos)]))
    ws = dr.workspace(n, B, 1)

    def run():
        slot = torch.full((n, B - 1), -1.0, dtype=torch.float32, device="cuda")
        loss = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
        z = torch.full((n * B, shape.vocab), float("nan"), dtype=torch.float32, device="cuda")
        dr.train_forward(cache, B, bseq, apos, anchor_ids, labels, 7.0, slot, loss, ws,
                         dbg_logits=z)
        torch.cuda.synchronize()
        return slot, loss, z

    base = run()
    buf = _pack(torch, dr)
    packed = run()
    for x, y, what in zip(base, packed, ("slot losses", "loss", "logits")):
        assert torch.equal(x, y), f"training layout: {what} differ"
    del buf


@pytest.mark.parametrize("T", [300, 2048])
def test_packed_fuse_inject_bit_identical(torch, T):
    """Fusion and injection over T context rows on the tiled GEMM (fc and the
    layers' wk / wv packed): the fused context and every cache row bit for bit."""
    shape = small_bf16_shape()
    w = configs.make_weights(shape, 76)
    dr = L.Drafter(shape, w)
    feats = [L.to_device(f, shape.dtype) for f in configs.make_features(shape, 76, T)]
    ws = dr.workspace(1, 16, T)

    def run():
        ctx = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device="cuda")
        dr.fuse_context(feats, ctx, ws)
        cache = L.KVCache(shape, [T + 32], fill=0)
        dr.inject_kv(ctx, [T], cache, ws)
        torch.cuda.synchronize()
        return ctx, cache

    ctx0, c0 = run()
    buf = _pack(torch, dr)
    ctx1, c1 = run()
    assert torch.equal(ctx0, ctx1), "fused context differs"
    for l in range(shape.n_layers):
        assert torch.equal(c0.k[l], c1.k[l]), f"layer {l} K differs"
        assert torch.equal(c0.v[l], c1.v[l]), f"layer {l} V differs"
    del buf


@pytest.mark.parametrize("which", ["qwen3-8b batch 16", "27b batch 8"])
def test_packed_full_size_bit_identical(torch, which):
    """The benchmarked batched workloads at full size (device-drawn weights):
    Qwen3-8B-shaped batch 16 with contexts 512..8192 (M = 256) and the
    27B-shaped drafter at batch 8, context 4096, B = 8 (M = 64)."""
    if which.startswith("qwen"):
        shape, wl, B = configs.QWEN3_8B_LIKE, configs.qwen3_8b_b16_ragged(), 16
    else:
        shape, wl, B = configs.TARGET_27B_LIKE, configs.target27b_b8(), 8
    print(which, flush=True)
    w = _device_weights(torch, shape, 77)
    dr = L.Drafter(shape, w)
    lens = list(wl.ctx)
    cache = L.KVCache(shape, [n + 64 for n in lens])
    g = torch.Generator(device="cuda")
    g.manual_seed(7007)
    for t in cache.k + cache.v:
        t.copy_(torch.randn(t.shape, generator=g, device="cuda") * 1.28)
    cache.seq_len[:] = np.asarray(lens, dtype=np.int32)
    anchors = _i32(torch, configs.make_anchors(shape, wl.wid, wl.batch))
    ws = dr.workspace(wl.batch, B, 1)
    base = _draft(torch, dr, shape, cache, B, anchors, ws)
    buf = _pack(torch, dr)
    _same(torch, base, _draft(torch, dr, shape, cache, B, anchors, ws), which)
    dr.pack_weights(None)
    del buf, cache, w
    dr.close()
