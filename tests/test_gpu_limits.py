"""The interface's limits on the GPU, against the oracle (needs an MI355X).

- DFLASH_MAX_BATCH: 64 sequences with ragged contexts drafted in one call
  (B = 4: 256 block rows on the LDS-tiled GEMMs; 128 (sequence, kv head)
  attention entries in the longest-first order), every sequence checked.
- The largest hidden size, 8192 (configs.MAX_HIDDEN_BF16, one layer): the
  norm kernels at eight float4 per thread and at most four split-K slabs,
  fusion of 37 and 200 rows (both GEMM paths), injection and a draft.
- A vocabulary smaller than one LM-head tile (17 tokens), on both LM-head paths.
Bars as in test_gpu_parity.
"""
import numpy as np
import pytest

import oracle as O
from block_diffusion_drafter_concat_amd import configs, synth
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import (draft_compare, feats_dev, rel_err, small_bf16_shape, synthetic_cache,
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


def _draft(torch, dr, shape, cache, B, anchors, ws):
    N = cache.batch
    ids = torch.full((N, B - 1), -7, dtype=torch.int32, device="cuda")
    hid = torch.empty((N * B, shape.hidden), dtype=torch.float32, device="cuda")
    z = torch.empty((N * B, shape.vocab), dtype=torch.float32, device="cuda")
    dr.draft_block(cache, B, _i32(torch, anchors), ids, ws, dbg_hidden=hid, dbg_logits=z)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), hid.cpu().numpy(), z.cpu().numpy()


def test_max_batch_draft(torch):
    """64 sequences (contexts 0..199), B = 4, small bf16 drafter."""
    shape = small_bf16_shape()
    nb, B = L.DFLASH_MAX_BATCH, 4
    assert nb == 64
    w = configs.make_weights(shape, 86)
    dr = L.Drafter(shape, w)
    lens = [int(v) for v in synth.integers((nb,), 0, 200, 86, synth.STREAM_INDICES, "maxb_lens")]
    caches = synthetic_cache(shape, 86, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 86, nb)
    ids, hid, z = _draft(torch, dr, shape, cache, B, anchors, dr.workspace(nb, B, 1))
    res = O.draft_block(w, shape, caches, anchors, B)
    draft_compare(shape, res, ids, hid, z, f"{nb} sequences x B{B}")


@pytest.fixture(scope="module")
def max_hidden(torch):
    shape = configs.MAX_HIDDEN_BF16
    w = configs.make_weights(shape, 85)
    dr = L.Drafter(shape, w)
    yield shape, w, dr
    dr.close()


@pytest.mark.parametrize("T", [37, 200])
def test_max_hidden_fuse_inject(torch, max_hidden, T):
    """Fusion over two 8192-wide slabs and injection of T rows at hidden 8192."""
    shape, w, dr = max_hidden
    feats = configs.make_features(shape, 85, T, name=f"mh{T}")
    ws = dr.workspace(1, 16, T)
    ctx = torch.empty((T, shape.hidden), dtype=torch.bfloat16, device="cuda")
    dr.fuse_context(feats_dev(feats, "bf16"), ctx, ws)
    cache = L.KVCache(shape, [T + 32], fill=0)
    dr.inject_kv(ctx, [T], cache, ws)
    torch.cuda.synchronize()
    want_c = O.fuse_context(feats, w["fc"], w["fc_norm"], shape.rms_eps, True)
    e_c = rel_err(to_np(ctx), want_c)
    want = O.prefill(w, shape, [feats])[0]
    e_k = rel_err(to_np(cache.keys(0, 0)), want[0][0])
    e_v = rel_err(to_np(cache.values(0, 0)), want[0][1])
    print(f"hidden 8192 T={T}: fuse rel {e_c:.2e}, K rel {e_k:.2e}, V rel {e_v:.2e}", flush=True)
    assert max(e_c, e_k, e_v) <= tol(shape)


def test_max_hidden_draft(torch, max_hidden):
    """A 16-slot draft over a 100-row context at hidden 8192."""
    shape, w, dr = max_hidden
    caches = synthetic_cache(shape, 85, [100])
    cache = L.KVCache(shape, [100 + 32])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 85, 1)
    ids, hid, z = _draft(torch, dr, shape, cache, 16, anchors, dr.workspace(1, 16, 1))
    res = O.draft_block(w, shape, caches, anchors, 16)
    draft_compare(shape, res, ids, hid, z, "hidden 8192, ctx 100")


@pytest.mark.parametrize("nb", [1, 5])
def test_vocab_smaller_than_a_tile(torch, nb):
    """A 17-token vocabulary, less than one LM-head tile: one sequence (16 rows,
    weight-streaming LM head, one partial 32-row tile) and five (80 rows, tiled
    LM head, one partial 256-column tile); the same seeded inputs as the small
    family's vocab-17 noise-floor case for nb = 5."""
    shape = configs.scaled(small_bf16_shape(), vocab=17)
    w = configs.make_weights(shape, 87)
    dr = L.Drafter(shape, w)
    lens = [int(v) for v in synth.integers((5,), 0, 300, 87, synth.STREAM_INDICES, "v17_lens")]
    lens = lens[:nb]
    caches = synthetic_cache(shape, 87, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, caches)
    anchors = configs.make_anchors(shape, 87, nb)
    ids, hid, z = _draft(torch, dr, shape, cache, 16, anchors, dr.workspace(nb, 16, 1))
    assert ((ids >= 0) & (ids < shape.vocab)).all()
    res = O.draft_block(w, shape, caches, anchors, 16)
    draft_compare(shape, res, ids, hid, z, f"vocab 17, {nb} sequences")
