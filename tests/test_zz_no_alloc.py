"""dflash_draft_block_noalloc against dflash_draft_block (needs an MI355X).

The no-allocation draft runs the same kernels on the library's static
per-device scratch instead of a caller workspace; its draft ids, final hidden
states and logits must equal those of dflash_draft_block bit for bit, on two
calls in a row (the second smaller: fewer sequences, fewer slots), at the
small bf16 shape (tiled path, M = 64) and at the headline shape (batch 1,
context 2048, B = 16).  A call that needs more scratch than the array holds is
refused before anything is enqueued.
"""
import numpy as np
import pytest

from block_diffusion_drafter_concat_amd import configs
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import small_bf16_shape, synthetic_cache, upload_cache

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _both(torch, dr, shape, lens, B, wid):
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, synthetic_cache(shape, wid, lens))
    anchors = torch.from_numpy(configs.make_anchors(shape, wid, len(lens))).cuda()
    N = len(lens)
    ws = dr.workspace(N, B, 1)
    assert ws.numel() <= L.NOALLOC_SCRATCH_BYTES
    out = []
    for noalloc in (False, True):
        ids = torch.full((N, B - 1), -7, dtype=torch.int32, device="cuda")
        hid = torch.empty((N * B, shape.hidden), dtype=torch.float32, device="cuda")
        z = torch.empty((N * B, shape.vocab), dtype=torch.float32, device="cuda")
        print(f"{'noalloc' if noalloc else 'workspace'} draft: lens {lens} B {B}", flush=True)
        if noalloc:
            dr.draft_block_noalloc(cache, B, anchors, ids, dbg_hidden=hid, dbg_logits=z)
        else:
            dr.draft_block(cache, B, anchors, ids, ws, dbg_hidden=hid, dbg_logits=z)
        torch.cuda.synchronize()
        out.append((ids.cpu().numpy(), hid.cpu().numpy(), z.cpu().numpy()))
    for a, b in zip(*out):
        np.testing.assert_array_equal(a, b)
    assert (out[1][0] >= 0).all()


def test_noalloc_draft_equals_workspace_draft():
    import torch
    L.load()
    shape = small_bf16_shape()
    dr = L.Drafter(shape, configs.make_weights(shape, 81))
    _both(torch, dr, shape, [300, 45, 0, 130], 16, 81)    # M = 64: the tiled path
    _both(torch, dr, shape, [40], 8, 82)                  # smaller: one sequence, 8 slots
    # more scratch than the array holds: refused before anything is enqueued
    lens = [1] * 64
    cache = L.KVCache(shape, [33] * 64)
    cache.seq_len[:] = np.asarray(lens, dtype=np.int32)
    assert dr.workspace_size(64, 16, 1) > L.NOALLOC_SCRATCH_BYTES
    ids = torch.full((64, 15), -7, dtype=torch.int32, device="cuda")
    anchors = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(L.DflashError) as e:
        dr.draft_block_noalloc(cache, 16, anchors, ids)
    assert e.value.status == L.ERR_SCRATCH
    torch.cuda.synchronize()
    assert (ids == -7).all()
    dr.close()


def test_noalloc_draft_headline_shape():
    import torch
    L.load()
    shape = configs.QWEN3_8B_LIKE
    dr = L.Drafter(shape, configs.make_weights(shape, 2))
    _both(torch, dr, shape, [2048], 16, 2)
    _both(torch, dr, shape, [700], 8, 3)
    dr.close()
