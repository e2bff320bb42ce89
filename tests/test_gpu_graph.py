"""The per-block launch sequence (draft_block, then verify_greedy) captured in
a HIP graph and replayed.

Each replay runs after eager work (torch fills of the outputs, another eager
draft into other buffers through the same workspace, synchronisations) and
must reproduce the eager call's outputs bit for bit: the kernels are
deterministic, take the sequence table by value and clear their own scratch
with kernels (no memset nodes).
"""
import numpy as np
import pytest

from block_diffusion_drafter_concat_amd import configs, synth
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import dev, small_bf16_shape, synthetic_cache, upload_cache

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def torch():
    import torch
    L.load()
    return torch


# small: two ragged sequences; headline: the Qwen3-8B-shaped drafter at one
# sequence of context 2048, the shape whose replayed draft bench.py times
@pytest.mark.parametrize("which", ["small", "headline"])
def test_draft_and_verify_graph_replays_match_eager(torch, which):
    if which == "small":
        shape, wid, lens = small_bf16_shape(), 41, [300, 45]
    else:
        shape, wid, lens = configs.QWEN3_8B_LIKE, 2, [2048]
    w = configs.make_weights(shape, wid)
    dr = L.Drafter(shape, w)
    N, B, V = len(lens), 16, shape.vocab
    cache = L.KVCache(shape, [n + 32 for n in lens])
    upload_cache(cache, synthetic_cache(shape, wid, lens))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    anchors = i32(configs.make_anchors(shape, wid, N))
    other = i32(configs.make_anchors(shape, wid + 1, N))
    ws = dr.workspace(N, B, 1)
    ids = torch.empty((N, B - 1), dtype=torch.int32, device="cuda")
    hid = torch.empty((N * B, shape.hidden), dtype=torch.float32, device="cuda")
    z = torch.empty((N * B, V), dtype=torch.float32, device="cuda")
    lg = synth.values((N, B, V), "bf16", wid, synth.STREAM_LOGITS, "graph_logits")
    logits = dev(lg.reshape(N * B, V), "bf16").reshape(N, B, V)
    acc = torch.empty(N, dtype=torch.int32, device="cuda")
    bon = torch.empty(N, dtype=torch.int32, device="cuda")
    vws = torch.empty(L.verify_workspace_size(N, B, V), dtype=torch.uint8, device="cuda")

    def seq():
        dr.draft_block(cache, B, anchors, ids, ws, dbg_hidden=hid, dbg_logits=z)
        L.verify_greedy(logits, ids, acc, bon, vws)

    seq()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (ids, hid, z, acc, bon)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        seq()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    torch.cuda.synchronize()

    ids2 = torch.empty_like(ids)
    for r in range(4):
        for t in (ids, acc, bon):
            t.fill_(-7)
        hid.zero_()
        z.zero_()
        dr.draft_block(cache, B, other, ids2, ws)      # eager work through the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("ids", "hidden", "logits", "accept", "bonus"),
                                   (ids, hid, z, acc, bon), ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager call"
    del g
