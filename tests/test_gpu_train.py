"""Training-layout forward on the GPU against the oracle.

Several blocks per sequence at sampled anchors share one read-only context
cache; block i sees the first a_i context rows and its own slots.  Compared:
the logits of every slot, the per-slot cross-entropy and the weighted loss.
The cross-entropy is 1-Lipschitz in each of log-sum-exp and the label logit,
so |loss error| <= 2 max|logit error| bounds the loss comparison.
"""
import dataclasses

import numpy as np
import pytest

import oracle as O
from block_diffusion_drafter_concat_amd import configs
from block_diffusion_drafter_concat_amd import lib as L

from conftest import gpu_available
from gpu_util import rel_err, small_bf16_shape, synthetic_cache, to_np, tol, upload_cache

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def torch():
    import torch
    L.load()
    return torch


def _run(torch, shape, wid, lens, B, gamma, per_seq=4, layout=None):
    w = configs.make_weights(shape, wid)
    dr = L.Drafter(shape, w)
    caches = synthetic_cache(shape, wid, lens)
    cache = L.KVCache(shape, [n + 32 for n in lens], fill=0)   # no NaN patterns in unused rows
    upload_cache(cache, caches)
    tokens, bseq, apos = configs.make_training_layout(shape, wid, lens, per_seq, B)
    if layout is not None:
        bseq, apos = (np.asarray(a, dtype=np.int32) for a in layout)
    n = len(bseq)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    anchor_ids = i32([tokens[s][a] for s, a in zip(bseq, apos)])
    labels = i32(np.stack([tokens[s][a + 1:a + B] for s, a in zip(bseq, apos)]))
    ws = dr.workspace(n, B, 1)
    slot = torch.full((n, B - 1), -1.0, dtype=torch.float32, device="cuda")
    loss = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    z = torch.empty((n * B, shape.vocab), dtype=torch.float32, device="cuda")
    k0 = cache.k[0].clone()
    v0 = cache.v[-1].clone()
    lens_before = cache.seq_len.copy()
    print(f"train_forward {shape.dtype} lens={lens} B={B} blocks={n} anchors={apos.tolist()}",
          flush=True)
    dr.train_forward(cache, B, bseq, apos, anchor_ids, labels, gamma, slot, loss, ws,
                     dbg_logits=z)
    torch.cuda.synchronize()
    # the context cache is only read
    assert (cache.seq_len == lens_before).all()
    assert torch.equal(cache.k[0], k0) and torch.equal(cache.v[-1], v0)
    want = O.train_forward(w, shape, caches, bseq, apos, tokens, B, gamma)
    return want, to_np(z).reshape(n, B, shape.vocab), to_np(slot), float(loss.item())


def _check(shape, want, z, slot, loss, label):
    e_z = rel_err(z, want["logits"])
    dz = float(np.max(np.abs(z.astype(np.float64) - want["logits"])))
    bound = 2.0 * dz + 1e-5 * max(1.0, float(np.max(np.abs(want["slot_loss"]))))
    d_slot = float(np.max(np.abs(slot - want["slot_loss"])))
    d_loss = abs(loss - want["loss"])
    info = (f"{label}: logits rel {e_z:.2e} (max abs {dz:.2e}), slot loss max abs {d_slot:.2e}, "
            f"loss {loss:.6f} vs {want['loss']:.6f} (bound {bound:.2e})")
    print(info, flush=True)
    assert e_z <= tol(shape), info
    assert d_slot <= bound, info
    assert d_loss <= bound, info


@pytest.mark.parametrize("which", ["tiny", "small", "small_few_rows"])
def test_train_forward_matches_oracle(torch, which):
    per_seq = 4
    if which == "tiny":
        shape, lens, B, gamma = configs.TINY_F32, [45, 0, 130], 8, 4.0
    elif which == "small":        # 144 block rows: the tiled layer GEMMs
        shape, lens, B, gamma = small_bf16_shape(), [300, 0, 77], 16, 7.0
    else:                         # 48 block rows: the weight-streaming layer GEMMs
        shape, lens, B, gamma, per_seq = small_bf16_shape(), [90], 16, 2.0, 3
    wid = {"tiny": 61, "small": 62, "small_few_rows": 65}[which]
    want, z, slot, loss = _run(torch, shape, wid, lens, B, gamma, per_seq=per_seq)
    _check(shape, want, z, slot, loss, which)


def test_train_forward_lm_head_split(torch):
    """144 block rows against a 76900-token vocabulary: the cross-entropy
    partials come from two LM-head launches (256 x 256 tiles, then the tail on
    128 x 256 tiles)."""
    shape = dataclasses.replace(small_bf16_shape(), vocab=76900)
    want, z, slot, loss = _run(torch, shape, 66, [300, 0, 77], 16, 5.0)
    _check(shape, want, z, slot, loss, "lm head split")


def test_train_forward_anchor_extremes_and_shared_context(torch):
    """Anchors at 0 (no context) and at the full length, twice at the same
    position, and blocks of two sequences interleaved."""
    shape = small_bf16_shape()
    lens = [200, 33]
    layout = ([0, 1, 0, 0, 1, 0], [0, 33, 200, 97, 0, 97])
    want, z, slot, loss = _run(torch, shape, 63, lens, 12, 3.0, layout=layout)
    _check(shape, want, z, slot, loss, "extremes")
    np.testing.assert_array_equal(z[3], z[5])   # same block twice: same numbers


def test_train_forward_long_context_many_chunks(torch):
    """Contexts spanning many attention chunks plus the blocks' own chunk."""
    shape = configs.scaled(small_bf16_shape(), n_layers=1)
    want, z, slot, loss = _run(torch, shape, 64, [2900, 1300], 16, 5.0, per_seq=6)
    _check(shape, want, z, slot, loss, "long")
