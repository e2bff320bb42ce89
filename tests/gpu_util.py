"""Shared set-up of the GPU parity tests: seeded inputs go to both sides."""
from __future__ import annotations

import os

import numpy as np

from block_diffusion_drafter_concat_amd import configs, synth
from block_diffusion_drafter_concat_amd import lib as L


def rel_err(got, want) -> float:
    """Per-tensor max relative error: max|g - o| / max|o|."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    return float(np.max(np.abs(got - want)) / max(np.max(np.abs(want)), 1e-30))


def tol(shape) -> float:
    return 1e-4 if shape.dtype == "f32" else 2e-2


def dev(a, dtype):
    return L.to_device(a, dtype)


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def feats_dev(feats, dtype):
    return [dev(f, dtype) for f in feats]


def upload_cache(cache: "L.KVCache", caches_np, seqs=None):
    """Write per-sequence (K, V) [L_b, Hkv, d] into the device cache layout
    (entry i goes to sequence seqs[i], default i)."""
    import torch
    for i, per_layer in enumerate(caches_np):
        b = i if seqs is None else int(seqs[i])
        o = int(cache.offs[b])
        for l, (k, v) in enumerate(per_layer):
            n = k.shape[0]
            dt = cache.k[l].dtype
            kt = torch.from_numpy(np.ascontiguousarray(k, dtype=np.float32)).to(dt)
            vt = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dt)
            cache.k[l][:, o:o + n, :] = kt.permute(1, 0, 2).cuda()
            cache.v[l][:, :, o:o + n] = vt.permute(1, 2, 0).cuda()
        cache.seq_len[b] = per_layer[0][0].shape[0]


def synthetic_cache(shape, wid, lens, std=1.28):
    """Context K/V drawn directly (bf16/f32 values), per sequence and layer."""
    out = []
    for b, n in enumerate(lens):
        per = []
        for l in range(shape.n_layers):
            k = synth.values((n, shape.n_kv_heads, shape.head_dim), shape.dtype, wid,
                             synth.STREAM_FEATURES, f"cacheK{b}.{l}", std=std)
            v = synth.values((n, shape.n_kv_heads, shape.head_dim), shape.dtype, wid,
                             synth.STREAM_FEATURES, f"cacheV{b}.{l}", std=std)
            per.append((k, v))
        out.append(per)
    return out


_FLOOR_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "bf16_noise_floor.txt")


def bf16_noise_floor(shape) -> float:
    """Largest |logit difference| between two correct bf16 evaluations of the
    drafter family of ``shape``: the float64 oracle and the same steps in
    float32 arithmetic (tests/golden/bf16_noise_floor.py; read from the file
    it writes, never from the device)."""
    family = {512: "small-bf16", 384: "small-bf16-d64", 4096: "qwen3-8b-shaped",
              5120: "27b-target-shaped", 8192: "max-hidden-bf16"}[shape.hidden]
    with open(_FLOOR_FILE) as f:
        for ln in f:
            if ln.startswith(family + ":"):
                return float(ln.split(":")[1])
    raise KeyError(family)


def id_gate(shape) -> float:
    """Oracle top-2 gap from which a draft id must match bit for bit.

    float32 workloads: 1e-2.  bf16 workloads: the larger of 1e-2 and twice
    the family's noise floor -- a flip needs the errors of the two leading
    candidates to differ by more than their gap, and each error is within the
    floor.  The gate is a constant of the shape; it never reads the GPU output.
    """
    if shape.dtype == "f32":
        return 1e-2
    return max(1e-2, 2.0 * bf16_noise_floor(shape))


def draft_compare(shape, res, ids_gpu, hid_gpu, z_gpu, label=""):
    """Floats within tolerance; draft ids bit-exact wherever the logits decide them.

    A draft id is compared bit-exactly when the oracle's top-2 logit gap is at
    least ``id_gate(shape)``; an exempt id must still be a near-argmax of the
    oracle's logits (within the gate), and at most two thirds of the ids (or
    one) may be exempt, so every comparison checks at least a third of its ids
    exactly.  (Random-init drafters have flat logits -- most of all over long
    random contexts -- so a good share of ids can sit inside the noise.)
    """
    t = tol(shape)
    e_h = rel_err(hid_gpu, res["final_hidden"].reshape(hid_gpu.shape))
    e_z = rel_err(z_gpu, res["logits"].reshape(z_gpu.shape))
    zo = res["logits"]                                  # [N, B, V]
    dz = float(np.max(np.abs(np.asarray(z_gpu, dtype=np.float64).reshape(zo.shape) - zo)))
    gate = id_gate(shape)
    want = res["draft_ids"]
    assert ids_gpu.min() >= 0 and ids_gpu.max() < shape.vocab, ids_gpu
    ok = res["gap"] >= gate
    mism = (ids_gpu != want) & ok
    z1 = zo[:, 1:, :]
    picked = np.take_along_axis(z1, ids_gpu[..., None].astype(np.int64), axis=2)[..., 0]
    near = picked >= z1.max(axis=2) - gate
    ex = np.argwhere(~ok)
    ex_list = ", ".join(f"({int(n)},{int(j) + 1}) gap {res['gap'][n, j]:.4f}"
                        f"{'' if ids_gpu[n, j] == want[n, j] else ' differs'}" for n, j in ex)
    info = (f"{label} final_hidden rel {e_h:.2e}, logits rel {e_z:.2e} (max abs {dz:.3e}), "
            f"gate {gate:.3e}, exempt {len(ex)}/{ok.size}, mismatches {int(mism.sum())}"
            + (f"; exempt (seq, slot): {ex_list}" if len(ex) else ""))
    print(info, flush=True)
    assert e_h <= t, info
    assert e_z <= t, info
    assert not mism.any(), info
    assert near.all(), info
    assert len(ex) <= max(1, (2 * ok.size) // 3), info
    return e_h, e_z


def small_bf16_shape():
    """bf16 drafter with every dimension spanning several tiles and a ragged vocab."""
    return configs.DrafterShape(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                ffn=1536, vocab=5003, dtype="bf16")
