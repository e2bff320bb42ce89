"""Seeded synthetic inputs for the drafter hot path.

This module is the only code shared by the CPU oracle side and the HIP side of
the tests and the benchmark.  It draws random numbers and shapes them into
inputs; it holds none of the method's arithmetic (no normalisation, no
projection, no attention, no argmax over model outputs).

Every tensor gets its own generator: ``SeedSequence([workload, stream,
crc32(name)])``, split into fixed 4 Mi-element chunks that are filled in
parallel threads.  The chunking is part of the definition, so the values do
not depend on the number of threads.

Values are drawn in float32.  For bf16 workloads they are rounded once to
bf16 (torch's round-to-nearest-even conversion) and returned as float32
arrays that hold exactly those bf16 values; ``bf16_bits`` gives the raw
16-bit patterns that the device receives.
"""
from __future__ import annotations

import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_CHUNK = 1 << 22

# Streams: which kind of input a generator feeds.
STREAM_WEIGHTS = 0
STREAM_FEATURES = 1
STREAM_INDICES = 2      # anchors, lengths, token counts
STREAM_LOGITS = 3       # synthetic target logits and their planting


def seed_sequence(workload: int, stream: int, name: str) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(workload), int(stream), zlib.crc32(name.encode())])


def rng(workload: int, stream: int, name: str) -> np.random.Generator:
    return np.random.default_rng(seed_sequence(workload, stream, name))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal(shape, workload: int, stream: int, name: str, std: float = 1.0,
           mean: float = 0.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws, chunk-parallel and reproducible."""
    shape = tuple(int(s) for s in shape)
    size = int(np.prod(shape)) if shape else 1
    out = np.empty(size, dtype=np.float32)
    n_chunks = max(1, (size + _CHUNK - 1) // _CHUNK)
    children = seed_sequence(workload, stream, name).spawn(n_chunks)

    def fill(i: int) -> None:
        lo = i * _CHUNK
        hi = min(size, lo + _CHUNK)
        if hi > lo:
            g = np.random.default_rng(children[i])
            g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if n_chunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(n_chunks)))
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out.reshape(shape)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (torch RNE) and return them as float32."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    if np.any(bits & np.uint32(0xFFFF)):
        raise ValueError("bf16_bits: values are not bf16-exact; round them first")
    return (bits >> np.uint32(16)).astype(np.uint16)


def values(shape, dtype: str, workload: int, stream: int, name: str,
           std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """N(mean, std^2) in the workload's storage type ("f32" or "bf16")."""
    x = normal(shape, workload, stream, name, std=std, mean=mean)
    if dtype == "bf16":
        x = to_bf16_values(x)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return x


def integers(shape, low: int, high: int, workload: int, stream: int, name: str) -> np.ndarray:
    """int32 uniform on [low, high] (inclusive)."""
    return rng(workload, stream, name).integers(low, high + 1, size=shape).astype(np.int32)


def geometric_capped(n: int, p: float, cap: int, workload: int, stream: int, name: str) -> np.ndarray:
    """int32 min(Geometric(p) on {1, 2, ...}, cap)."""
    g = rng(workload, stream, name).geometric(p, size=n)
    return np.minimum(g, cap).astype(np.int32)


def plant_target_logits(logits: np.ndarray, drafts: np.ndarray, accept: np.ndarray,
                        dtype: str, tie_rows: np.ndarray | None = None,
                        workload: int = 0, name: str = "plant") -> np.ndarray:
    """Make synthetic target logits whose greedy rows agree with given drafts.

    ``logits`` is [N, B, V] random, ``drafts`` [N, B-1] int, ``accept`` [N] with
    0 <= accept[n] <= B-1.  Row j < accept[n] gets its entry at drafts[n, j]
    raised to (row maximum + 1), so that row's largest entry is that draft.
    Row accept[n] (when < B-1) is made to disagree with drafts[n, accept[n]] by
    lowering that entry below the row's minimum.  ``tie_rows`` (bool [N])
    plants an exact tie for the largest entry in row accept[n] between two
    columns, so a consumer must break it by the lower column.  Values are
    rounded to the storage type afterwards (the raise and the lowering use
    offsets of 1.0, which bf16 keeps distinct near |x| < 8).
    """
    out = np.array(logits, dtype=np.float32, copy=True)
    n_seq, B, V = out.shape
    g = rng(workload, STREAM_LOGITS, name + ":ties")
    for n in range(n_seq):
        a = int(accept[n])
        for j in range(a):
            row = out[n, j]
            row[int(drafts[n, j])] = row.max() + 1.0
        if a < B - 1:
            row = out[n, a]
            d = int(drafts[n, a])
            row[d] = row.min() - 1.0
        if tie_rows is not None and tie_rows[n]:
            row = out[n, a]
            top = float(row.max()) + 1.0
            forbid = int(drafts[n, a]) if a < B - 1 else -1
            cols = [c for c in g.choice(V, size=4, replace=False) if c != forbid][:2]
            row[cols[0]] = top
            row[cols[1]] = top
    if dtype == "bf16":
        out = to_bf16_values(out)
    return out
