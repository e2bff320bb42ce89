"""Drafter shapes and the synthetic workloads used by tests and the benchmark.

A drafter (``DrafterShape``) is a stack of pre-norm decoder layers with
grouped-query attention and a SwiGLU feed-forward block, fed by a fusion FC
over the hidden states of ``n_feat`` target layers and read out through the
target's own embedding and LM head.  Weight layout is ``[out, in]`` row-major.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import synth


@dataclass(frozen=True)
class DrafterShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_feat: int = 5
    rms_eps: float = 1e-6
    rope_theta: float = 1e6
    dtype: str = "bf16"          # storage type of weights, features, caches

    @property
    def mask_token_id(self) -> int:
        return self.vocab - 1

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def layer_params(self) -> int:
        H = self.hidden
        return (2 * H + H * self.q_dim + 2 * H * self.kv_dim + self.q_dim * H
                + 3 * H * self.ffn)

    def fc_params(self) -> int:
        return self.hidden * self.n_feat * self.hidden + self.hidden

    def drafter_params(self) -> int:
        """Parameters the drafter owns (layers, fusion FC, final norm)."""
        return self.n_layers * self.layer_params() + self.fc_params() + self.hidden


@dataclass(frozen=True)
class Workload:
    wid: int                     # seeds every generator of this workload
    name: str
    shape: DrafterShape
    batch: int
    block: int                   # B: block slots including the anchor
    ctx: tuple = ()              # context length per sequence (prefill)
    extra: dict = field(default_factory=dict)


TINY_F32 = DrafterShape(n_layers=1, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64,
                        ffn=768, vocab=1024, dtype="f32")
QWEN3_8B_LIKE = DrafterShape(n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8,
                             head_dim=128, ffn=12288, vocab=151936, dtype="bf16")
TARGET_27B_LIKE = DrafterShape(n_layers=5, hidden=5120, n_q_heads=40, n_kv_heads=8,
                               head_dim=128, ffn=17408, vocab=151936, dtype="bf16")
# bf16 test shape with head dim 64, three q heads per kv head and six fused
# target layers (the largest count the interface takes)
SMALL_D64_BF16 = DrafterShape(n_layers=2, hidden=384, n_q_heads=6, n_kv_heads=2, head_dim=64,
                              ffn=1024, vocab=5003, n_feat=6, dtype="bf16")
# bf16 test shape at the largest hidden size the interface takes (8192), kept
# to one layer and two fused target layers so the oracle's weights stay small
MAX_HIDDEN_BF16 = DrafterShape(n_layers=1, hidden=8192, n_q_heads=32, n_kv_heads=8,
                               head_dim=128, ffn=4096, vocab=2048, n_feat=2, dtype="bf16")


def tiny_f32() -> Workload:
    return Workload(1, "tiny-f32 1-layer H256 ctx128 B8", TINY_F32, batch=1, block=8,
                    ctx=(128,))


def qwen3_8b_b1_ctx2048() -> Workload:
    return Workload(2, "qwen3-8b-shaped 5-layer bf16, batch 1, ctx 2048, B16",
                    QWEN3_8B_LIKE, batch=1, block=16, ctx=(2048,))


def qwen3_8b_b16_ragged() -> Workload:
    ctx = tuple(int(v) for v in synth.integers((16,), 512, 8192, 3, synth.STREAM_INDICES, "ctx"))
    return Workload(3, "qwen3-8b-shaped, batch 16, ragged ctx 512-8192, B16",
                    QWEN3_8B_LIKE, batch=16, block=16, ctx=ctx)


def qwen3_8b_long_incremental() -> Workload:
    return Workload(4, "qwen3-8b-shaped, batch 1, ctx 32768 + 256 incremental steps, B16",
                    QWEN3_8B_LIKE, batch=1, block=16, ctx=(32768,),
                    extra={"steps": 256, "capacity": 36864})


def target27b_b8(block: int = 16) -> Workload:
    return Workload(5, f"27b-target-shaped 5-layer bf16, batch 8, ctx 4096, B{block}",
                    TARGET_27B_LIKE, batch=8, block=block, ctx=(4096,) * 8)


def scaled(shape: DrafterShape, **kw) -> DrafterShape:
    d = dict(shape.__dict__)
    d.update(kw)
    return DrafterShape(**d)


# ---------------------------------------------------------------- weights

def make_weights(shape: DrafterShape, wid: int) -> dict:
    """Random-init weights: matrices N(0, 0.02^2), RMSNorm gains 1 + N(0, 0.02^2).

    Returns float32 arrays holding values exact in ``shape.dtype``.
    """
    dt = shape.dtype
    S = synth.STREAM_WEIGHTS
    H, F = shape.hidden, shape.ffn

    def mat(name, rows, cols):
        return synth.values((rows, cols), dt, wid, S, name, std=0.02)

    def gain(name):
        return synth.values((H,), dt, wid, S, name, std=0.02, mean=1.0)

    w = {
        "fc": mat("fc", H, shape.n_feat * H),
        "fc_norm": gain("fc_norm"),
        "final_norm": gain("final_norm"),
        "embed": mat("embed", shape.vocab, H),
        "lm_head": mat("lm_head", shape.vocab, H),
        "layers": [],
    }
    for l in range(shape.n_layers):
        p = f"layer{l}."
        w["layers"].append({
            "attn_norm": gain(p + "attn_norm"),
            "wq": mat(p + "wq", shape.q_dim, H),
            "wk": mat(p + "wk", shape.kv_dim, H),
            "wv": mat(p + "wv", shape.kv_dim, H),
            "wo": mat(p + "wo", H, shape.q_dim),
            "ffn_norm": gain(p + "ffn_norm"),
            "wg": mat(p + "wg", F, H),
            "wu": mat(p + "wu", F, H),
            "wd": mat(p + "wd", H, F),
        })
    return w


def make_features(shape: DrafterShape, wid: int, n_tokens: int, name: str = "feat") -> list:
    """``n_feat`` target hidden-state slabs [n_tokens, H] drawn N(0, 1)."""
    return [synth.values((n_tokens, shape.hidden), shape.dtype, wid, synth.STREAM_FEATURES,
                         f"{name}{i}") for i in range(shape.n_feat)]


def make_anchors(shape: DrafterShape, wid: int, batch: int, name: str = "anchor") -> np.ndarray:
    """Anchor token ids uniform on [0, V-2] (V-1 is the mask token)."""
    return synth.integers((batch,), 0, shape.vocab - 2, wid, synth.STREAM_INDICES, name)


def make_training_layout(shape: DrafterShape, wid: int, lens, blocks_per_seq: int,
                         block_size: int) -> tuple:
    """Seeded training layout over sequences with context lengths ``lens``.

    Returns (tokens, block_seq, anchor_pos): tokens[s] holds lens[s] + block_size
    ids uniform on [0, V-2] (so every anchor in 0..lens[s] has its labels);
    block i belongs to sequence block_seq[i] and starts at anchor_pos[i], drawn
    uniformly from 0..lens[s] without repeats while there are enough positions.
    """
    tokens, block_seq, anchor_pos = [], [], []
    for s, L in enumerate(lens):
        tokens.append(synth.integers((int(L) + block_size,), 0, shape.vocab - 2, wid,
                                     synth.STREAM_INDICES, f"train_tokens{s}"))
        g = synth.rng(wid, synth.STREAM_INDICES, f"train_anchors{s}")
        n = min(blocks_per_seq, int(L) + 1)
        anchor_pos += [int(a) for a in np.sort(g.choice(int(L) + 1, size=n, replace=False))]
        block_seq += [s] * n
    return tokens, np.asarray(block_seq, dtype=np.int32), np.asarray(anchor_pos, dtype=np.int32)
