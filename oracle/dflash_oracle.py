"""CPU oracle of the DFlash drafter hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product (the HIP library and its
Python binding) never imports, calls or links it, and this module imports
nothing from the product.

What it computes: the drafter's work for one speculative cycle, written out
step by step in float64 numpy, in the order the pages describe it.  Where the
device stores a tensor in bf16 or feeds it to a bf16 matrix instruction, the
oracle rounds the same tensor to bf16 (round to nearest, ties to even) with
``bf16_round`` -- see the list in ``ROUNDING_POINTS``.  Everything else stays
float64.  For float32 workloads nothing is rounded.

Sources (web pages on DFlash, cited by page and section):
  [Arch]    zhichai.net, "DFlash 的架构密码——扩散模型如何「寄生」在自回归模型上"
            sections: 第一层 Feature Fusion, 第二层 KV Injection, 第三层 Block
            Diffusion, 训练策略 1-3, 技术细节补充 (提取层数, 投影层, 稀疏注意力训练).
  [Summary] ai-stack.site, "DFlash：基于块扩散的闪存推测解码方法", 实践 2
            (block verification; keep up to the last correct token) and FAQ 4
            (output is lossless).
  [News]    zaocj.com news article on DFlash (ICML 2026): one forward pass with
            bidirectional attention fills 8-16 token slots; 5-6 target layers.

Readings of points the pages leave open (each repeated where it is used):
  R1 layer ids are 1-based; "from layer 2 to the third-from-last" is
     [2, L-2]; uniform positions are rounded half up.
  R2 the fusion FC has no bias; RMSNorm eps = 1e-6; concat order = ascending id.
  R3 RoPE (rotate-half pairing i <-> i+d/2, theta = 1e6) on q and k; context
     token t sits at position t, block slot j at L + j.
  R4 block slot 0 holds the anchor (the previous cycle's bonus token), slots
     1..B-1 hold the mask token; draft j is the argmax of slot j's logits.
  R5 no mask inside a block; a block sees its own sequence's context and block.
  R6 every argmax breaks ties by the lowest index.
  R7 verification: a = length of the longest prefix with target_argmax[j] ==
     draft[j+1]; bonus = target_argmax[a].
  R8 training layout: block i of sequence s starts at anchor position a_i
     (0 <= a_i <= L_s): slot 0 holds the token at a_i, slots 1..B-1 the mask
     token, slot j sits at position a_i + j; the block sees context rows
     [0, a_i) of s and its own block, nothing else; slot j >= 1 is scored
     against the token at a_i + j.
  R9 loss weights: the k-th predicted slot (k = j = 1..B-1) weighs
     exp(-(k-1)/gamma); the loss is the weighted mean over every scored slot
     of every block, sum(w * ce) / sum(w).
  R10 stochastic drafting and verification (the pages: candidates are
     accepted or rejected by the target's distribution and a rejection is
     resampled, so the output distribution is the target's; the rule itself is
     the textbook one the pages point to): drafter and target distributions
     are softmax(logits / T) at one temperature T > 0; draft j (slot j >= 1)
     is drawn by the Gumbel-max rule from caller uniforms; draft k (slot k+1)
     is accepted while r_k * p_{k+1}(x) < q_k(x); at the first rejection a the
     next token is drawn from (q_a - p_{a+1})_+ by inverse CDF with a caller
     uniform u (smallest index whose cumulative weight exceeds u * total);
     after B-1 acceptances it is drawn from q_{B-1} the same way.
  R11 one loop cycle after the target scored a block (the pages: the block
     starts at the verified bonus token; the committed tokens' target
     features become context): the target's hidden states at the block's B
     positions are given; slots 0..a (the anchor and the a accepted drafts)
     are appended at positions L..L+a, L becomes L+a+1, and the next block is
     drafted from the bonus token at position L+a+1.
"""
from __future__ import annotations

import numpy as np

# Tensors the device holds in bf16 (or feeds to bf16 MFMA) on bf16 workloads.
ROUNDING_POINTS = (
    "c: fused context feature",
    "K, V cache entries after RoPE",
    "u: every RMSNorm output that feeds a projection",
    "q, k, v of the block after RoPE",
    "o: attention output feeding the O projection",
    "h: silu(gate) * up feeding the down projection",
)

_BF16_MAX = float.fromhex("0x1.fep127")


# --------------------------------------------------------------- numerics

def bf16_round(x) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits and float32's exponent range; below 2**-126
    its spacing is fixed at 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def _maybe_round(x, rb: bool):
    return bf16_round(x) if rb else x


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rmsnorm(x, gain, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * gain over the last axis ([Arch] 投影层: FC + RMSNorm)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * _f64(gain)


def rope(x, positions, theta: float) -> np.ndarray:
    """Rotary embedding, reading R3.  x: [T, heads, d]; positions: [T].

    Pair (i, i + d/2) is rotated by angle p * theta^(-2i/d).
    """
    x = _f64(x)
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-(2.0 * np.arange(half, dtype=np.float64)) / d)
    ang = _f64(positions)[:, None, None] * inv_freq[None, None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def silu(x) -> np.ndarray:
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def argmax_lowest(z, axis: int = -1) -> np.ndarray:
    """Index of the largest entry; ties go to the lowest index (reading R6)."""
    return np.argmax(z, axis=axis)


# ------------------------------------------------------- (a1) layer rule

def target_layer_ids(n_target_layers: int, n_select: int = 5) -> list:
    """1-based ids of the target layers whose hidden states feed the drafter.

    [Arch] 技术细节补充 / 提取层数: n_select layers sampled uniformly from the
    2nd layer to the third-from-last layer ([News]: 5 to 6 layers).
    Reading R1: the k-th id is 2 + k (L - 4) / (n - 1), rounded half up.
    """
    L, n = int(n_target_layers), int(n_select)
    first, last = 2, L - 2
    if n < 2 or last - first + 1 < n:
        raise ValueError("need n_target_layers >= n_select + 3 and n_select >= 2")
    ids = []
    for k in range(n):
        num = first * (n - 1) + k * (last - first)   # position times (n - 1)
        ids.append((2 * num + (n - 1)) // (2 * (n - 1)))
    return ids


# ------------------------------------------- (a2, a3) feature fusion

def fuse_context(feats, w_fc, g_fc, eps: float, round_bf16: bool) -> np.ndarray:
    """Compact context feature c [T, H] from n target hidden-state slabs.

    [Arch] 第一层 Feature Fusion: the sampled layers' hidden states are
    concatenated and passed through a light projection; 技术细节补充 / 投影层:
    the projection is an FC followed by RMSNorm.  Reading R2.
    """
    X = np.concatenate([_f64(f) for f in feats], axis=1)     # [T, n*H]
    Y = X @ _f64(w_fc).T                                       # [T, H]
    c = rmsnorm(Y, g_fc, eps)
    return _maybe_round(c, round_bf16)


# ------------------------------------------------- (a4) KV injection

def inject_kv(c, positions, layers, shape, round_bf16: bool) -> list:
    """Per drafter layer, the context K and V that the feature c contributes.

    [Arch] 第二层 KV Injection: the context feature is not fed in as an
    embedding; it goes straight into every layer's K and V projection, so the
    drafter's cache holds the target's context at every layer.  Reading: each
    layer's own W_k / W_v (the ones its block tokens use), RoPE on K at the
    context positions (R3).  Returns [(K [T, Hkv, d], V [T, Hkv, d]), ...].
    """
    c = _f64(c)
    T = c.shape[0]
    Hkv, d = shape.n_kv_heads, shape.head_dim
    out = []
    for lw in layers:
        k = (c @ _f64(lw["wk"]).T).reshape(T, Hkv, d)
        v = (c @ _f64(lw["wv"]).T).reshape(T, Hkv, d)
        k = rope(k, positions, shape.rope_theta)
        out.append((_maybe_round(k, round_bf16), _maybe_round(v, round_bf16)))
    return out


# ------------------------------------------------- (a6') block attention

def block_attention(q, K, V) -> np.ndarray:
    """Softmax attention of one block's queries over the keys it may see.

    q: [B, Hq, d]; K, V: [Lk, Hkv, d] = this sequence's context keys followed
    by its own block's keys.  Every query sees every one of these keys (no mask
    inside the block) and nothing else ([Arch] 技术细节补充 / 稀疏注意力训练:
    bidirectional inside a block, no information flow between blocks; [News]:
    bidirectional attention).  q-head h reads kv-head h // (Hq / Hkv).
    """
    q, K, V = _f64(q), _f64(K), _f64(V)
    B, Hq, d = q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.empty((B, Hq, d), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = q[:, h, :] @ K[:, g, :].T / np.sqrt(d)            # [B, Lk]
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[:, g, :]
    return out


# ------------------------------------------------- (a6) decoder layer

def decoder_layer(x, positions, lw, k_ctx, v_ctx, shape, rb: bool) -> np.ndarray:
    """One pre-norm drafter layer applied to the blocks of one or more sequences.

    x: [B, H] (one sequence; k_ctx, v_ctx: [L, Hkv, d]) or [N, B, H] (N
    sequences; k_ctx, v_ctx: lists of N such arrays); float64 residual stream.
    Attention half then SwiGLU feed-forward half, each with its own RMSNorm and
    a residual add.  The projections act on each row independently, so rows of
    all sequences are stacked for them; attention runs per sequence.
    """
    single = np.ndim(x) == 2
    if single:
        x, positions, k_ctx, v_ctx = x[None], np.asarray(positions)[None], [k_ctx], [v_ctx]
    x = _f64(x)
    N, B, H = x.shape
    Hq, Hkv, d = shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    eps = shape.rms_eps
    pos = np.asarray(positions).reshape(N * B)
    rows = x.reshape(N * B, H)
    u = _maybe_round(rmsnorm(rows, lw["attn_norm"], eps), rb)
    q = (u @ _f64(lw["wq"]).T).reshape(N * B, Hq, d)
    k = (u @ _f64(lw["wk"]).T).reshape(N * B, Hkv, d)
    v = (u @ _f64(lw["wv"]).T).reshape(N * B, Hkv, d)
    q = _maybe_round(rope(q, pos, shape.rope_theta), rb).reshape(N, B, Hq, d)
    k = _maybe_round(rope(k, pos, shape.rope_theta), rb).reshape(N, B, Hkv, d)
    v = _maybe_round(v, rb).reshape(N, B, Hkv, d)
    o = np.stack([block_attention(q[n], np.concatenate([_f64(k_ctx[n]), k[n]], axis=0),
                                  np.concatenate([_f64(v_ctx[n]), v[n]], axis=0))
                  for n in range(N)])
    o = _maybe_round(o.reshape(N * B, Hq * d), rb)
    rows = rows + o @ _f64(lw["wo"]).T
    u = _maybe_round(rmsnorm(rows, lw["ffn_norm"], eps), rb)
    h = _maybe_round(silu(u @ _f64(lw["wg"]).T) * (u @ _f64(lw["wu"]).T), rb)
    rows = rows + h @ _f64(lw["wd"]).T
    out = rows.reshape(N, B, H)
    return out[0] if single else out


# --------------------------------------- (a5, a6, a7) one block, one pass

def draft_block(weights, shape, caches, anchors, block_size: int) -> dict:
    """Fill one block of mask slots per sequence in a single forward pass.

    [Arch] 第三层 Block Diffusion: with the target's features as condition the
    block (e.g. 16 tokens) is produced in one step, one forward pass; 训练策略
    1: each block starts at an already verified token (the previous cycle's
    bonus token); 训练策略 3: the drafter reuses the target's embedding and LM
    head.  Readings R3-R6.

    caches[b] = [(K_ctx [L_b, Hkv, d], V_ctx [L_b, Hkv, d]) per layer].
    Returns draft_ids [N, B-1], final_hidden [N, B, H] (residual after the
    last layer), logits [N, B, V], gap [N, B-1] (top-1 minus top-2 logit of
    each draft slot).
    """
    rb = shape.dtype == "bf16"
    N, B = len(anchors), int(block_size)
    emb, lm = weights["embed"], weights["lm_head"]
    tokens = np.array([[int(a)] + [shape.mask_token_id] * (B - 1) for a in anchors])
    lens = np.array([caches[b][0][0].shape[0] for b in range(N)])
    positions = lens[:, None] + np.arange(B)[None, :]
    x = _f64(emb[tokens.reshape(-1)]).reshape(N, B, shape.hidden)
    for l, lw in enumerate(weights["layers"]):
        x = decoder_layer(x, positions, lw, [caches[b][l][0] for b in range(N)],
                          [caches[b][l][1] for b in range(N)], shape, rb)
    final_h = x
    u = _maybe_round(rmsnorm(x.reshape(N * B, shape.hidden), weights["final_norm"],
                             shape.rms_eps), rb)
    logits = (u @ _f64(lm).T).reshape(N, B, shape.vocab)
    z = logits[:, 1:, :]
    draft_ids = argmax_lowest(z, axis=2).astype(np.int32)
    srt = np.sort(z, axis=2)
    gap = srt[:, :, -1] - srt[:, :, -2]
    return {"draft_ids": draft_ids, "final_hidden": final_h, "logits": logits, "gap": gap}


# ------------------------------------------------- (a8) greedy verify

def verify_greedy(target_logits, drafts) -> tuple:
    """Accepted draft count and bonus token per sequence.

    The target scores the whole block in one pass; row j is its greedy choice
    for the token after slot j.  Drafts are kept up to the last one that
    matches ([Summary] 实践 2: keep up to the last correct token), and the
    target's own choice at the first mismatch (or after the last draft) is the
    bonus token that starts the next block ([Arch] 训练策略 1).  Reading R7.
    target_logits: [N, B, V]; drafts: [N, B-1].  Returns (accept [N], bonus [N]).
    """
    t = argmax_lowest(_f64(target_logits), axis=2)
    drafts = np.asarray(drafts)
    N, Bm1 = drafts.shape
    accept = np.zeros(N, dtype=np.int32)
    bonus = np.zeros(N, dtype=np.int32)
    for n in range(N):
        a = 0
        while a < Bm1 and t[n, a] == drafts[n, a]:
            a += 1
        accept[n] = a
        bonus[n] = t[n, a]
    return accept, bonus


# ------------------------------------------------- whole-cycle helpers

def prefill(weights, shape, feats_per_seq) -> list:
    """Context caches for each sequence: fuse its features, inject them at 0..L-1."""
    rb = shape.dtype == "bf16"
    caches = []
    for feats in feats_per_seq:
        c = fuse_context(feats, weights["fc"], weights["fc_norm"], shape.rms_eps, rb)
        caches.append(inject_kv(c, np.arange(c.shape[0]), weights["layers"], shape, rb))
    return caches


def append_context(cache, weights, shape, feats) -> list:
    """Append the features of newly committed tokens to one sequence's cache."""
    rb = shape.dtype == "bf16"
    L = cache[0][0].shape[0]
    c = fuse_context(feats, weights["fc"], weights["fc_norm"], shape.rms_eps, rb)
    new = inject_kv(c, L + np.arange(c.shape[0]), weights["layers"], shape, rb)
    return [(np.concatenate([k, nk]), np.concatenate([v, nv]))
            for (k, v), (nk, nv) in zip(cache, new)]


def verify_append_draft(weights, shape, caches, target_logits, drafts, block_feats,
                        block_size: int) -> dict:
    """One cycle of the speculative loop once the target has scored a block.

    Verify the drafts ([Summary] 实践 2), append the anchor and the accepted
    drafts -- whose target features the target produced while scoring the
    block -- to each sequence's context, and draft the next block from the
    bonus token ([Arch] 训练策略 1: every block starts at the verified token).
    Reading R11.

    caches[b]: as in draft_block; target_logits [N, B, V]; drafts [N, B-1];
    block_feats: per fused target layer, [N*B, H] with row b*B + j = slot j
    of sequence b.  Returns accept [N], bonus [N], the new caches, the next
    draft_ids [N, B-1], their top-2 gaps, the block's logits [N, B, V] and
    final hidden states [N, B, H].
    """
    B = int(block_size)
    accept, bonus = verify_greedy(target_logits, drafts)
    new = []
    for b, cache in enumerate(caches):
        rows = slice(b * B, b * B + int(accept[b]) + 1)
        new.append(append_context(cache, weights, shape, [np.asarray(f)[rows] for f in block_feats]))
    d = draft_block(weights, shape, new, bonus, B)
    return {"accept": accept, "bonus": bonus, "caches": new, "draft_ids": d["draft_ids"],
            "gap": d["gap"], "logits": d["logits"], "final_hidden": d["final_hidden"]}


# ------------------------------------------- (N2) training-layout forward

def loss_weights(block_size: int, gamma: float) -> np.ndarray:
    """Weight of draft slots 1..B-1: w_k = exp(-(k-1)/gamma) for the k-th
    predicted token of a block ([Arch] 训练策略 2: earlier slots weigh more,
    because an early miss cascades).  Reading R9: k = slot index j."""
    k = np.arange(1, int(block_size), dtype=np.float64)
    return np.exp(-(k - 1.0) / float(gamma))


def cross_entropy(logits, label) -> np.ndarray:
    """-log softmax(logits)[label] over the last axis, float64."""
    z = _f64(logits)
    m = z.max(axis=-1, keepdims=True)
    lse = m[..., 0] + np.log(np.exp(z - m).sum(axis=-1))
    return lse - np.take_along_axis(z, np.asarray(label)[..., None], axis=-1)[..., 0]


def train_forward(weights, shape, caches, block_seq, anchor_pos, tokens, block_size: int,
                  gamma: float) -> dict:
    """Training-layout forward and its position-weighted loss (readings R8, R9).

    [Arch] 训练策略 1: blocks start at randomly sampled anchor tokens, as each
    draft block at inference starts at a verified token; 技术细节补充 /
    稀疏注意力训练: bidirectional inside a block, no flow between blocks.
    Block i is exactly an inference block whose context is the first a_i rows
    of its sequence's cache, so it is computed as one: ``draft_block`` over
    per-block views of the caches.

    caches[s] = [(K [L_s, Hkv, d], V [L_s, Hkv, d]) per layer]; block_seq,
    anchor_pos: [n]; tokens[s]: the token ids of sequence s (length >
    a_i + B - 1 for its blocks).  Returns logits [n, B, V], slot_loss [n, B-1]
    (cross-entropy of slot j against tokens[s][a_i + j]) and loss (weighted
    mean).
    """
    B = int(block_size)
    views, anchors, labels = [], [], []
    for s_i, a in zip(block_seq, anchor_pos):
        s_i, a = int(s_i), int(a)
        views.append([(k[:a], v[:a]) for k, v in caches[s_i]])
        tok = np.asarray(tokens[s_i])
        anchors.append(int(tok[a]))
        labels.append(tok[a + 1:a + B])
    out = draft_block(weights, shape, views, anchors, B)
    logits = out["logits"]
    labels = np.stack(labels).astype(np.int64)
    slot_loss = cross_entropy(logits[:, 1:, :], labels)
    w = loss_weights(B, gamma)[None, :] * np.ones_like(slot_loss)
    loss = float((w * slot_loss).sum() / w.sum())
    return {"logits": logits, "slot_loss": slot_loss, "loss": loss, "labels": labels}


# ------------------------------------------- (N3) stochastic draft and verify

def softmax_t(z, temperature: float) -> np.ndarray:
    """softmax(z / T) over the last axis, float64."""
    x = _f64(z) / float(temperature)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def gumbel_sample(logits, temperature: float, uniforms) -> np.ndarray:
    """A draw from softmax(logits / T) per row by the Gumbel-max rule:
    argmax_v (z_v / T - log(-log u_v)) with u_v uniform on (0, 1); ties to the
    lowest index (reading R10)."""
    g = -np.log(-np.log(_f64(uniforms)))
    return argmax_lowest(_f64(logits) / float(temperature) + g, axis=-1).astype(np.int32)


def sample_inverse_cdf(w, u: float) -> int:
    """Smallest index whose cumulative weight exceeds u * sum(w) (u in [0, 1))."""
    c = np.cumsum(_f64(w))
    return int(np.searchsorted(c, float(u) * c[-1], side="right"))


def verify_stochastic(target_logits, draft_logits, drafts, temperature: float, r, u) -> tuple:
    """Speculative sampling over one block per sequence (reading R10).

    target_logits [N, B, V]: row j is the target's distribution q_j of the
    token after slot j; draft_logits [N, B, V]: slot j >= 1 proposed drafts[j-1]
    from p_j; r [N, B-1], u [N]: caller uniforms.  Draft k is kept while
    r_k * p_{k+1}(x_k) < q_k(x_k); the first rejected position a gets a fresh
    token from (q_a - p_{a+1})_+, and a fully accepted block a bonus from
    q_{B-1}.  Returns (accept [N], next_token [N]).
    """
    drafts = np.asarray(drafts)
    N, Bm1 = drafts.shape
    q = softmax_t(target_logits, temperature)
    p = softmax_t(draft_logits, temperature)
    accept = np.zeros(N, dtype=np.int32)
    nxt = np.zeros(N, dtype=np.int32)
    for n in range(N):
        a = 0
        while a < Bm1:
            x = int(drafts[n, a])
            if float(r[n, a]) * p[n, a + 1, x] < q[n, a, x]:
                a += 1
            else:
                break
        accept[n] = a
        w = np.maximum(q[n, a] - p[n, a + 1], 0.0) if a < Bm1 else q[n, a]
        nxt[n] = sample_inverse_cdf(w, u[n])
    return accept, nxt
