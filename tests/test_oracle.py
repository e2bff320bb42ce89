"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks the oracle against one of: values worked out from the pages
(tests/golden/), a library routine (torch, transformers' Llama modules), a
closed form or invariant, or brute force on tiny inputs.  Nothing here needs a
GPU.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import oracle as O
from block_diffusion_drafter_concat_amd import configs, synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------ layer rule

def test_layer_ids_golden():
    for ln in _golden_lines("layer_ids.txt"):
        depth, ids = ln.split(":")
        assert O.target_layer_ids(int(depth)) == [int(v) for v in ids.split()]


@pytest.mark.parametrize("n", [5, 6])
def test_layer_ids_properties(n):
    for L in range(n + 3, 160):
        ids = O.target_layer_ids(L, n)
        assert len(ids) == n
        assert ids[0] == 2 and ids[-1] == L - 2
        gaps = np.diff(ids)
        assert np.all(gaps >= 1)
        assert gaps.max() - gaps.min() <= 1
        # each id is a nearest integer to its uniform grid point; halves go up
        from fractions import Fraction
        for k, v in enumerate(ids):
            grid = 2 + Fraction(k * (L - 4), n - 1)
            dist = abs(v - grid)
            assert dist < Fraction(1, 2) or (dist == Fraction(1, 2) and v > grid)


def test_layer_ids_too_shallow():
    with pytest.raises(ValueError):
        O.target_layer_ids(7, 5)


# ------------------------------------------------------------------ bf16 rounding

def test_bf16_round_matches_torch_on_float32():
    g = np.random.default_rng(0)
    x = np.concatenate([
        g.standard_normal(20000).astype(np.float32) * 3,
        (g.standard_normal(2000) * 1e-39).astype(np.float32),        # subnormal range
        (g.standard_normal(2000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 3.3895e38, -3.3896e38, 1e-45], dtype=np.float32),
    ])
    # exact ties: a bf16 value plus half its spacing
    base = synth.to_bf16_values(g.standard_normal(4000).astype(np.float32))
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_round(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_round_float64_is_nearest():
    g = np.random.default_rng(1)
    x = g.standard_normal(5000) * 10.0
    r = O.bf16_round(x)
    # r is a bf16 value
    np.testing.assert_array_equal(torch.from_numpy(r).to(torch.bfloat16).double().numpy(), r)
    # and no bf16 neighbour is closer
    r32 = r.astype(np.float32)
    bits = r32.view(np.uint32).astype(np.int64)
    up = ((bits + (1 << 16)) & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
    dn = ((bits - (1 << 16)) & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.all(np.abs(x - r) <= np.abs(x - up))
    assert np.all(np.abs(x - r) <= np.abs(x - dn))


# ------------------------------------------------------------------ RMSNorm, RoPE

def test_rmsnorm_matches_torch():
    g = np.random.default_rng(2)
    x = g.standard_normal((7, 96)) * 5
    w = 1 + 0.1 * g.standard_normal(96)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(w),
                                        eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(x, w, 1e-6), want, rtol=1e-13, atol=1e-13)
    y = O.rmsnorm(x, np.ones(96), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1.0, rtol=1e-12)


def test_rope_complex_form_and_invariants():
    g = np.random.default_rng(3)
    T, Hh, d, theta = 9, 3, 16, 1e6
    x = g.standard_normal((T, Hh, d))
    pos = g.integers(0, 40000, size=T)
    y = O.rope(x, pos, theta)
    # complex form: z_i = x_i + j x_{i+d/2} multiplied by exp(j p w_i)
    w = np.array([theta ** (-2.0 * i / d) for i in range(d // 2)])
    z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * pos[:, None, None] * w)
    np.testing.assert_allclose(y[..., : d // 2], z.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(y[..., d // 2:], z.imag, rtol=1e-12, atol=1e-12)
    # position 0 is the identity; norms are kept; dot products depend on p - q only
    np.testing.assert_array_equal(O.rope(x, np.zeros(T), theta), x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    q, k = x[:1], x[1:2]
    s1 = np.sum(O.rope(q, [100], theta) * O.rope(k, [37], theta))
    s2 = np.sum(O.rope(q, [100 + 999], theta) * O.rope(k, [37 + 999], theta))
    assert abs(s1 - s2) < 1e-9


def test_rope_matches_transformers(hf_llama):
    transformers, ml = hf_llama
    d, theta = 32, 1e6
    cfg = transformers.LlamaConfig(hidden_size=64, num_attention_heads=2, num_key_value_heads=2,
                                   head_dim=d, rope_parameters={"rope_type": "default",
                                                                "rope_theta": theta})
    rot = ml.LlamaRotaryEmbedding(cfg).double()
    g = np.random.default_rng(4)
    T = 6
    pos = np.array([0, 1, 5, 100, 2047, 30000])
    x = g.standard_normal((T, 2, d))
    xt = torch.from_numpy(x).permute(1, 0, 2)[None]           # [1, heads, T, d]
    cos, sin = rot(xt, torch.from_numpy(pos)[None])
    qh, _ = ml.apply_rotary_pos_emb(xt, xt, cos, sin)
    want = qh[0].permute(1, 0, 2).numpy()
    # transformers forms its inverse frequencies in float32, so its angle error
    # grows like p * 2**-24; a convention error (pairing, sign, exponent) is O(1)
    tol = 1e-6 + 2.0 * pos[:, None, None] * 2.0 ** -24 * np.abs(x).max()
    assert np.all(np.abs(O.rope(x, pos, theta) - want) <= tol)


# ------------------------------------------------------------------ fusion

def test_fusion_is_sum_of_slab_projections():
    g = np.random.default_rng(5)
    T, H, n = 11, 24, 5
    feats = [g.standard_normal((T, H)) for _ in range(n)]
    W = g.standard_normal((H, n * H)) * 0.1
    gain = 1 + 0.1 * g.standard_normal(H)
    Y = sum(f @ W[:, i * H:(i + 1) * H].T for i, f in enumerate(feats))
    want = torch.nn.functional.rms_norm(torch.from_numpy(Y), (H,), torch.from_numpy(gain),
                                        eps=1e-6).numpy()
    np.testing.assert_allclose(O.fuse_context(feats, W, gain, 1e-6, False), want, rtol=1e-12,
                               atol=1e-12)
    # selecting the first slab only gives that slab, normalised
    sel = np.zeros((H, n * H))
    sel[:, :H] = np.eye(H)
    c = O.fuse_context(feats, sel, np.ones(H), 0.0, False)
    want = torch.nn.functional.rms_norm(torch.from_numpy(feats[0]), (H,), eps=0.0).numpy()
    np.testing.assert_allclose(c, want, rtol=1e-12)


def test_fusion_bf16_output_is_bf16():
    g = np.random.default_rng(6)
    feats = [synth.to_bf16_values(g.standard_normal((4, 16)).astype(np.float32)) for _ in range(5)]
    W = synth.to_bf16_values((0.1 * g.standard_normal((16, 80))).astype(np.float32))
    c = O.fuse_context(feats, W, np.ones(16), 1e-6, True)
    np.testing.assert_array_equal(c, torch.from_numpy(c).to(torch.bfloat16).double().numpy())


# ------------------------------------------------------------------ injection

def _tiny_shape(**kw):
    base = dict(n_layers=2, hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, ffn=48,
                vocab=40, dtype="f32")
    base.update(kw)
    return configs.DrafterShape(**base)


def test_incremental_injection_equals_one_shot():
    shape = _tiny_shape(dtype="bf16")
    w = configs.make_weights(shape, 901)
    T = 37
    feats = configs.make_features(shape, 901, T)
    one = O.prefill(w, shape, [feats])[0]
    cache = O.prefill(w, shape, [[f[:5] for f in feats]])[0]
    t = 5
    g = np.random.default_rng(7)
    while t < T:
        n = min(int(g.integers(1, 17)), T - t)
        cache = O.append_context(cache, w, shape, [f[t:t + n] for f in feats])
        t += n
    for (k1, v1), (k2, v2) in zip(one, cache):
        np.testing.assert_array_equal(k1, k2)
        np.testing.assert_array_equal(v1, v2)


def test_injection_position_zero_and_values():
    shape = _tiny_shape()
    w = configs.make_weights(shape, 902)
    c = np.random.default_rng(8).standard_normal((3, shape.hidden))
    kv = O.inject_kv(c, np.zeros(3), w["layers"], shape, False)
    for lw, (k, v) in zip(w["layers"], kv):
        np.testing.assert_allclose(k.reshape(3, -1), c @ lw["wk"].astype(np.float64).T, rtol=1e-12)
        np.testing.assert_allclose(v.reshape(3, -1), c @ lw["wv"].astype(np.float64).T, rtol=1e-12)


# ------------------------------------------------------------------ attention

def _sdpa(q, k, v, mask):
    """torch reference: q [Hq, Lq, d], k/v [Hq, Lk, d], bool mask [Lq, Lk]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask)).numpy()


def test_block_attention_equals_dense_masked_reference():
    """Several sequences packed together, one dense score matrix with a mask.

    Query rows of sequence b may see exactly: b's context keys and b's block
    keys.  The oracle handles one sequence at a time; the reference sees the
    whole pack and relies on the mask alone.
    """
    g = np.random.default_rng(9)
    Hq, Hkv, d, B = 6, 2, 16, 5
    lens = [0, 7, 19]
    qs, ks, vs, cks, cvs = [], [], [], [], []
    for L in lens:
        qs.append(g.standard_normal((B, Hq, d)))
        ks.append(g.standard_normal((B, Hkv, d)))
        vs.append(g.standard_normal((B, Hkv, d)))
        cks.append(g.standard_normal((L, Hkv, d)))
        cvs.append(g.standard_normal((L, Hkv, d)))
    # packed key order: all contexts, then all blocks (so own keys are not adjacent)
    keys = np.concatenate(cks + ks)
    vals = np.concatenate(cvs + vs)
    Q = np.concatenate(qs)
    mask = np.zeros((len(lens) * B, keys.shape[0]), dtype=bool)
    ctx_start = np.cumsum([0] + lens)
    blk0 = ctx_start[-1]
    for b, L in enumerate(lens):
        rows = slice(b * B, (b + 1) * B)
        mask[rows, ctx_start[b]:ctx_start[b] + L] = True
        mask[rows, blk0 + b * B: blk0 + (b + 1) * B] = True
    G = Hq // Hkv
    kk = np.repeat(keys.transpose(1, 0, 2), G, axis=0)
    vv = np.repeat(vals.transpose(1, 0, 2), G, axis=0)
    ref = _sdpa(Q.transpose(1, 0, 2), kk, vv, mask).transpose(1, 0, 2)
    for b in range(len(lens)):
        got = O.block_attention(qs[b], np.concatenate([cks[b], ks[b]]),
                                np.concatenate([cvs[b], vs[b]]))
        np.testing.assert_allclose(got, ref[b * B:(b + 1) * B], rtol=1e-10, atol=1e-12)


def test_block_attention_special_cases():
    g = np.random.default_rng(10)
    # no context, one slot: the output is the slot's own value
    q = g.standard_normal((1, 4, 8))
    k = g.standard_normal((1, 2, 8))
    v = g.standard_normal((1, 2, 8))
    out = O.block_attention(q, k, v)
    np.testing.assert_allclose(out, np.repeat(v, 2, axis=1), rtol=1e-14)
    # Hkv == Hq: textbook multi-head attention with no mask
    q = g.standard_normal((5, 3, 8))
    K = g.standard_normal((12, 3, 8))
    V = g.standard_normal((12, 3, 8))
    ref = _sdpa(q.transpose(1, 0, 2), K.transpose(1, 0, 2), V.transpose(1, 0, 2),
                np.ones((5, 12), bool)).transpose(1, 0, 2)
    np.testing.assert_allclose(O.block_attention(q, K, V), ref, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ whole drafter

def _hf_drafter(transformers, ml, shape, w):
    cfg = transformers.LlamaConfig(
        hidden_size=shape.hidden, intermediate_size=shape.ffn,
        num_attention_heads=shape.n_q_heads, num_key_value_heads=shape.n_kv_heads,
        head_dim=shape.head_dim, num_hidden_layers=shape.n_layers, vocab_size=shape.vocab,
        rms_norm_eps=shape.rms_eps, attention_bias=False, mlp_bias=False,
        rope_parameters={"rope_type": "default", "rope_theta": shape.rope_theta})
    cfg._attn_implementation = "eager"
    layers = []
    for i, lw in enumerate(w["layers"]):
        layer = ml.LlamaDecoderLayer(cfg, layer_idx=i).double()
        t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
        with torch.no_grad():
            layer.input_layernorm.weight.copy_(t(lw["attn_norm"]))
            layer.post_attention_layernorm.weight.copy_(t(lw["ffn_norm"]))
            layer.self_attn.q_proj.weight.copy_(t(lw["wq"]))
            layer.self_attn.k_proj.weight.copy_(t(lw["wk"]))
            layer.self_attn.v_proj.weight.copy_(t(lw["wv"]))
            layer.self_attn.o_proj.weight.copy_(t(lw["wo"]))
            layer.mlp.gate_proj.weight.copy_(t(lw["wg"]))
            layer.mlp.up_proj.weight.copy_(t(lw["wu"]))
            layer.mlp.down_proj.weight.copy_(t(lw["wd"]))
        layers.append(layer)
    rot = ml.LlamaRotaryEmbedding(cfg).double()
    norm = ml.LlamaRMSNorm(shape.hidden, eps=shape.rms_eps).double()
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(w["final_norm"].astype(np.float64)))
    return cfg, layers, rot, norm


class _InjectedCache:
    """Duck-typed cache: the attention sees injected context keys, then its own."""

    def __init__(self, kv):
        self.kv = kv

    def update(self, k, v, layer_idx, *args, **kwargs):
        ck, cv = self.kv[layer_idx]
        return torch.cat([ck, k], dim=2), torch.cat([cv, v], dim=2)


def test_draft_block_matches_transformers_llama(hf_llama):
    """fp32 workload (no rounding): oracle vs transformers' Llama layers in float64.

    The context K/V are built on the transformers side from the oracle's fused
    feature with its own rotary module, so RoPE of the injection is checked too.
    """
    transformers, ml = hf_llama
    shape = _tiny_shape(n_layers=2)
    w = configs.make_weights(shape, 903)
    L, B = 13, 6
    feats = configs.make_features(shape, 903, L)
    c = O.fuse_context(feats, w["fc"], w["fc_norm"], shape.rms_eps, False)
    cache = O.inject_kv(c, np.arange(L), w["layers"], shape, False)
    anchor = 17
    res = O.draft_block(w, shape, [cache], [anchor], B)

    cfg, layers, rot, norm = _hf_drafter(transformers, ml, shape, w)
    ct = torch.from_numpy(c)[None]                            # [1, L, H]
    cos_c, sin_c = rot(ct, torch.arange(L)[None])
    kv = []
    for layer in layers:
        a = layer.self_attn
        k = a.k_proj(ct).view(1, L, shape.n_kv_heads, shape.head_dim).transpose(1, 2)
        v = a.v_proj(ct).view(1, L, shape.n_kv_heads, shape.head_dim).transpose(1, 2)
        k, _ = ml.apply_rotary_pos_emb(k, k, cos_c, sin_c)
        kv.append((k, v))
    tokens = [anchor] + [shape.mask_token_id] * (B - 1)
    x = torch.from_numpy(w["embed"][tokens].astype(np.float64))[None]
    pos = torch.arange(L, L + B)[None]
    cos, sin = rot(x, pos)
    cache_obj = _InjectedCache(kv)
    with torch.no_grad():
        for layer in layers:
            x = layer(x, attention_mask=None, position_ids=pos, past_key_values=cache_obj,
                      position_embeddings=(cos, sin))
            if isinstance(x, tuple):
                x = x[0]
        z = norm(x) @ torch.from_numpy(w["lm_head"].astype(np.float64)).T
    # transformers' eager softmax runs in float32, hence the tolerance
    np.testing.assert_allclose(res["final_hidden"][0], x[0].numpy(), rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(res["logits"][0], z[0].numpy(), rtol=1e-5, atol=1e-6)
    zz = z[0, 1:].numpy()
    ok = res["gap"][0] > 1e-4
    np.testing.assert_array_equal(res["draft_ids"][0][ok], np.argmax(zz, axis=1)[ok])


def _tiny_batch(shape, wid, lens, B=6):
    w = configs.make_weights(shape, wid)
    feats = [configs.make_features(shape, wid, L, name=f"s{b}") for b, L in enumerate(lens)]
    caches = O.prefill(w, shape, feats)
    anchors = configs.make_anchors(shape, wid, len(lens))
    return w, caches, anchors


def test_no_flow_between_sequences():
    shape = _tiny_shape(dtype="bf16")
    w, caches, anchors = _tiny_batch(shape, 904, [9, 4, 15])
    base = O.draft_block(w, shape, caches, anchors, 6)
    caches2 = [caches[0], [(k + 1.0, v - 2.0) for k, v in caches[1]], caches[2]]
    anchors2 = anchors.copy()
    anchors2[1] = (anchors2[1] + 3) % (shape.vocab - 1)
    pert = O.draft_block(w, shape, caches2, anchors2, 6)
    for key in ("final_hidden", "logits"):
        np.testing.assert_array_equal(base[key][0], pert[key][0])
        np.testing.assert_array_equal(base[key][2], pert[key][2])
        assert not np.array_equal(base[key][1], pert[key][1])


def test_block_is_bidirectional_not_causal():
    """All mask slots with the same position see the same keys: equal outputs.

    Under a causal mask slot j would see j copies of the mask key and the
    outputs would differ.
    """
    shape = _tiny_shape()
    w = configs.make_weights(shape, 905)
    L, B = 8, 7
    c = np.random.default_rng(11).standard_normal((L, shape.hidden))
    cache = O.inject_kv(c, np.arange(L), w["layers"], shape, False)
    x = w["embed"][[5] + [shape.mask_token_id] * (B - 1)].astype(np.float64)
    for lw, (kc, vc) in zip(w["layers"], cache):
        x = O.decoder_layer(x, np.zeros(B), lw, kc, vc, shape, False)
    for j in range(2, B):
        np.testing.assert_allclose(x[j], x[1], rtol=1e-13, atol=1e-13)
    assert not np.allclose(x[0], x[1])


def test_relative_positions_only():
    shape = _tiny_shape()
    w = configs.make_weights(shape, 906)
    L, B, s = 10, 5, 1234
    c = np.random.default_rng(12).standard_normal((L, shape.hidden))
    out = []
    for shift in (0, s):
        cache = O.inject_kv(c, shift + np.arange(L), w["layers"], shape, False)
        x = w["embed"][[3] + [shape.mask_token_id] * (B - 1)].astype(np.float64)
        for lw, (kc, vc) in zip(w["layers"], cache):
            x = O.decoder_layer(x, shift + L + np.arange(B), lw, kc, vc, shape, False)
        out.append(x)
    np.testing.assert_allclose(out[0], out[1], rtol=1e-8, atol=1e-9)


def test_single_pass_uses_each_weight_once(monkeypatch):
    """One call = one forward pass: every layer runs once, the LM head once."""
    shape = _tiny_shape()
    w, caches, anchors = _tiny_batch(shape, 907, [6])
    calls = []
    real = O.dflash_oracle.decoder_layer

    def counting(*a, **k):
        calls.append(1)
        return real(*a, **k)

    monkeypatch.setattr(O.dflash_oracle, "decoder_layer", counting)
    O.draft_block(w, shape, caches, anchors, 8)
    assert len(calls) == shape.n_layers


def test_argmax_ties_lowest_index():
    z = np.array([[0.0, 3.0, 1.0, 3.0], [5.0, 5.0, 5.0, 5.0], [-1.0, -2.0, -1.0, -3.0]])
    np.testing.assert_array_equal(O.argmax_lowest(z), [1, 0, 0])


# ------------------------------------------------------------------ verify

def _literal_accept(t, d):
    """Longest m such that the first m target choices equal the first m drafts."""
    best = 0
    for m in range(len(d) + 1):
        if all(t[j] == d[j] for j in range(m)):
            best = m
    return best


def test_verify_brute_force_tiny():
    V = 4
    for B in (2, 3, 4):
        for t in itertools.product(range(V), repeat=B):
            for d in itertools.product(range(V), repeat=B - 1):
                logits = np.zeros((1, B, V))
                for j, tj in enumerate(t):
                    # ties everywhere below tj: the row max sits at tj and at
                    # every higher column, so only the lowest-index rule gives tj
                    logits[0, j, tj:] = 1.0
                acc, bon = O.verify_greedy(logits, np.array([d]))
                a = _literal_accept(t, d)
                assert acc[0] == a and bon[0] == t[a], (t, d)


def test_verify_planted_logits_recover_accept():
    V, B, N = 300, 16, 40
    g = np.random.default_rng(13)
    drafts = g.integers(0, V, size=(N, B - 1))
    accept = g.integers(0, B, size=N)
    ties = g.random(N) < 0.3
    for dt in ("f32", "bf16"):
        logits = synth.plant_target_logits(
            synth.values((N, B, V), dt, 99, synth.STREAM_LOGITS, "l"), drafts, accept, dt,
            tie_rows=ties, workload=99)
        acc, bon = O.verify_greedy(logits, drafts)
        np.testing.assert_array_equal(acc, accept)
        rows = logits[np.arange(N), accept]
        assert np.all(rows[np.arange(N), bon] == rows.max(axis=1))
        for n in np.nonzero(ties)[0]:
            top = np.nonzero(rows[n] == rows[n].max())[0]
            assert len(top) == 2 and bon[n] == top[0]


# ------------------------------------------------------------------ lossless loop

def test_speculative_loop_is_lossless(hf_llama):
    """Greedy speculative decoding with the oracle drafter = plain greedy decoding.

    A tiny random transformers Llama plays the target.  Whatever the drafter
    proposes, the committed tokens must equal the target's own greedy output
    ([Summary] FAQ 4).  A drafter that proposes the true continuation must have
    every draft accepted, which checks that row j of the target is compared with
    slot j + 1 of the block.
    """
    transformers, ml = hf_llama
    torch.manual_seed(0)
    n_t_layers, H, V = 8, 32, 40
    tcfg = transformers.LlamaConfig(hidden_size=H, intermediate_size=64, num_attention_heads=4,
                                    num_key_value_heads=2, head_dim=8,
                                    num_hidden_layers=n_t_layers, vocab_size=V,
                                    rms_norm_eps=1e-6, initializer_range=0.5)
    tcfg._attn_implementation = "eager"
    target = transformers.LlamaForCausalLM(tcfg).double().eval()
    ids = O.target_layer_ids(n_t_layers)
    shape = _tiny_shape(hidden=H, vocab=V)
    w = configs.make_weights(shape, 908)

    def run(seq):
        with torch.no_grad():
            out = target(torch.tensor([seq]), output_hidden_states=True)
        feats = [out.hidden_states[i][0].numpy() for i in ids]
        return out.logits[0].numpy(), feats

    prompt = [3, 14, 15, 9, 2, 6]
    n_new = 40
    plain = list(prompt)
    for _ in range(n_new):
        plain.append(int(np.argmax(run(plain)[0][-1])))

    for perfect in (False, True):
        B = 5
        seq = list(prompt)
        logits, feats = run(seq)
        cache = O.prefill(w, shape, [feats])[0]
        anchor = int(np.argmax(logits[-1]))
        accepted = []
        while len(seq) + 1 < len(prompt) + n_new:
            P = len(seq)
            if perfect:
                drafts = np.array([plain[P + 1: P + B]])
                if drafts.shape[1] < B - 1:
                    drafts = np.pad(drafts, ((0, 0), (0, B - 1 - drafts.shape[1])))
            else:
                drafts = O.draft_block(w, shape, [cache], [anchor], B)["draft_ids"]
            blk = [anchor] + [int(t) for t in drafts[0]]
            tl, tf = run(seq + blk)
            a, bonus = O.verify_greedy(tl[None, P:P + B], drafts)
            a = int(a[0])
            accepted.append(a)
            seq += blk[: a + 1]
            cache = O.append_context(cache, w, shape, [f[P:P + a + 1] for f in tf])
            anchor = int(bonus[0])
        seq.append(anchor)
        n = min(len(seq), len(plain))
        assert seq[:n] == plain[:n]
        if perfect:
            assert all(a == B - 1 for a in accepted[:-1])


def test_verify_append_draft_matches_one_shot_context(hf_llama):
    """The loop cycle keeps the context equal to a fresh prefill of everything committed.

    A tiny random Llama is the target.  Each cycle it scores [anchor, drafts]
    and hands over its hidden states at those positions; the drafts follow
    the target's own continuation for a planned number of slots (0 .. B-1,
    different per sequence) and then go wrong, so the accepted count is
    known.  After verify_append_draft the caches must equal the prefill of
    the target's features over the whole committed sequence (run again from
    scratch), the next drafts must be those drafted on that prefill from the
    bonus token, and the committed tokens must be the target's own greedy
    output.  A wrong slot range, a position shift or a stale anchor fails.
    """
    transformers, ml = hf_llama
    torch.manual_seed(1)
    n_t_layers, H, V = 8, 32, 40
    tcfg = transformers.LlamaConfig(hidden_size=H, intermediate_size=64, num_attention_heads=4,
                                    num_key_value_heads=2, head_dim=8,
                                    num_hidden_layers=n_t_layers, vocab_size=V,
                                    rms_norm_eps=1e-6, initializer_range=0.5)
    tcfg._attn_implementation = "eager"
    target = transformers.LlamaForCausalLM(tcfg).double().eval()
    ids = O.target_layer_ids(n_t_layers)
    shape = _tiny_shape(hidden=H, vocab=V)
    w = configs.make_weights(shape, 911)

    def run(seq):
        with torch.no_grad():
            out = target(torch.tensor([seq]), output_hidden_states=True)
        return out.logits[0].numpy(), [out.hidden_states[i][0].numpy() for i in ids]

    B, n_new, N = 4, 40, 2
    prompts = [[3, 14, 15, 9, 2, 6], [7, 1, 8, 2, 8]]
    plain = [list(p) for p in prompts]
    for b in range(N):
        for _ in range(n_new):
            plain[b].append(int(np.argmax(run(plain[b])[0][-1])))

    seqs = [list(p) for p in prompts]
    caches, anchors = [], []
    for b in range(N):
        lg, fs = run(seqs[b])
        caches += O.prefill(w, shape, [fs])
        anchors.append(int(np.argmax(lg[-1])))
    plan = [[0, 3, 1, 2, 3, 0], [2, 0, 3, 3, 1, 2]]   # accepted drafts per cycle
    for cyc in range(len(plan[0])):
        drafts = np.zeros((N, B - 1), dtype=np.int64)
        tls, feats = [], [[] for _ in ids]
        for b in range(N):
            P = len(seqs[b])
            true = plain[b][P + 1:P + B]
            a = plan[b][cyc]
            drafts[b] = [true[j] if j < a else (true[j] + 1 + j) % V for j in range(B - 1)]
            tl, tf = run(seqs[b] + [anchors[b]] + [int(t) for t in drafts[b]])
            tls.append(tl[P:P + B])
            for i, f in enumerate(tf):
                feats[i].append(f[P:P + B])
        feats = [np.concatenate(f) for f in feats]
        st = O.verify_append_draft(w, shape, caches, np.stack(tls), drafts, feats, B)
        np.testing.assert_array_equal(st["accept"], [plan[b][cyc] for b in range(N)])
        fresh = []
        for b in range(N):
            seqs[b] += [anchors[b]] + [int(t) for t in drafts[b][:plan[b][cyc]]]
            fresh += O.prefill(w, shape, [run(seqs[b])[1]])
        # (the target's RMSNorm runs in float32 even on a float64 model, so
        # its features for the same prefix differ by ~1e-8 between runs of
        # different length; a wrong row or position differs by ~0.1)
        for b in range(N):
            assert st["caches"][b][0][0].shape[0] == len(seqs[b])
            for (k1, v1), (k2, v2) in zip(st["caches"][b], fresh[b]):
                np.testing.assert_allclose(k1, k2, rtol=0, atol=1e-6)
                np.testing.assert_allclose(v1, v2, rtol=0, atol=1e-6)
        again = O.draft_block(w, shape, fresh, st["bonus"], B)
        np.testing.assert_array_equal(st["draft_ids"], again["draft_ids"])
        caches, anchors = st["caches"], [int(x) for x in st["bonus"]]
        for b in range(N):
            assert seqs[b] + [anchors[b]] == plain[b][:len(seqs[b]) + 1]


# ------------------------------------------------------------------ scale anchor

def test_param_count_matches_2b_claim():
    want = int(_golden_lines("param_scale.txt")[0].split(":")[1])
    p = configs.TARGET_27B_LIKE.drafter_params()
    assert round(p / 1e9) == want


# ------------------------------------------------------------ training layout

def test_loss_weights_properties():
    """w_k = exp(-(k-1)/gamma): the first draft slot weighs 1, the weights fall
    geometrically with ratio exp(-1/gamma), and a large gamma is uniform."""
    for B, gamma in [(2, 1.0), (8, 3.0), (16, 7.0)]:
        w = O.loss_weights(B, gamma)
        assert w.shape == (B - 1,) and w[0] == 1.0
        assert np.all(np.diff(w) < 0) or B == 2
        np.testing.assert_allclose(w[1:] / w[:-1], np.full(B - 2, np.e ** (-1.0 / gamma)),
                                   rtol=1e-14)
    np.testing.assert_allclose(O.loss_weights(16, 1e12), np.ones(15), rtol=1e-10)


def test_cross_entropy_matches_torch_and_limits():
    g = np.random.default_rng(31)
    z = g.standard_normal((3, 5, 17)) * 4
    lab = g.integers(0, 17, size=(3, 5))
    want = torch.nn.functional.cross_entropy(torch.from_numpy(z).reshape(-1, 17),
                                             torch.from_numpy(lab).reshape(-1),
                                             reduction="none").numpy().reshape(3, 5)
    np.testing.assert_allclose(O.cross_entropy(z, lab), want, rtol=1e-12, atol=1e-12)
    # equal logits: log V; one dominant logit at the label: ~0; far from it: the gap
    np.testing.assert_allclose(O.cross_entropy(np.zeros((2, 9)), [0, 4]), np.log(9), rtol=1e-14)
    big = np.zeros(6); big[2] = 800.0
    assert O.cross_entropy(big, 2) < 1e-300 + 1e-12
    np.testing.assert_allclose(O.cross_entropy(big, 0), 800.0, rtol=1e-14)


def _train_case(dtype="f32"):
    shape = _tiny_shape(dtype=dtype)
    w = configs.make_weights(shape, 921)
    lens = [13, 0, 29]
    feats = [configs.make_features(shape, 921, L, name=f"s{s}_") if L else None
             for s, L in enumerate(lens)]
    caches = []
    for f, L in zip(feats, lens):
        if L:
            caches += O.prefill(w, shape, [f])
        else:
            caches.append([(np.zeros((0, shape.n_kv_heads, shape.head_dim)),) * 2
                           for _ in range(shape.n_layers)])
    tokens, bseq, apos = configs.make_training_layout(shape, 921, lens, 4, 6)
    return shape, w, feats, caches, tokens, bseq, apos


def test_training_block_equals_inference_on_the_prefix():
    """Block i of the training layout is the inference draft of the sequence
    cut at its anchor: its context cache is the prefill of the first a_i
    feature rows (injection is per row and position), its anchor the token at
    a_i, its positions a_i .. a_i + B - 1."""
    shape, w, feats, caches, tokens, bseq, apos = _train_case()
    B = 6
    out = O.train_forward(w, shape, caches, bseq, apos, tokens, B, gamma=4.0)
    for i, (s, a) in enumerate(zip(bseq, apos)):
        if a:
            pre = O.prefill(w, shape, [[f[:a] for f in feats[s]]])
        else:
            pre = [[(np.zeros((0, shape.n_kv_heads, shape.head_dim)),) * 2
                    for _ in range(shape.n_layers)]]
        ref = O.draft_block(w, shape, pre, [tokens[s][a]], B)
        np.testing.assert_allclose(out["logits"][i], ref["logits"][0], rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(out["labels"][i], tokens[s][a + 1:a + B])


def test_training_blocks_see_nothing_past_their_anchor_or_each_other():
    shape, w, feats, caches, tokens, bseq, apos = _train_case()
    B = 6
    out = O.train_forward(w, shape, caches, bseq, apos, tokens, B, gamma=4.0)
    # rows at or after every anchor of sequence 2 replaced by noise: no block of
    # sequence 2 may change; rows before the last anchor do matter
    s2 = [i for i in range(len(bseq)) if bseq[i] == 2]
    a_min = min(apos[i] for i in s2)
    g = np.random.default_rng(5)
    noisy = [list(c) for c in caches]
    noisy[2] = [(np.concatenate([k[:a_min], g.standard_normal(k[a_min:].shape)]),
                 np.concatenate([v[:a_min], g.standard_normal(v[a_min:].shape)]))
                for k, v in caches[2]]
    out2 = O.train_forward(w, shape, noisy, bseq, apos, tokens, B, gamma=4.0)
    for i in range(len(bseq)):
        if bseq[i] != 2 or apos[i] == a_min:
            np.testing.assert_array_equal(out2["logits"][i], out["logits"][i])
        else:
            assert np.abs(out2["logits"][i] - out["logits"][i]).max() > 1e-6
    # one block alone gives the same numbers as inside the whole layout (up to
    # the summation order of the stacked row products)
    for i in (0, len(bseq) - 1):
        one = O.train_forward(w, shape, caches, bseq[i:i + 1], apos[i:i + 1], tokens, B, 4.0)
        np.testing.assert_allclose(one["logits"][0], out["logits"][i], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(one["slot_loss"][0], out["slot_loss"][i], rtol=1e-12)


def test_training_loss_is_the_weighted_mean_of_slot_losses():
    shape, w, feats, caches, tokens, bseq, apos = _train_case()
    B = 6
    out = O.train_forward(w, shape, caches, bseq, apos, tokens, B, gamma=2.5)
    z = torch.from_numpy(out["logits"][:, 1:, :]).reshape(-1, shape.vocab)
    ce = torch.nn.functional.cross_entropy(z, torch.from_numpy(out["labels"]).reshape(-1),
                                           reduction="none").numpy().reshape(-1, B - 1)
    np.testing.assert_allclose(out["slot_loss"], ce, rtol=1e-12, atol=1e-12)
    big = O.train_forward(w, shape, caches, bseq, apos, tokens, B, gamma=1e15)
    np.testing.assert_allclose(big["loss"], ce.mean(), rtol=1e-12)
    # gamma -> 0: only the first draft slot of each block counts
    small = O.train_forward(w, shape, caches, bseq, apos, tokens, B, gamma=1e-3)
    np.testing.assert_allclose(small["loss"], ce[:, 0].mean(), rtol=1e-9)


def test_multi_block_attention_equals_dense_masked_reference():
    """Several blocks of one sequence at different anchors, packed with the
    sequence's whole context: block i may see context rows before a_i and its
    own block (inter-block flow blocked), nothing else."""
    g = np.random.default_rng(12)
    Hq, Hkv, d, B, L = 4, 2, 8, 4, 23
    anchors = [0, 5, 5, 23]
    ck, cv = g.standard_normal((L, Hkv, d)), g.standard_normal((L, Hkv, d))
    qs = [g.standard_normal((B, Hq, d)) for _ in anchors]
    ks = [g.standard_normal((B, Hkv, d)) for _ in anchors]
    vs = [g.standard_normal((B, Hkv, d)) for _ in anchors]
    keys = np.concatenate([ck] + ks)
    vals = np.concatenate([cv] + vs)
    mask = np.zeros((len(anchors) * B, keys.shape[0]), dtype=bool)
    for i, a in enumerate(anchors):
        mask[i * B:(i + 1) * B, :a] = True
        mask[i * B:(i + 1) * B, L + i * B:L + (i + 1) * B] = True
    G = Hq // Hkv
    kk = np.repeat(keys.transpose(1, 0, 2), G, axis=0)
    vv = np.repeat(vals.transpose(1, 0, 2), G, axis=0)
    ref = _sdpa(np.concatenate(qs).transpose(1, 0, 2), kk, vv, mask).transpose(1, 0, 2)
    for i, a in enumerate(anchors):
        got = O.block_attention(qs[i], np.concatenate([ck[:a], ks[i]]),
                                np.concatenate([cv[:a], vs[i]]))
        np.testing.assert_allclose(got, ref[i * B:(i + 1) * B], rtol=1e-10, atol=1e-12)


# ------------------------------------------------- stochastic draft and verify

def test_inverse_cdf_closed_forms():
    assert O.sample_inverse_cdf([0, 0, 5, 0], 0.0) == 2
    assert O.sample_inverse_cdf([0, 0, 5, 0], 0.999) == 2
    assert O.sample_inverse_cdf([1, 0, 3], 0.0) == 0
    assert O.sample_inverse_cdf([1, 0, 3], 0.2499) == 0
    assert O.sample_inverse_cdf([1, 0, 3], 0.25) == 2      # boundary goes right
    g = np.random.default_rng(41)
    w = g.random(17)
    us = np.sort(g.random(50))
    idx = [O.sample_inverse_cdf(w, u) for u in us]
    assert all(a <= b for a, b in zip(idx, idx[1:])) and 0 <= idx[0] and idx[-1] < 17


def test_gumbel_sample_limits_and_frequencies():
    g = np.random.default_rng(42)
    z = g.standard_normal((3, 9)) * 3
    u = g.random((3, 9))
    # a vanishing temperature is the greedy argmax; equal logits pick the largest u
    np.testing.assert_array_equal(O.gumbel_sample(z, 1e-9, u), O.argmax_lowest(z, axis=1))
    np.testing.assert_array_equal(O.gumbel_sample(np.zeros((3, 9)), 1.0, u), np.argmax(u, axis=1))
    # frequencies of 40000 seeded draws against softmax(z / T)
    zz = np.array([0.3, -1.0, 1.2, 0.0, 0.7])
    T = 0.8
    uu = g.random((40000, 5))
    ids = O.gumbel_sample(np.broadcast_to(zz, (40000, 5)), T, uu)
    freq = np.bincount(ids, minlength=5) / 40000
    assert np.abs(freq - O.softmax_t(zz, T)).max() < 0.01


def _verify_first_token_law(q_logits, p_logits, T, K):
    """Law of the first emitted token of a 2-slot block (one draft): the draft x
    weighted by p(x), r and u on K-point midpoint grids."""
    V = q_logits.shape[-1]
    p = O.softmax_t(p_logits, T)
    xs, rs, us = np.meshgrid(np.arange(V), (np.arange(K) + 0.5) / K, (np.arange(K) + 0.5) / K,
                             indexing="ij")
    n = xs.size
    tl = np.broadcast_to(q_logits, (n, 2, V))
    dl = np.broadcast_to(p_logits, (n, 2, V))
    acc, nxt = O.verify_stochastic(tl, dl, xs.reshape(n, 1), T, rs.reshape(n, 1), us.reshape(n))
    first = np.where(acc > 0, xs.reshape(n), nxt)
    law = np.zeros(V)
    np.add.at(law, first, p[1][xs.reshape(n)] / (K * K))
    return law


def test_stochastic_verify_is_lossless():
    """The first emitted token follows the target's distribution q_0 whatever
    the drafter's p is (grid integration over the draft, r and u)."""
    g = np.random.default_rng(43)
    V, T = 4, 0.9
    for _ in range(3):
        ql = np.stack([g.standard_normal(V) * 1.5, g.standard_normal(V)])
        pl = np.stack([np.zeros(V), g.standard_normal(V) * 1.5])
        law = _verify_first_token_law(ql, pl, T, 120)
        np.testing.assert_allclose(law, O.softmax_t(ql[0], T), atol=2.5 / 120)


def test_stochastic_verify_special_cases():
    g = np.random.default_rng(44)
    N, B, V = 6, 5, 11
    tl = g.standard_normal((N, B, V)) * 2
    # drafter equal to the target (slot j proposes what row j-1 predicts): all accepted,
    # the next token comes from the last row
    dl = np.concatenate([np.zeros((N, 1, V)), tl[:, :-1, :]], axis=1)
    drafts = g.integers(0, V, size=(N, B - 1))
    r = g.random((N, B - 1)) * 0.999
    u = g.random(N)
    acc, nxt = O.verify_stochastic(tl, dl, drafts, 1.3, r, u)
    assert (acc == B - 1).all()
    for n in range(N):
        assert nxt[n] == O.sample_inverse_cdf(O.softmax_t(tl[n, -1], 1.3), u[n])
    # vanishing temperature with greedy drafts: the greedy rule (accept length and bonus)
    dl = g.standard_normal((N, B, V)) * 2
    gdr = O.argmax_lowest(dl[:, 1:, :], axis=2)
    planted = tl.copy()
    for n in range(N):          # plant agreement for the first n % B drafts
        for j in range(min(n % B, B - 1)):
            planted[n, j, gdr[n, j]] = planted[n, j].max() + 1.0
    acc, nxt = O.verify_stochastic(planted, dl, gdr, 1e-9, r, u)
    ga, gb = O.verify_greedy(planted, gdr)
    np.testing.assert_array_equal(acc, ga)
    np.testing.assert_array_equal(nxt, gb)
