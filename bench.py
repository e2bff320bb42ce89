#!/usr/bin/env python3
"""Draft-block throughput of the DFlash drafter hot path on one MI355X.

Workload: Qwen3-8B-shaped bf16 drafter (5 layers, hidden 4096, 32/8 heads of
128, SwiGLU 12288, shared embedding / LM head over 151936 tokens), batch 1,
context 2048, blocks of 16 slots.  Synthetic seeded weights and inputs.

One step = the drafter's share of one speculative cycle, every row of the hot
path once:
  fuse the target features of the n tokens committed last cycle (n ~ accept
  length, Geometric(0.15) capped at 16) -> inject them into every layer's
  cache at positions 2048-n .. 2047 (the context stays 2048) -> draft one
  16-slot block in one forward pass -> greedy-verify it against synthetic
  target logits.  The bonus token of step i anchors step i+1 on the device.

Prints one JSON line: blocks/s, the dominant kernel's roofline figures
(measured live with HIP events on the library's stream) and the CPU oracle
timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/s (16-tok, 5-layer drafter, ctx 2048) + % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
CTX, BLOCK, BATCH = 2048, 16, 1


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pack", action="store_true",
                    help="leave the weights row-major (no dflash_pack_weights copy)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-timing-pass", action="store_true",
                    help="skip the per-section timing pass (for counter collection)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the batch-16 / long-context / 27B-shaped kernel measurements")
    ap.add_argument("--kernel-probe", action="store_true",
                    help="only run the kernels whose counters the profiles report (2048-row "
                         "prefill fusion and injection, batch-16 ragged draft, 35K-context "
                         "draft, batch-16 greedy verify), three calls each, and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, 5 times "
                         "(scale reference for HBM byte counters) and exit")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)


def kernel_probe(torch, L, configs) -> None:
    """Three calls each of the kernels the counter profiles cover, on the
    Qwen3-8B-shaped drafter with device-drawn weights: the 2048-row prefill
    fusion and injection (MFMA-bound), a batch-16 ragged draft and a 35K-context
    draft (block attention), and a batch-16 greedy verify."""
    shape = configs.QWEN3_8B_LIKE
    dr = packed(torch, L.Drafter(shape, device_weights(torch, shape, 11)))
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    feats = [torch.randn((CTX, shape.hidden), generator=g, device="cuda").to(torch.bfloat16)
             for _ in range(shape.n_feat)]
    ctx = torch.empty((CTX, shape.hidden), dtype=torch.bfloat16, device="cuda")
    cache = L.KVCache(shape, [CTX + 64])
    ws = dr.workspace(1, BLOCK, CTX)
    for _ in range(3):
        dr.fuse_context(feats, ctx, ws)
        dr.inject_kv(ctx, [CTX], cache, ws, pos_start=[0])
    torch.cuda.synchronize()
    log("probe: prefill done")
    del feats, ctx, cache, ws
    for lens, seed in ((list(configs.qwen3_8b_b16_ragged().ctx), 3001), ([35000], 3002)):
        cache = L.KVCache(shape, [n + 64 for n in lens])
        fill_cache(torch, cache, lens, seed)
        nb = len(lens)
        anchors = torch.from_numpy(configs.make_anchors(shape, 2, nb)).cuda()
        draft = torch.empty((nb, BLOCK - 1), dtype=torch.int32, device="cuda")
        ws = dr.workspace(nb, BLOCK, 1)
        for _ in range(3):
            dr.draft_block(cache, BLOCK, anchors, draft, ws)
        torch.cuda.synchronize()
        log(f"probe: draft of {nb} sequence(s) done")
        del cache, ws
    nb = 16
    logits = torch.randn((nb, BLOCK, shape.vocab), generator=g, device="cuda").to(torch.bfloat16)
    drafts = torch.randint(0, shape.vocab, (nb, BLOCK - 1), generator=g, device="cuda",
                           dtype=torch.int32)
    acc = torch.empty(nb, dtype=torch.int32, device="cuda")
    bon = torch.empty(nb, dtype=torch.int32, device="cuda")
    vws = torch.empty(L.verify_workspace_size(nb, BLOCK, shape.vocab), dtype=torch.uint8,
                      device="cuda")
    for _ in range(3):
        L.verify_greedy(logits, drafts, acc, bon, vws)
    torch.cuda.synchronize()
    dr.close()
    log("probe: verify done")
    print(json.dumps({"kernel_probe": "done"}), flush=True)


def lm_head_traffic():
    """HBM bytes per LM-head launch from the committed rocprofv3 counter record,
    or None when the kernel's sources differ from the ones it was taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "counters_lm_head.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return int(rec["fetch_kib_per_launch"] * 1024 * rec["fetch_scale"] +
                   rec["write_kib_per_launch"] * 1024 * rec["write_scale"])
    except (OSError, KeyError, ValueError):
        return None


def time_prefill(torch, dr, shape, feats_dev, ctx_all, cache, ws, reps: int = 5) -> dict:
    """Fusion and injection GEMMs over the 2048-row prefill (MFMA-bound)."""
    H, T = shape.hidden, CTX
    fuse_flops = 2.0 * T * shape.n_feat * H * H
    inj_flops = 2.0 * T * H * shape.n_layers * 2 * shape.kv_dim
    sec = [("fuse_gemm", -1), ("inject", -1)]
    evs = []
    for _ in range(reps):
        pts = []
        for s_, l in sec:
            a = TimingEvent(torch)
            b = TimingEvent(torch)
            a.record()
            b.record()
            pts.append((s_, l, a, b))
        evs.append(pts)
    torch.cuda.synchronize()
    for pts in evs:
        dr.set_timing(pts)
        dr.fuse_context(feats_dev, ctx_all, ws)
        dr.inject_kv(ctx_all, [CTX], cache, ws, pos_start=[0])
    dr.set_timing([])
    torch.cuda.synchronize()
    f_us = float(np.mean([p[0][2].elapsed_time(p[0][3]) for p in evs])) * 1e3
    i_us = float(np.mean([p[1][2].elapsed_time(p[1][3]) for p in evs])) * 1e3
    out = {}
    for name, us, fl in (("fusion_gemm", f_us, fuse_flops), ("injection_gemm", i_us, inj_flops)):
        tf = fl / (us * 1e-6) / 1e12
        out[name] = {"rows": T, "avg_us": round(us, 2), "TFLOP/s": round(tf, 1),
                     "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    return out


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it adds a timestamp without the system-scope fence (cache
    write-back and invalidation) that a default event performs, which would
    otherwise land between the kernels being timed and inflate them."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes
        if TimingEvent._hip is None:
            # the runtime torch already loaded (same soname as the library's)
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so.7")
        self._torch = torch
        h = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(h),
                                                      ctypes.c_uint(self.DISABLE_SYSTEM_FENCE))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.cuda_event = h.value

    def record(self) -> None:
        import ctypes
        st = self._torch.cuda.current_stream().cuda_stream
        rc = TimingEvent._hip.hipEventRecord(ctypes.c_void_p(self.cuda_event), ctypes.c_void_p(st))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        import ctypes
        ms = ctypes.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.cuda_event),
                                                  ctypes.c_void_p(end.cuda_event))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def __del__(self):
        import ctypes
        if TimingEvent._hip is not None and self.cuda_event:
            TimingEvent._hip.hipEventDestroy(ctypes.c_void_p(self.cuda_event))


def section_times(torch, dr, fn, sections, reps: int) -> dict:
    """Mean duration (ms) per section name over every layer and repetition,
    from HIP events the library records around each section of ``fn()``."""
    runs = []
    for _ in range(reps):
        pts = []
        for s_, l in sections:
            a = TimingEvent(torch)
            b = TimingEvent(torch)
            a.record()
            b.record()
            pts.append((s_, l, a, b))
        runs.append(pts)
    torch.cuda.synchronize()
    for pts in runs:
        dr.set_timing(pts)
        fn()
    dr.set_timing([])
    torch.cuda.synchronize()
    acc = {}
    for pts in runs:
        for s_, l, a, b in pts:
            acc.setdefault(s_, []).append(a.elapsed_time(b))
    return {k: float(np.mean(v)) for k, v in acc.items()}


def event_time_ms(torch, fn, reps: int, warm: int = 2) -> float:
    """Mean ms per call of ``fn`` over ``reps`` back-to-back calls."""
    for _ in range(warm):
        fn()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def layer_sections(n_layers: int) -> list:
    out = [("lm_head", -1), ("lm_gemm", -1), ("embed", -1), ("final_norm", -1)]
    for l in range(n_layers):
        out += [("qkv", l), ("attention", l), ("o_proj", l), ("gate_up", l), ("down", l)]
    return out


def kernel_report(shape, kern_ms: dict, M: int, kv_rows: int) -> dict:
    """HBM fraction per kernel: weight bytes (+ the M activation rows) for the
    GEMMs, K and V rows for attention (per layer, per launch)."""
    H, F, qd, kvd, V = shape.hidden, shape.ffn, shape.q_dim, shape.kv_dim, shape.vocab
    s = 2
    kb = {"qkv": (qd + 2 * kvd) * H * s + M * H * s, "o_proj": H * qd * s + M * qd * s,
          "gate_up": 2 * F * H * s + M * H * s, "down": H * F * s + M * F * s,
          "lm_head": V * H * s + M * H * s, "lm_gemm": V * H * s + M * H * s,
          "attention": kv_rows * kvd * 2 * s}
    out = {}
    for k, ms in kern_ms.items():
        e = {"avg_us": round(ms * 1e3, 2)}
        if k in kb:
            gbs = kb[k] / (ms * 1e-3) / 1e9
            e.update({"bytes": kb[k], "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        out[k] = e
    return out


PACK = True   # pack the bf16 GEMM weights for the LDS-tiled GEMMs (--no-pack: off)


def packed(torch, dr):
    """dr with its fragment-major weight copy bound (bit-identical results;
    faster loads on the LDS-tiled GEMMs of batches, prefill and training)."""
    if PACK and dr.shape.dtype == "bf16":
        dr.pack_weights(torch.empty(dr.packed_weights_size(), dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
    return dr


def device_weights(torch, shape, seed: int) -> dict:
    """Seeded random-init weights generated on the device (same distributions
    as configs.make_weights: matrices N(0, 0.02^2), gains 1 + N(0, 0.02^2))."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = torch.bfloat16

    def mat(r, c):
        return (torch.randn((r, c), generator=g, device="cuda") * 0.02).to(bf)

    def gain():
        return (1.0 + 0.02 * torch.randn((shape.hidden,), generator=g, device="cuda")).to(bf)

    H = shape.hidden
    w = {"fc": mat(H, shape.n_feat * H), "fc_norm": gain(), "final_norm": gain(),
         "embed": mat(shape.vocab, H), "lm_head": mat(shape.vocab, H), "layers": []}
    for _ in range(shape.n_layers):
        w["layers"].append({"attn_norm": gain(), "wq": mat(shape.q_dim, H),
                            "wk": mat(shape.kv_dim, H), "wv": mat(shape.kv_dim, H),
                            "wo": mat(H, shape.q_dim), "ffn_norm": gain(),
                            "wg": mat(shape.ffn, H), "wu": mat(shape.ffn, H),
                            "wd": mat(H, shape.ffn)})
    return w


def fill_cache(torch, cache, lens, seed: int, std: float = 1.28) -> None:
    """Context K/V drawn on the device (seeded), committed lengths set."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for t in cache.k + cache.v:
        t.copy_(torch.randn(t.shape, generator=g, device="cuda") * std)
    cache.seq_len[:] = np.asarray(lens, dtype=np.int32)


def graph_vs_eager(torch, dr, cache, anchor, draft, ws, reps: int) -> dict:
    """The per-block launch sequence (one draft_block call) eager and as a
    replayed HIP graph, same inputs."""
    dr.set_timing([])
    eager = event_time_ms(torch, lambda: dr.draft_block(cache, BLOCK, anchor, draft, ws), reps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            dr.draft_block(cache, BLOCK, anchor, draft, ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dr.draft_block(cache, BLOCK, anchor, draft, ws)
    graph = event_time_ms(torch, g.replay, reps)
    del g
    return {"draft_block_eager_us": round(eager * 1e3, 2),
            "draft_block_graph_us": round(graph * 1e3, 2),
            "graph_blocks_per_s": round(1e3 / graph, 2)}


def workload_batch16(torch, L, configs, synth, dr, shape, reps: int) -> dict:
    """Batch 16, ragged contexts 512..8192 (M = 256 block rows)."""
    wl = configs.qwen3_8b_b16_ragged()
    lens = list(wl.ctx)
    cache = L.KVCache(shape, [n + 64 for n in lens])
    fill_cache(torch, cache, lens, 3001)
    anchors = torch.from_numpy(configs.make_anchors(shape, wl.wid, wl.batch)).cuda()
    draft = torch.empty((wl.batch, BLOCK - 1), dtype=torch.int32, device="cuda")
    ws = dr.workspace(wl.batch, BLOCK, 1)
    fn = lambda: dr.draft_block(cache, BLOCK, anchors, draft, ws)
    ms = event_time_ms(torch, fn, reps)
    M = wl.batch * BLOCK
    kern = section_times(torch, dr, fn, layer_sections(shape.n_layers), max(3, reps // 4))
    g = torch.Generator(device="cuda")
    g.manual_seed(3002)
    logits = torch.randn((wl.batch, BLOCK, shape.vocab), generator=g, device="cuda").to(torch.bfloat16)
    acc = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
    bon = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
    vws = torch.empty(L.verify_workspace_size(wl.batch, BLOCK, shape.vocab), dtype=torch.uint8,
                      device="cuda")
    v_ms = event_time_ms(torch, lambda: L.verify_greedy(logits, draft, acc, bon, vws), reps)
    v_bytes = wl.batch * BLOCK * shape.vocab * 2
    # sampling at a temperature: Gumbel-max drafts from the drafter's fp32
    # logits, then speculative-sampling verification against the target's
    z = torch.empty((M, shape.vocab), dtype=torch.float32, device="cuda")
    dr.draft_block(cache, BLOCK, anchors, draft, ws, dbg_logits=z)
    z3 = z.reshape(wl.batch, BLOCK, shape.vocab)
    uni = torch.rand((wl.batch, BLOCK - 1, shape.vocab), generator=g, device="cuda").clamp_(1e-12, 1 - 1e-7)
    r = torch.rand((wl.batch, BLOCK - 1), generator=g, device="cuda")
    u = torch.rand((wl.batch,), generator=g, device="cuda")
    sws = torch.empty(L.stochastic_workspace_size(wl.batch, BLOCK, shape.vocab), dtype=torch.uint8,
                      device="cuda")
    nxt = torch.empty(wl.batch, dtype=torch.int32, device="cuda")
    s_ms = event_time_ms(torch, lambda: L.sample_drafts(z3, 0.8, uni, draft, sws), reps)
    vs_ms = event_time_ms(torch, lambda: L.verify_stochastic(logits, z3, draft, 0.8, r, u, acc, nxt,
                                                             sws), reps)
    s_bytes = 2 * wl.batch * (BLOCK - 1) * shape.vocab * 4                    # logits + uniforms
    vs_bytes = wl.batch * BLOCK * shape.vocab * (2 + 4)                       # target bf16 + drafter fp32
    stochastic = {"temperature": 0.8,
                  "sample_drafts": {"avg_us": round(s_ms * 1e3, 2), "bytes": s_bytes,
                                    "hbm_frac": round(s_bytes / (s_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
                  "verify_stochastic": {"avg_us": round(vs_ms * 1e3, 2), "bytes": vs_bytes,
                                        "hbm_frac": round(vs_bytes / (vs_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                        "mean_accept": round(float(acc.float().mean().item()), 3)}}
    out = {"workload": wl.name, "ctx_sum": int(sum(lens)), "draft_block_ms": round(ms, 4),
           "blocks_per_s": round(wl.batch / (ms * 1e-3), 1),
           "kernels": kernel_report(shape, kern, M, sum(lens) + wl.batch * BLOCK),
           "verify": {"avg_us": round(v_ms * 1e3, 2), "bytes": v_bytes,
                      "hbm_frac": round(v_bytes / (v_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
           "stochastic": stochastic}
    del cache
    return out


def workload_training(torch, L, configs, dr, shape, reps: int) -> dict:
    """Training layout: 4 sequences of context 2048 sharing nothing, 16 blocks
    of 16 slots each at sampled anchors (64 blocks, 1024 block rows); one
    dflash_train_forward call = the forward of every block and the weighted
    cross-entropy of its 15 draft slots (gamma = 4)."""
    lens, per_seq, B, gamma = [CTX] * 4, 16, BLOCK, 4.0
    cache = L.KVCache(shape, [n + 64 for n in lens])
    fill_cache(torch, cache, lens, 5001)
    tokens, bseq, apos = configs.make_training_layout(shape, 5001, lens, per_seq, B)
    n = len(bseq)
    anchor_ids = torch.tensor([int(tokens[s][a]) for s, a in zip(bseq, apos)], dtype=torch.int32,
                              device="cuda")
    labels = torch.from_numpy(np.stack([tokens[s][a + 1:a + B] for s, a in zip(bseq, apos)])
                              .astype(np.int32)).cuda()
    ws = dr.workspace(n, B, 1)
    slot = torch.empty((n, B - 1), dtype=torch.float32, device="cuda")
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    fn = lambda: dr.train_forward(cache, B, bseq, apos, anchor_ids, labels, gamma, slot, loss, ws)
    ms = event_time_ms(torch, fn, reps)
    kern = section_times(torch, dr, fn, layer_sections(shape.n_layers), max(3, reps // 4))
    M, H, F, V = n * B, shape.hidden, shape.ffn, shape.vocab
    qd, kvd = shape.q_dim, shape.kv_dim
    flops = {"qkv": 2.0 * M * (qd + 2 * kvd) * H, "o_proj": 2.0 * M * H * qd,
             "gate_up": 2.0 * M * 2 * F * H, "down": 2.0 * M * H * F, "lm_gemm": 2.0 * M * V * H}
    kernels = {}
    for k, v in kern.items():
        e = {"avg_us": round(v * 1e3, 2)}
        if k in flops:
            tf = flops[k] / (v * 1e-3) / 1e12
            e.update({"TFLOP/s": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)})
        kernels[k] = e
    out = {"workload": "qwen3-8b-shaped training layout: 4 x ctx 2048, 16 blocks/seq of 16 slots",
           "blocks": n, "block_rows": M, "train_forward_ms": round(ms, 4),
           "blocks_per_s": round(n / (ms * 1e-3), 1),
           "scored_tokens_per_s": round(n * (B - 1) / (ms * 1e-3), 1),
           "loss": round(float(loss.item()), 5), "kernels": kernels}
    del cache
    return out


def workload_long(torch, L, configs, dr, shape, repeats: int = 3) -> dict:
    """Batch 1: one 32768-token prefill (fuse + inject), then 256 steps that
    each append n ~ U{1..16} fresh feature rows and draft a 16-slot block."""
    wl = configs.qwen3_8b_long_incremental()
    from block_diffusion_drafter_concat_amd import synth
    T, steps, cap = wl.ctx[0], wl.extra["steps"], wl.extra["capacity"]
    H = shape.hidden
    g = torch.Generator(device="cuda")
    g.manual_seed(4001)
    feats = [torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
             for _ in range(shape.n_feat)]
    ctx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    cache = L.KVCache(shape, [cap])
    ws = dr.workspace(1, BLOCK, T)
    sec = section_times(torch, dr, lambda: (dr.fuse_context(feats, ctx, ws),
                                            dr.inject_kv(ctx, [T], cache, ws, pos_start=[0])),
                        [("fuse_gemm", -1), ("inject", -1)], 2)
    pre = {}
    for name, key, fl in (("fusion_gemm", "fuse_gemm", 2.0 * T * shape.n_feat * H * H),
                          ("injection_gemm", "inject", 2.0 * T * H * shape.n_layers * 2 * shape.kv_dim)):
        tf = fl / (sec[key] * 1e-3) / 1e12
        pre[name] = {"rows": T, "avg_us": round(sec[key] * 1e3, 1), "TFLOP/s": round(tf, 1),
                     "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    del feats
    n_new = synth.integers((steps,), 1, 16, wl.wid, synth.STREAM_INDICES, "n_new")
    pool = [torch.randn((steps * BLOCK, H), generator=g, device="cuda").to(torch.bfloat16)
            for _ in range(shape.n_feat)]
    ctx_new = torch.empty((BLOCK, H), dtype=torch.bfloat16, device="cuda")
    anchor = torch.from_numpy(configs.make_anchors(shape, wl.wid, 1)).cuda()
    draft = torch.empty((1, BLOCK - 1), dtype=torch.int32, device="cuda")

    def loop():
        for i in range(steps):
            n = int(n_new[i])
            dr.fuse_context([p[i * BLOCK:i * BLOCK + n] for p in pool], ctx_new, ws)
            dr.inject_kv(ctx_new, [n], cache, ws)
            dr.draft_block(cache, BLOCK, anchor, draft, ws)

    times = []
    for _ in range(repeats):
        cache.seq_len[:] = T          # restore the post-prefill snapshot
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        loop()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    end_len = int(cache.seq_len[0])
    # per-kernel figures at the end of the loop (context ~ end_len)
    kern = section_times(torch, dr, lambda: dr.draft_block(cache, BLOCK, anchor, draft, ws),
                         layer_sections(shape.n_layers), 4)
    out = {"workload": wl.name, "prefill": pre, "loop_ms": round(float(np.median(times)), 3),
           "loop_ms_all": [round(t, 3) for t in times],
           "mean_step_ms": round(float(np.median(times)) / steps, 4),
           "ctx_after_loop": end_len,
           "kernels_at_end": kernel_report(shape, kern, BLOCK, end_len + BLOCK)}
    del cache, pool
    return out


def workload_resident(torch, L, configs, dr, shape, steps: int = 64) -> dict:
    """Batch 1, ctx 2048, B 16: the verify -> append -> draft loop three ways.
    host_sync: verify, read the accepted count on the host, fuse and inject
    that many rows, draft (one device-to-host sync per step); resident: one
    dflash_step_resident per step, no host read; graph: that step captured
    once in a HIP graph and replayed.  Target logits and features are fixed
    random tensors, so most drafts are rejected (one appended row per step)."""
    CTX, B, H, V = 2048, BLOCK, shape.hidden, shape.vocab
    g = torch.Generator(device="cuda")
    g.manual_seed(7001)
    feats = [torch.randn((CTX, H), generator=g, device="cuda").to(torch.bfloat16)
             for _ in range(shape.n_feat)]
    ctx = torch.empty((CTX, H), dtype=torch.bfloat16, device="cuda")
    len_max = CTX + (steps + 1) * B
    cache = L.KVCache(shape, [len_max + B])
    ws = dr.workspace(1, B, CTX)
    dr.fuse_context(feats, ctx, ws)
    dr.inject_kv(ctx, [CTX], cache, ws, pos_start=[0])
    del feats, ctx
    blk = [torch.randn((B, H), generator=g, device="cuda").to(torch.bfloat16)
           for _ in range(shape.n_feat)]
    logits = (torch.randn((1, B, V), generator=g, device="cuda") * 3).to(torch.bfloat16)
    ctx_new = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
    anchor0 = torch.from_numpy(configs.make_anchors(shape, 7001, 1)).cuda()
    anchor = anchor0.clone()
    draft = torch.empty((1, B - 1), dtype=torch.int32, device="cuda")
    accept = torch.zeros(1, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dev_len = torch.full((1,), CTX, dtype=torch.int32, device="cuda")
    vws = torch.empty(L.verify_workspace_size(1, B, V), dtype=torch.uint8, device="cuda")

    def reset():
        cache.seq_len[:] = CTX
        dev_len.fill_(CTX)
        anchor.copy_(anchor0)
        status.zero_()
        dr.draft_block(cache, B, anchor, draft, ws)
        torch.cuda.synchronize()

    def host_step():
        L.verify_greedy(logits, draft, accept, anchor, vws)
        n = int(accept.item()) + 1                   # device -> host
        dr.fuse_context([f[:n] for f in blk], ctx_new, ws)
        dr.inject_kv(ctx_new, [n], cache, ws)
        dr.draft_block(cache, B, anchor, draft, ws)

    def resident_step():
        dr.step_resident(cache, B, dev_len, len_max, logits, blk, draft, anchor, accept, status,
                         ws)

    def timed(fn):
        reset()
        fn()                                          # one untimed step
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    out = {"workload": "qwen3-8b-shaped, batch 1, ctx 2048, B16: verify + append + draft loop",
           "steps": steps}
    out["host_sync_ms_per_step"] = round(timed(host_step), 4)
    host_len = int(cache.seq_len[0])
    out["resident_ms_per_step"] = round(timed(resident_step), 4)
    res_len = int(dev_len.item())
    reset()
    resident_step()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        resident_step()
    torch.cuda.synchronize()

    def replay():
        gr.replay()
    out["graph_ms_per_step"] = round(timed(replay), 4)
    out["ctx_after"] = {"host_sync": host_len, "resident": res_len, "graph": int(dev_len.item())}
    out["status"] = int(status.item())
    del cache, gr
    return out


def workload_27b(torch, L, configs, reps: int) -> dict:
    """27B-target-shaped drafter (H 5120, 40/8 heads, FFN 17408), batch 8,
    context 4096 each, blocks of 8 and 16 slots."""
    shape = configs.TARGET_27B_LIKE
    w = device_weights(torch, shape, 5001)
    dr = packed(torch, L.Drafter(shape, w))
    wl = configs.target27b_b8()
    lens = list(wl.ctx)
    cache = L.KVCache(shape, [n + 64 for n in lens])
    fill_cache(torch, cache, lens, 5002)
    anchors = torch.from_numpy(configs.make_anchors(shape, wl.wid, wl.batch)).cuda()
    out = {"workload": "27b-target-shaped 5-layer bf16, batch 8, ctx 4096"}
    for B in (8, 16):
        draft = torch.empty((wl.batch, B - 1), dtype=torch.int32, device="cuda")
        ws = dr.workspace(wl.batch, B, 1)
        fn = lambda: dr.draft_block(cache, B, anchors, draft, ws)
        ms = event_time_ms(torch, fn, reps)
        kern = section_times(torch, dr, fn, layer_sections(shape.n_layers), max(3, reps // 4))
        out[f"B{B}"] = {"draft_block_ms": round(ms, 4),
                        "blocks_per_s": round(wl.batch / (ms * 1e-3), 1),
                        "kernels": kernel_report(shape, kern, wl.batch * B,
                                                 sum(lens) + wl.batch * B)}
    dr.close()
    del cache, w
    return out


def draft_latency(torch, L, configs, shape, w, reps: int = 20) -> dict:
    """Latency of one block pass (5 layers, 16 slots: 15 drafts) against an
    autoregressive stand-in of the same width: 1 layer, 8 sequential steps,
    each a 2-slot pass (anchor + one draft) whose draft anchors the next
    step, the anchor's K/V row kept by advancing the committed length (the
    autoregressive cache append).  Same kernels, same LM head; ctx 2048."""
    one = configs.scaled(shape, n_layers=1)
    w1 = dict(w)
    w1["layers"] = w["layers"][:1]
    dr5, dr1 = L.Drafter(shape, w), L.Drafter(one, w1)
    lens = [CTX]
    c5 = L.KVCache(shape, [CTX + 64])
    c1 = L.KVCache(one, [CTX + 64])
    fill_cache(torch, c5, lens, 6001)
    fill_cache(torch, c1, lens, 6002)
    anchor = torch.zeros(1, dtype=torch.int32, device="cuda")
    d15 = torch.empty((1, BLOCK - 1), dtype=torch.int32, device="cuda")
    d1 = torch.empty((1, 1), dtype=torch.int32, device="cuda")
    ws5, ws1 = dr5.workspace(1, BLOCK, 1), dr1.workspace(1, 2, 1)
    block_ms = event_time_ms(torch, lambda: dr5.draft_block(c5, BLOCK, anchor, d15, ws5), reps)
    ar_steps = 8

    def ar_loop():
        c1.seq_len[0] = CTX
        a = anchor
        for _ in range(ar_steps):
            dr1.draft_block(c1, 2, a, d1, ws1)
            a = d1.view(1)
            c1.seq_len[0] += 1
    ar_ms = event_time_ms(torch, ar_loop, reps)
    dr5.close()
    dr1.close()
    return {"block_pass": {"layers": shape.n_layers, "slots": BLOCK, "drafts": BLOCK - 1,
                           "ms": round(block_ms, 4)},
            "autoregressive": {"layers": 1, "steps": ar_steps, "drafts": ar_steps,
                               "ms": round(ar_ms, 4)},
            "block_drafts_per_ms": round((BLOCK - 1) / block_ms, 2),
            "ar_drafts_per_ms": round(ar_steps / ar_ms, 2),
            "ctx": CTX}


def step_bytes(shape, n_new: int) -> dict:
    """Algorithmic HBM bytes of one step (each tensor read or written once)."""
    H, V, L = shape.hidden, shape.vocab, shape.n_layers
    s = 2
    layer_w = shape.layer_params() * s
    lm = V * H * s
    kv = (CTX + BLOCK) * shape.kv_dim * 2 * s * L
    fuse = shape.n_feat * H * H * s + shape.n_feat * n_new * H * s + n_new * H * s
    inject = L * 2 * shape.kv_dim * H * s + n_new * H * s + L * 2 * n_new * shape.kv_dim * s
    verify = BLOCK * V * s
    return {"layers": L * layer_w, "lm_head": lm, "kv": kv, "fuse": fuse, "inject": inject,
            "verify": verify, "embed": BLOCK * H * s}


def main():
    global PACK
    args = parse()
    PACK = not args.no_pack
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_diffusion_drafter_concat_amd import configs, synth
    from block_diffusion_drafter_concat_amd import lib as L

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    L.load()
    if args.kernel_probe:
        kernel_probe(torch, L, configs)
        return
    shape = configs.QWEN3_8B_LIKE
    wid = 2
    K, W = args.steps, args.warmup

    t0 = time.time()
    w = configs.make_weights(shape, wid)
    dr = packed(torch, L.Drafter(shape, w))
    log(f"weights ready in {time.time() - t0:.1f}s")

    # prefill (untimed): fuse and inject the 2048-token context
    feats = configs.make_features(shape, wid, CTX)
    cache = L.KVCache(shape, [CTX + 64])
    ws = dr.workspace(BATCH, BLOCK, CTX)
    ctx_all = torch.empty((CTX, shape.hidden), dtype=torch.bfloat16, device="cuda")
    feats_dev = [L.to_device(f, "bf16") for f in feats]
    dr.fuse_context(feats_dev, ctx_all, ws)
    dr.inject_kv(ctx_all, [CTX], cache, ws)
    prefill = time_prefill(torch, dr, shape, feats_dev, ctx_all, cache, ws)
    del ctx_all, feats_dev

    # per-step inputs
    n_steps = W + K
    tau = synth.geometric_capped(n_steps, 0.15, BLOCK, wid, synth.STREAM_INDICES, "bench_tau")
    new_feats = [L.to_device(f, "bf16") for f in
                 configs.make_features(shape, wid, BLOCK, name="bench_new")]
    rand_drafts = synth.integers((BATCH, BLOCK - 1), 0, shape.vocab - 2, wid,
                                 synth.STREAM_LOGITS, "bench_drafts")
    logits_np = synth.plant_target_logits(
        synth.values((BATCH, BLOCK, shape.vocab), "bf16", wid, synth.STREAM_LOGITS, "bench_lg"),
        rand_drafts, np.array([int(tau[0]) - 1]), "bf16", workload=wid)
    logits = L.to_device(logits_np.reshape(BATCH * BLOCK, -1), "bf16").reshape(
        BATCH, BLOCK, shape.vocab)
    ctx_new = torch.empty((BLOCK, shape.hidden), dtype=torch.bfloat16, device="cuda")
    anchor = torch.from_numpy(configs.make_anchors(shape, wid, BATCH)).cuda()
    draft = torch.empty((BATCH, BLOCK - 1), dtype=torch.int32, device="cuda")
    accept = torch.empty(BATCH, dtype=torch.int32, device="cuda")
    vws = torch.empty(L.verify_workspace_size(BATCH, BLOCK, shape.vocab), dtype=torch.uint8,
                      device="cuda")

    def step(i, verify_events=None):
        n = int(tau[i])
        dr.fuse_context([f[:n] for f in new_feats], ctx_new, ws)
        dr.inject_kv(ctx_new, [n], cache, ws, pos_start=[CTX - n])
        dr.draft_block(cache, BLOCK, anchor, draft, ws)
        if verify_events:
            verify_events[0].record()
        L.verify_greedy(logits, draft, accept, anchor, vws)   # bonus -> next anchor
        if verify_events:
            verify_events[1].record()

    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps, eager launches on the current stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    for i in range(W, W + K):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = ev0.elapsed_time(ev1)
    ms_per_step = gpu_ms / K
    blocks_per_s = BATCH * K / (gpu_ms / 1e3)
    log(f"timed: {K} steps, {ms_per_step:.3f} ms/step (wall {wall * 1e3 / K:.3f} ms/step)")


    # ---- kernel-timing pass: HIP events around each section, same steps
    if args.no_timing_pass:
        print(json.dumps({"value": round(blocks_per_s, 2), "ms_per_step": ms_per_step}))
        return

    # ---- spread: 5 more repeats of the same K steps, timed the same way
    rep_ms = []
    for r in range(5):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(W, W + K):
            step(i)
        b.record()
        torch.cuda.synchronize()
        rep_ms.append(a.elapsed_time(b) / K)
    repeats = {"repeats": 5, "steps_each": K,
               "ms_per_step_median": round(float(np.median(rep_ms)), 4),
               "ms_per_step_p10": round(float(np.percentile(rep_ms, 10)), 4),
               "ms_per_step_p90": round(float(np.percentile(rep_ms, 90)), 4)}
    log(f"repeats: {repeats}")

    sections = [("lm_head", -1), ("lm_gemm", -1), ("fuse_gemm", -1), ("inject", -1),
                ("embed", -1), ("final_norm", -1)]
    for l in range(shape.n_layers):
        sections += [("qkv", l), ("attention", l), ("o_proj", l), ("gate_up", l), ("down", l)]
    per_step = []
    for i in range(K):
        pts = []
        for s, l in sections:
            a = TimingEvent(torch)
            b = TimingEvent(torch)
            a.record()
            b.record()
            pts.append((s, l, a, b))
        ve = (TimingEvent(torch), TimingEvent(torch))
        per_step.append((pts, ve))
    torch.cuda.synchronize()
    for i in range(K):
        pts, ve = per_step[i]
        dr.set_timing(pts)
        step(W + i, verify_events=ve)
    dr.set_timing([])
    torch.cuda.synchronize()
    sec_ms = {}
    for pts, ve in per_step:
        for s, l, a, b in pts:
            key = s if l < 0 else s
            sec_ms.setdefault(key, []).append(a.elapsed_time(b))
        sec_ms.setdefault("verify", []).append(ve[0].elapsed_time(ve[1]))
    # per-layer sections: mean per launch (average over layers and steps)
    kern = {k: float(np.mean(v)) for k, v in sec_ms.items()}
    # the dominant kernel: the LM-head GEMM launch alone (events around it only;
    # the argmax fold that follows is a separate small kernel)
    lm_ms = kern["lm_gemm"]
    M = BATCH * BLOCK
    lm_bytes = shape.vocab * shape.hidden * 2 + M * shape.hidden * 2
    lm_gbs = lm_bytes / (lm_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": "skinny_gemm_kernel<EpiLMHead> (LM-head GEMM, argmax partials in its epilogue)",
                "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(lm_gbs / HBM_PEAK_GBS, 4), "traffic": lm_head_traffic(),
                "bytes_per_launch": lm_bytes, "avg_launch_us": round(lm_ms * 1e3, 2)}

    # per-kernel HBM fractions of the weight-streaming GEMMs (per launch)
    H, F, qd, kvd = shape.hidden, shape.ffn, shape.q_dim, shape.kv_dim
    kbytes = {"qkv": (qd + 2 * kvd) * H * 2, "o_proj": H * qd * 2, "gate_up": 2 * F * H * 2,
              "down": H * F * 2, "lm_head": lm_bytes, "lm_gemm": lm_bytes,
              "attention": (CTX + BLOCK) * kvd * 2 * 2,
              "fuse_gemm": shape.n_feat * H * H * 2, "inject": shape.n_layers * 2 * kvd * H * 2,
              "verify": BATCH * BLOCK * shape.vocab * 2}
    kernels = {}
    for k, ms in kern.items():
        ent = {"avg_us": round(ms * 1e3, 2)}
        if k in kbytes:
            gbs = kbytes[k] / (ms * 1e-3) / 1e9
            ent.update({"bytes": kbytes[k], "GB/s": round(gbs, 1),
                        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        kernels[k] = ent

    mean_n = float(np.mean(tau[W:W + K]))
    sb = step_bytes(shape, int(round(mean_n)))
    tot = sum(sb.values())
    step_roof = {"bytes_per_step": tot, "roofline_ms": tot / (HBM_PEAK_GBS * 1e9) * 1e3,
                 "frac": round(tot / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3), 4)}

    # ---- the per-block launch sequence as a HIP graph, then other workloads
    graph = graph_vs_eager(torch, dr, cache, anchor, draft, ws, K)
    log(f"graph: {graph}")
    latency = draft_latency(torch, L, configs, shape, dr.w)   # device weights, no copy
    log(f"draft latency: {latency}")
    workloads = None
    if not args.no_workloads:
        workloads = {}
        t1 = time.time()
        workloads["batch16_ragged"] = workload_batch16(torch, L, configs, synth, dr, shape, 20)
        log(f"batch-16 ragged done ({time.time() - t1:.1f}s)")
        t1 = time.time()
        workloads["long_ctx_incremental"] = workload_long(torch, L, configs, dr, shape)
        log(f"long-context loop done ({time.time() - t1:.1f}s)")
        t1 = time.time()
        workloads["training_layout"] = workload_training(torch, L, configs, dr, shape, 10)
        log(f"training layout done ({time.time() - t1:.1f}s)")
        t1 = time.time()
        workloads["resident_loop"] = workload_resident(torch, L, configs, dr, shape)
        log(f"resident loop done ({time.time() - t1:.1f}s): {workloads['resident_loop']}")
        dr.close()
        del dr
        torch.cuda.empty_cache()
        t1 = time.time()
        workloads["target27b_batch8"] = workload_27b(torch, L, configs, 20)
        log(f"27b-shaped done ({time.time() - t1:.1f}s)")

    # ---- CPU oracle on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shape, w, feats, new_feats_np=configs.make_features(
            shape, wid, BLOCK, name="bench_new"), tau=tau, logits=logits_np,
            budget=args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(blocks_per_s, 2), "unit": "blocks/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b-shaped drafter, batch 1, ctx 2048, block 16",
                   "layers": shape.n_layers, "hidden": shape.hidden, "heads": "32q/8kv x 128",
                   "ffn": shape.ffn, "vocab": shape.vocab, "batch": BATCH, "ctx": CTX,
                   "block": BLOCK, "mean_new_tokens_per_step": round(mean_n, 2),
                   "launch": "eager", "packed_weights": PACK},
        "tokens_per_s": round(blocks_per_s * BLOCK, 1),
        "draft_tokens_per_s": round(blocks_per_s * (BLOCK - 1), 1),
        "roofline": roofline,
        "step_roofline": step_roof,
        "spread": repeats,
        "kernels": kernels,
        "prefill_mfma": prefill,
        "graph": graph,
        "draft_latency": latency,
        "workloads": workloads,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (as lscpu reports it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(shape, w, feats, new_feats_np, tau, logits, budget: float) -> dict:
    """Time the oracle's step (same workload) on the host, untuned."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(p.get("num_threads", 1)) for p in threadpool_info()
                     if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    t0 = time.perf_counter()
    cache = O.prefill(w, shape, [feats])[0]
    log(f"oracle prefill {time.perf_counter() - t0:.1f}s")
    anchors = np.array([7], dtype=np.int32)
    done, t_start = 0, time.perf_counter()
    while True:
        n = int(tau[done % len(tau)])
        c = [(k[:CTX - n], v[:CTX - n]) for k, v in cache]
        c = O.append_context(c, w, shape, [f[:n] for f in new_feats_np])
        res = O.draft_block(w, shape, [c], anchors, BLOCK)
        acc, bonus = O.verify_greedy(logits, res["draft_ids"])
        anchors = bonus
        done += 1
        el = time.perf_counter() - t_start
        if el >= budget or done >= 50:
            break
    return {"value": round(done / el, 4), "unit": "blocks/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{done} oracle steps of the same workload (fuse+inject of the step's new "
                      f"rows, one 16-slot block through 5 layers at ctx 2048, LM-head argmax, "
                      f"verify), float64 numpy, {el:.1f}s"}


if __name__ == "__main__":
    main()
