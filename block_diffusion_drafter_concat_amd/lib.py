"""ctypes binding of libdflash.so (include/dflash.h): argument marshalling only.

Every step of the drafter's work runs in the HIP library; this module turns
torch device tensors into pointers and host arrays into C arrays.  It loads
the library lazily and raises ``RuntimeError`` if it is missing -- there is no
fallback.  PyTorch supplies device memory and the stream.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_MAX_BATCH = 64
DFLASH_MAX_BLOCK = 16
DFLASH_MAX_LAYERS = 16
DFLASH_MAX_FEAT = 6

OK, ERR_INVALID_ARG, ERR_CAPACITY, ERR_UNSUPPORTED, ERR_HIP, ERR_SCRATCH = range(6)
NOALLOC_SCRATCH_BYTES = 64 << 20
F32, BF16 = 0, 1

EXPORTS = ("dflash_target_layer_ids", "dflash_create", "dflash_destroy",
           "dflash_workspace_size", "dflash_fuse_context", "dflash_inject_kv",
           "dflash_draft_block", "dflash_verify_greedy", "dflash_verify_workspace_size",
           "dflash_train_forward", "dflash_set_timing", "dflash_status_string",
           "dflash_stochastic_workspace_size", "dflash_sample_drafts",
           "dflash_verify_stochastic", "dflash_step_resident", "dflash_debug_bf16_round",
           "dflash_draft_block_noalloc", "dflash_packed_weights_size", "dflash_pack_weights")

# dflash_section
SECTIONS = {"fuse_gemm": 1, "fuse_norm": 2, "inject": 3, "embed": 4, "attn_norm": 5, "qkv": 6,
            "attention": 7, "o_proj": 8, "ffn_norm": 9, "gate_up": 10, "down": 11,
            "final_norm": 12, "lm_head": 13, "lm_gemm": 14}


class DflashError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


class Config(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("ffn", C.c_int32),
                ("vocab", C.c_int32), ("n_feat_layers", C.c_int32), ("mask_token_id", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float), ("dtype", C.c_int)]


class LayerWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "wg", "wu", "wd")]


class Weights(C.Structure):
    _fields_ = [("fc", C.c_void_p), ("fc_norm", C.c_void_p),
                ("layers", C.POINTER(LayerWeights)), ("final_norm", C.c_void_p),
                ("embed", C.c_void_p), ("lm_head", C.c_void_p)]


class KV(C.Structure):
    _fields_ = [("k", C.POINTER(C.c_void_p)), ("v", C.POINTER(C.c_void_p)),
                ("batch", C.c_int32), ("cap_total", C.c_int64),
                ("seq_off", C.POINTER(C.c_int64)), ("seq_cap", C.POINTER(C.c_int32)),
                ("seq_len", C.POINTER(C.c_int32))]


class TimingPoint(C.Structure):
    _fields_ = [("section", C.c_int32), ("layer", C.c_int32), ("ev_start", C.c_void_p),
                ("ev_stop", C.c_void_p)]


_lib = None


def load() -> C.CDLL:
    """Load libdflash.so (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_diffusion_drafter_concat_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    pi32 = C.POINTER(C.c_int32)
    lib.dflash_target_layer_ids.argtypes = [i32, i32, pi32]
    lib.dflash_target_layer_ids.restype = i32
    lib.dflash_create.argtypes = [C.POINTER(Config), C.POINTER(Weights), C.POINTER(vp)]
    lib.dflash_create.restype = C.c_int
    lib.dflash_destroy.argtypes = [vp]
    lib.dflash_destroy.restype = C.c_int
    lib.dflash_workspace_size.argtypes = [vp, i32, i32, i64, C.POINTER(C.c_size_t)]
    lib.dflash_workspace_size.restype = C.c_int
    lib.dflash_packed_weights_size.argtypes = [vp, C.POINTER(C.c_size_t)]
    lib.dflash_packed_weights_size.restype = C.c_int
    lib.dflash_pack_weights.argtypes = [vp, vp, C.c_size_t, vp]
    lib.dflash_pack_weights.restype = C.c_int
    lib.dflash_fuse_context.argtypes = [vp, C.POINTER(vp), i64, vp, vp, vp]
    lib.dflash_fuse_context.restype = C.c_int
    lib.dflash_inject_kv.argtypes = [vp, vp, pi32, pi32, C.POINTER(KV), vp, vp]
    lib.dflash_inject_kv.restype = C.c_int
    lib.dflash_draft_block.argtypes = [vp, C.POINTER(KV), i32, vp, vp, vp, vp, vp, vp]
    lib.dflash_draft_block.restype = C.c_int
    lib.dflash_draft_block_noalloc.argtypes = [vp, C.POINTER(KV), i32, vp, vp, vp, vp, vp]
    lib.dflash_draft_block_noalloc.restype = C.c_int
    lib.dflash_verify_greedy.argtypes = [vp, C.c_int, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.dflash_verify_greedy.restype = C.c_int
    lib.dflash_verify_workspace_size.argtypes = [i32, i32, i32]
    lib.dflash_verify_workspace_size.restype = C.c_size_t
    lib.dflash_train_forward.argtypes = [vp, C.POINTER(KV), i32, i32, pi32, pi32, vp, vp,
                                         C.c_float, vp, vp, vp, vp, vp]
    lib.dflash_train_forward.restype = C.c_int
    lib.dflash_step_resident.argtypes = [vp, C.POINTER(KV), i32, vp, i32, vp, C.c_int,
                                         C.POINTER(vp), vp, vp, vp, vp, vp, vp]
    lib.dflash_step_resident.restype = C.c_int
    lib.dflash_stochastic_workspace_size.argtypes = [i32, i32, i32]
    lib.dflash_stochastic_workspace_size.restype = C.c_size_t
    lib.dflash_sample_drafts.argtypes = [vp, i32, i32, i32, C.c_float, vp, vp, vp, vp]
    lib.dflash_sample_drafts.restype = C.c_int
    lib.dflash_verify_stochastic.argtypes = [vp, C.c_int, vp, vp, i32, i32, i32, C.c_float, vp,
                                             vp, vp, vp, vp, vp]
    lib.dflash_verify_stochastic.restype = C.c_int
    lib.dflash_debug_bf16_round.argtypes = [vp, vp, i64, i32, vp]
    lib.dflash_debug_bf16_round.restype = C.c_int
    lib.dflash_set_timing.argtypes = [vp, C.POINTER(TimingPoint), i32]
    lib.dflash_set_timing.restype = C.c_int
    lib.dflash_status_string.argtypes = [C.c_int]
    lib.dflash_status_string.restype = C.c_char_p
    _lib = lib
    return lib


def status_string(s: int) -> str:
    return load().dflash_status_string(int(s)).decode()


def _check(status: int, what: str) -> None:
    if status != OK:
        raise DflashError(status, what)


def target_layer_ids(n_target_layers: int, n_select: int = 5) -> list:
    out = (C.c_int32 * max(1, n_select))()
    n = load().dflash_target_layer_ids(n_target_layers, n_select, out)
    if n < 0:
        raise DflashError(ERR_INVALID_ARG, "dflash_target_layer_ids")
    return [int(out[i]) for i in range(n)]


# ---------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream(stream=None) -> int | None:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream) or None


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Upload float32 values (bf16-exact for "bf16") as a device tensor."""
    torch = _torch()
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        bits = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def torch_dtype(dtype: str):
    torch = _torch()
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class Drafter:
    """A libdflash handle over device-resident weights (torch tensors).

    ``weights`` is the dict layout of ``configs.make_weights`` holding torch
    device tensors (or numpy arrays, uploaded here).
    """

    def __init__(self, shape, weights: dict, device="cuda"):
        self.shape = shape
        self.lib = load()
        up = (lambda a: a if hasattr(a, "data_ptr") else to_device(a, shape.dtype, device))
        self.w = {k: up(v) for k, v in weights.items() if k != "layers"}
        self.w["layers"] = [{k: up(v) for k, v in lw.items()} for lw in weights["layers"]]
        self.cfg = Config(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads,
                          shape.head_dim, shape.ffn, shape.vocab, shape.n_feat,
                          shape.mask_token_id, shape.rms_eps, shape.rope_theta,
                          BF16 if shape.dtype == "bf16" else F32)
        L = shape.n_layers
        self._layers = (LayerWeights * L)(*[
            LayerWeights(*[_ptr(lw[n]) for n in ("attn_norm", "wq", "wk", "wv", "wo",
                                                 "ffn_norm", "wg", "wu", "wd")])
            for lw in self.w["layers"]])
        self._weights = Weights(_ptr(self.w["fc"]), _ptr(self.w["fc_norm"]), self._layers,
                                _ptr(self.w["final_norm"]), _ptr(self.w["embed"]),
                                _ptr(self.w["lm_head"]))
        h = C.c_void_p()
        _check(self.lib.dflash_create(C.byref(self.cfg), C.byref(self._weights), C.byref(h)),
               "dflash_create")
        self.handle = h
        self._packed = None   # the packed-weight buffer while bound

    def close(self):
        if getattr(self, "handle", None):
            self.lib.dflash_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, max_batch: int, max_block: int, max_tokens: int) -> int:
        n = C.c_size_t()
        _check(self.lib.dflash_workspace_size(self.handle, max_batch, max_block, max_tokens,
                                              C.byref(n)), "dflash_workspace_size")
        return int(n.value)

    def workspace(self, max_batch: int, max_block: int, max_tokens: int, device="cuda"):
        torch = _torch()
        return torch.empty(self.workspace_size(max_batch, max_block, max_tokens),
                           dtype=torch.uint8, device=device)

    def packed_weights_size(self) -> int:
        n = C.c_size_t()
        _check(self.lib.dflash_packed_weights_size(self.handle, C.byref(n)),
               "dflash_packed_weights_size")
        return int(n.value)

    def pack_weights(self, dst=None, stream=None) -> None:
        """Fragment-major copy of the bf16 GEMM weights into dst (a device
        uint8 tensor of at least packed_weights_size() bytes, kept alive by
        this object while bound); None switches back to the row-major weights."""
        if dst is None:
            _check(self.lib.dflash_pack_weights(self.handle, None, 0, _stream(stream)),
                   "dflash_pack_weights")
            self._packed = None
            return
        _check(self.lib.dflash_pack_weights(self.handle, _ptr(dst), dst.numel() * dst.element_size(),
                                            _stream(stream)), "dflash_pack_weights")
        self._packed = dst

    def set_timing(self, points) -> None:
        """points: list of (section name, layer, start event, stop event) with
        torch.cuda.Event objects that have been recorded once (so they exist)."""
        arr = (TimingPoint * max(1, len(points)))(*[
            TimingPoint(SECTIONS[s], int(l), int(a.cuda_event), int(b.cuda_event))
            for s, l, a, b in points])
        _check(self.lib.dflash_set_timing(self.handle, arr, len(points)), "dflash_set_timing")

    # -------------------------------------------------------------- calls
    def fuse_context(self, feats, out, ws, stream=None) -> None:
        n = int(feats[0].shape[0])
        arr = (C.c_void_p * len(feats))(*[_ptr(f) for f in feats])
        _check(self.lib.dflash_fuse_context(self.handle, arr, n, _ptr(out), _ptr(ws),
                                            _stream(stream)), "dflash_fuse_context")

    def inject_kv(self, ctx, n_new, cache: "KVCache", ws, pos_start=None, stream=None) -> None:
        nn = (C.c_int32 * cache.batch)(*[int(v) for v in n_new])
        ps = None if pos_start is None else (C.c_int32 * cache.batch)(*[int(v) for v in pos_start])
        _check(self.lib.dflash_inject_kv(self.handle, _ptr(ctx), ps, nn, C.byref(cache.c),
                                         _ptr(ws), _stream(stream)), "dflash_inject_kv")

    def draft_block(self, cache: "KVCache", block_size: int, anchors, draft_ids, ws,
                    dbg_hidden=None, dbg_logits=None, stream=None) -> None:
        _check(self.lib.dflash_draft_block(self.handle, C.byref(cache.c), block_size,
                                           _ptr(anchors), _ptr(draft_ids), _ptr(dbg_hidden),
                                           _ptr(dbg_logits), _ptr(ws), _stream(stream)),
               "dflash_draft_block")

    def draft_block_noalloc(self, cache: "KVCache", block_size: int, anchors, draft_ids,
                            dbg_hidden=None, dbg_logits=None, stream=None) -> None:
        """draft_block on the library's static per-device scratch (no workspace)."""
        _check(self.lib.dflash_draft_block_noalloc(self.handle, C.byref(cache.c), block_size,
                                                   _ptr(anchors), _ptr(draft_ids),
                                                   _ptr(dbg_hidden), _ptr(dbg_logits),
                                                   _stream(stream)), "dflash_draft_block_noalloc")

    def train_forward(self, cache: "KVCache", block_size: int, block_seq, anchor_pos, anchor_ids,
                      labels, gamma: float, slot_loss, loss, ws, dbg_logits=None,
                      stream=None) -> None:
        """Training-layout forward: block i of sequence block_seq[i] at anchor
        anchor_pos[i] (host int sequences); anchor_ids int32 [n], labels int32
        [n, B-1], slot_loss float32 [n, B-1], loss float32 [1] (device)."""
        bs = np.ascontiguousarray(block_seq, dtype=np.int32)
        ap = np.ascontiguousarray(anchor_pos, dtype=np.int32)
        _check(self.lib.dflash_train_forward(
            self.handle, C.byref(cache.c), len(bs), block_size,
            bs.ctypes.data_as(C.POINTER(C.c_int32)), ap.ctypes.data_as(C.POINTER(C.c_int32)),
            _ptr(anchor_ids), _ptr(labels), float(gamma), _ptr(slot_loss), _ptr(loss),
            _ptr(dbg_logits), _ptr(ws), _stream(stream)), "dflash_train_forward")


    def step_resident(self, cache: "KVCache", block_size: int, dev_len, len_max: int,
                      target_logits, block_feats, draft_ids, anchor_ids, accept, status, ws,
                      stream=None) -> None:
        """Verify, append and draft in one device-resident step.  dev_len int32
        [N], target_logits [N, B, V] (float32 or bfloat16), block_feats: one
        [N * B, H] tensor per fused target layer, draft_ids int32 [N, B-1]
        (read, then overwritten), anchor_ids int32 [N] (overwritten with the
        bonus tokens), accept int32 [N], status int32 [1] (all device)."""
        torch = _torch()
        dt = BF16 if target_logits.dtype == torch.bfloat16 else F32
        arr = (C.c_void_p * len(block_feats))(*[_ptr(f) for f in block_feats])
        _check(self.lib.dflash_step_resident(
            self.handle, C.byref(cache.c), block_size, _ptr(dev_len), int(len_max),
            _ptr(target_logits), dt, arr, _ptr(draft_ids), _ptr(anchor_ids), _ptr(accept),
            _ptr(status), _ptr(ws), _stream(stream)), "dflash_step_resident")


def verify_greedy(target_logits, draft_ids, accept, bonus, ws, stream=None) -> None:
    """target_logits [N, B, V] (float32 or bfloat16 tensor), draft_ids int32 [N, B-1]."""
    torch = _torch()
    N, B, V = (int(s) for s in target_logits.shape)
    dt = BF16 if target_logits.dtype == torch.bfloat16 else F32
    _check(load().dflash_verify_greedy(_ptr(target_logits), dt, _ptr(draft_ids), N, B, V,
                                       _ptr(accept), _ptr(bonus), _ptr(ws), _stream(stream)),
           "dflash_verify_greedy")


def verify_workspace_size(batch: int, block: int, vocab: int) -> int:
    return int(load().dflash_verify_workspace_size(batch, block, vocab))


def stochastic_workspace_size(batch: int, block: int, vocab: int) -> int:
    return int(load().dflash_stochastic_workspace_size(batch, block, vocab))


def sample_drafts(draft_logits, temperature: float, uniforms, draft_ids, ws, stream=None) -> None:
    """draft_logits float32 [N, B, V], uniforms float32 [N, B-1, V], draft_ids int32 [N, B-1]."""
    N, B, V = (int(s) for s in draft_logits.shape)
    _check(load().dflash_sample_drafts(_ptr(draft_logits), N, B, V, float(temperature),
                                       _ptr(uniforms), _ptr(draft_ids), _ptr(ws),
                                       _stream(stream)), "dflash_sample_drafts")


def verify_stochastic(target_logits, draft_logits, draft_ids, temperature: float, r_accept,
                      u_sample, accept, next_token, ws, stream=None) -> None:
    """target_logits [N, B, V] (float32 or bfloat16), draft_logits float32 [N, B, V],
    draft_ids int32 [N, B-1], r_accept float32 [N, B-1], u_sample float32 [N]."""
    torch = _torch()
    N, B, V = (int(s) for s in target_logits.shape)
    dt = BF16 if target_logits.dtype == torch.bfloat16 else F32
    _check(load().dflash_verify_stochastic(_ptr(target_logits), dt, _ptr(draft_logits),
                                           _ptr(draft_ids), N, B, V, float(temperature),
                                           _ptr(r_accept), _ptr(u_sample), _ptr(accept),
                                           _ptr(next_token), _ptr(ws), _stream(stream)),
           "dflash_verify_stochastic")


def debug_bf16_round(inp, out, packed: bool = False, stream=None) -> None:
    """out (int16 / bfloat16 device tensor) = the library's bf16 rounding of
    inp (float32 device tensor), by its scalar or its pair conversion."""
    _check(load().dflash_debug_bf16_round(_ptr(inp), _ptr(out), int(inp.numel()), int(packed),
                                          _stream(stream)), "dflash_debug_bf16_round")


class KVCache:
    """Caller-owned drafter cache: per layer K [Hkv, cap, d] and V^T [Hkv, d, cap].

    Sequence b owns rows [off[b], off[b] + cap[b]) of the position axis; caps
    are rounded up to multiples of 32.  ``seq_len`` is a host int32 array that
    dflash_inject_kv updates.
    """

    def __init__(self, shape, caps, device="cuda", fill=None):
        torch = _torch()
        caps = [int((c + 31) // 32 * 32) for c in caps]
        self.batch = len(caps)
        self.caps = np.array(caps, dtype=np.int32)
        self.offs = np.concatenate([[0], np.cumsum(caps)[:-1]]).astype(np.int64)
        self.cap_total = int(sum(caps))
        self.seq_len = np.zeros(self.batch, dtype=np.int32)
        dt = torch_dtype(shape.dtype)
        mk = torch.zeros if fill == 0 else torch.empty
        self.k = [mk((shape.n_kv_heads, self.cap_total, shape.head_dim), dtype=dt, device=device)
                  for _ in range(shape.n_layers)]
        self.v = [mk((shape.n_kv_heads, shape.head_dim, self.cap_total), dtype=dt, device=device)
                  for _ in range(shape.n_layers)]
        self._k = (C.c_void_p * shape.n_layers)(*[_ptr(t) for t in self.k])
        self._v = (C.c_void_p * shape.n_layers)(*[_ptr(t) for t in self.v])
        self.c = KV(self._k, self._v, self.batch, self.cap_total,
                    self.offs.ctypes.data_as(C.POINTER(C.c_int64)),
                    self.caps.ctypes.data_as(C.POINTER(C.c_int32)),
                    self.seq_len.ctypes.data_as(C.POINTER(C.c_int32)))

    def keys(self, layer: int, b: int):
        """[len, Hkv, d] view of sequence b's committed keys (for tests)."""
        o, n = int(self.offs[b]), int(self.seq_len[b])
        return self.k[layer][:, o:o + n, :].permute(1, 0, 2)

    def values(self, layer: int, b: int):
        """[len, Hkv, d] view of sequence b's committed values (for tests)."""
        o, n = int(self.offs[b]), int(self.seq_len[b])
        return self.v[layer][:, :, o:o + n].permute(2, 0, 1)
