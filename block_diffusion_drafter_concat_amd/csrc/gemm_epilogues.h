// Epilogues of the weight-streaming GEMM.  Each one says which W rows make up
// pair tile `tile` (rows(): the W row this lane streams for sub-tile 0 and 1)
// and what to do with the pair of results (apply(): row m, column i of the
// 16-wide sub-tiles, K-split `split`).  State is per-thread scratch that lives
// across the tiles one workgroup walks; finish() runs once per workgroup.
#pragma once

#include "device_common.h"

namespace dflash {

struct NoState {};

// Float32 partial products, one slab per K-split:
//   out[(split * slab_rows + m) * ldo + n] = sum over this split's K of A[m] . W[n]
// with 32 consecutive W rows per tile.  The consumer sums the slabs in order.
template <typename T>
struct EpiPartialF32 {
  using State = NoState;
  const T* W;
  int K;
  float* out;
  int64_t ldo;
  int64_t slab_rows;   // rows per split slab
  __device__ void init(State&) const {}
  __device__ void rows(int tile, int r16, const T*& w0, const T*& w1) const {
    w0 = W + static_cast<int64_t>(tile * 32 + r16) * K;
    w1 = w0 + static_cast<int64_t>(16) * K;
  }
  __device__ void apply(State&, int, int tile, int split, int m, int i, bool valid, float v0,
                        float v1) const {
    if (!valid) return;
    float* o = out + (split * slab_rows + m) * ldo + tile * 32 + i;
    o[0] = v0;
    o[16] = v1;
  }
  __device__ void finish(State&, int, int, int) const {}
};

// Fused Q/K/V projection as fp32 K-split partials: output column n of the
// stacked [Wq; Wk; Wv] (qd + 2 kvd rows) goes to out[(split * slab_rows + m) *
// ldo + n]; a finishing kernel sums the splits and applies RoPE.  qd and kvd
// are multiples of 32, so a 32-row tile never straddles two matrices.
template <typename T>
struct EpiQKVPartF32 {
  using State = NoState;
  const T* wq;
  const T* wk;
  const T* wv;
  int K, qd, kvd;
  float* out;
  int64_t ldo;
  int64_t slab_rows;
  __device__ void init(State&) const {}
  __device__ void rows(int tile, int r16, const T*& w0, const T*& w1) const {
    const int n = tile * 32;
    const T* base = n < qd ? wq + static_cast<int64_t>(n) * K
                  : n < qd + kvd ? wk + static_cast<int64_t>(n - qd) * K
                                 : wv + static_cast<int64_t>(n - qd - kvd) * K;
    w0 = base + static_cast<int64_t>(r16) * K;
    w1 = w0 + static_cast<int64_t>(16) * K;
  }
  __device__ void apply(State&, int, int tile, int split, int m, int i, bool valid, float v0,
                        float v1) const {
    if (!valid) return;
    float* o = out + (split * slab_rows + m) * ldo + tile * 32 + i;
    o[0] = v0;
    o[16] = v1;
  }
  __device__ void finish(State&, int, int, int) const {}
};

// SwiGLU: h[m, j] = silu(u . wg[j]) * (u . wu[j]), stored in the handle type,
// row-major (row stride ldh) or fragment-major (row length ldh) for the down
// projection's A operand.
template <typename T>
struct EpiSwiGLU {
  using State = NoState;
  const T* wg;
  const T* wu;
  int K;
  T* h;
  int64_t ldh;
  int frag;
  __device__ void init(State&) const {}
  __device__ void rows(int tile, int r16, const T*& w0, const T*& w1) const {
    w0 = wg + static_cast<int64_t>(tile * 16 + r16) * K;
    w1 = wu + static_cast<int64_t>(tile * 16 + r16) * K;
  }
  __device__ void apply(State&, int, int tile, int, int m, int i, bool valid, float g,
                        float u) const {
    if (!valid) return;
    const float s = g / (1.0f + expf(-g));
    const int j = tile * 16 + i;
    stf(h + (frag ? frag_major(m, j, static_cast<int>(ldh)) : static_cast<int64_t>(m) * ldh + j),
        s * u);
  }
  __device__ void finish(State&, int, int, int) const {}
};

// Pair tiles of a K or Q projection: tile covers, for one head, columns
// i0..i0+15 (sub-tile 0) and i0+D/2..i0+D/2+15 (sub-tile 1) -- the two members
// of every RoPE pair land in the same thread.
struct RopePairTile {
  int head, i0;
};
__device__ __forceinline__ RopePairTile rope_pair_tile(int t, int d) {
  const int per_head = d / 32;
  return RopePairTile{t / per_head, (t % per_head) * 16};
}

// Block QKV projection of one layer: q (RoPE) -> q buffer; k (RoPE), v -> the
// cache rows just past each sequence's committed context.
template <typename T>
struct EpiQKV {
  using State = NoState;
  const T* wq;
  const T* wk;
  const T* wv;
  int K, d, Hq, Hkv, B;
  T* q;
  int64_t ldq;
  T* kc;
  T* vc;
  int64_t cap;
  RopeFreq freq;
  SeqTable seq;
  __device__ void init(State&) const {}
  __device__ int nq() const { return Hq * (d / 32); }
  __device__ int nk() const { return Hkv * (d / 32); }
  __device__ void rows(int tile, int r16, const T*& w0, const T*& w1) const {
    if (tile < nq() + nk()) {
      const bool is_q = tile < nq();
      const RopePairTile pt = rope_pair_tile(is_q ? tile : tile - nq(), d);
      const T* W = is_q ? wq : wk;
      w0 = W + static_cast<int64_t>(pt.head * d + pt.i0 + r16) * K;
      w1 = w0 + static_cast<int64_t>(d / 2) * K;
    } else {
      const int c0 = (tile - nq() - nk()) * 32;
      w0 = wv + static_cast<int64_t>(c0 + r16) * K;
      w1 = w0 + static_cast<int64_t>(16) * K;
    }
  }
  __device__ void apply(State&, int, int tile, int, int m, int i, bool valid, float v0,
                        float v1) const {
    if (!valid) return;
    const int b = m / B, j = m % B;
    const int pos = seq_len_of(seq, b) + j;
    const int64_t row = seq.off[b] + pos;
    if (tile < nq() + nk()) {
      const bool is_q = tile < nq();
      const RopePairTile pt = rope_pair_tile(is_q ? tile : tile - nq(), d);
      const int c = pt.i0 + i;
      float cs, sn;
      rope_cos_sin(pos, c, freq, cs, sn);
      const float o0 = v0 * cs - v1 * sn;
      const float o1 = v1 * cs + v0 * sn;
      T* dst = is_q ? q + static_cast<int64_t>(m) * ldq + pt.head * d
                    : kc + (static_cast<int64_t>(pt.head) * cap + row) * d;
      stf(dst + c, o0);
      stf(dst + c + d / 2, o1);
    } else {
      const int ca = (tile - nq() - nk()) * 32 + i, cb = ca + 16;
      stf(vc + (static_cast<int64_t>(ca / d) * d + ca % d) * cap + row, v0);
      stf(vc + (static_cast<int64_t>(cb / d) * d + cb % d) * cap + row, v1);
    }
  }
  __device__ void finish(State&, int, int, int) const {}
};

// KV injection of context rows into every layer's cache: per layer, K pair
// tiles (RoPE at the row's position) then plain V tiles.
template <typename T>
struct EpiInject {
  using State = NoState;
  const T* wk[kMaxLayers];
  const T* wv[kMaxLayers];
  T* kc[kMaxLayers];
  T* vc[kMaxLayers];
  int K, d, Hkv;
  int64_t cap;
  RopeFreq freq;
  SeqTable seq;
  __device__ void init(State&) const {}
  __device__ int kt() const { return Hkv * (d / 32); }
  __device__ void rows(int tile, int r16, const T*& w0, const T*& w1) const {
    const int l = tile / (2 * kt()), t = tile % (2 * kt());
    if (t < kt()) {
      const RopePairTile pt = rope_pair_tile(t, d);
      w0 = wk[l] + static_cast<int64_t>(pt.head * d + pt.i0 + r16) * K;
      w1 = w0 + static_cast<int64_t>(d / 2) * K;
    } else {
      w0 = wv[l] + static_cast<int64_t>((t - kt()) * 32 + r16) * K;
      w1 = w0 + static_cast<int64_t>(16) * K;
    }
  }
  __device__ void apply(State&, int, int tile, int, int m, int i, bool valid, float v0,
                        float v1) const {
    int b, pos;
    if (!valid || !inject_row(seq, m, b, pos)) return;
    const int l = tile / (2 * kt()), t = tile % (2 * kt());
    const int64_t row = seq.off[b] + pos;
    if (t < kt()) {
      const RopePairTile pt = rope_pair_tile(t, d);
      const int c = pt.i0 + i;
      float cs, sn;
      rope_cos_sin(pos, c, freq, cs, sn);
      T* dst = kc[l] + (static_cast<int64_t>(pt.head) * cap + row) * d;
      stf(dst + c, v0 * cs - v1 * sn);
      stf(dst + c + d / 2, v1 * cs + v0 * sn);
    } else {
      const int ca = (t - kt()) * 32 + i, cb = ca + 16;
      stf(vc[l] + (static_cast<int64_t>(ca / d) * d + ca % d) * cap + row, v0);
      stf(vc[l] + (static_cast<int64_t>(cb / d) * d + cb % d) * cap + row, v1);
    }
  }
  __device__ void finish(State&, int, int, int) const {}
};

// LM head with fused argmax: logits never reach memory (unless dbg is set).
// Each thread keeps, for its rows, the best (value, lowest column) over the
// columns it sees across the workgroup's tiles; finish() folds the 16 columns
// of a row and writes one partial per (row, workgroup) for the finalize
// kernel (zhichai.net, "DFlash 的架构密码", 训练策略 3: the drafter reads out
// through the target's own LM head).
template <typename T, int MT>
struct EpiLMHead {
  struct State {
    float best[MT];
    int idx[MT];
  };
  const T* W;
  int K, V;
  int n_wg;            // workgroups of this launch
  float2* part;        // [rows][n_wg]: (value, index as float bits)
  float* dbg;          // [rows][V] or null
  __device__ void init(State& s) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { s.best[mt] = -INFINITY; s.idx[mt] = 0x7fffffff; }
  }
  __device__ void rows(int tile, int r16, const T*& w0, const T*& w1) const {
    const int c0 = min(tile * 32 + r16, V - 1), c1 = min(tile * 32 + 16 + r16, V - 1);
    w0 = W + static_cast<int64_t>(c0) * K;
    w1 = W + static_cast<int64_t>(c1) * K;
  }
  __device__ void apply(State& s, int mt, int tile, int, int m, int i, bool valid, float v0,
                        float v1) const {
    const int c0 = tile * 32 + i, c1 = c0 + 16;
    if (valid && dbg) {
      if (c0 < V) dbg[static_cast<int64_t>(m) * V + c0] = v0;
      if (c1 < V) dbg[static_cast<int64_t>(m) * V + c1] = v1;
    }
#pragma unroll
    for (int q = 0; q < MT; ++q) {
      if (q != mt) continue;
      // columns grow with the tile, so ">" keeps the lowest on ties
      if (c0 < V && v0 > s.best[q]) { s.best[q] = v0; s.idx[q] = c0; }
      if (c1 < V && v1 > s.best[q]) { s.best[q] = v1; s.idx[q] = c1; }
    }
  }
  __device__ void finish(State& s, int wg, int m0, int mc) const {
    const int t = threadIdx.x, i = t & 15, rr = t >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float best = s.best[mt];
      int bi = s.idx[mt];
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 16);
        const int oi = __shfl_xor(bi, o, 16);
        if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
      }
      const int m = mt * 16 + rr;
      if (i == 0 && m < mc)
        part[static_cast<int64_t>(m0 + m) * n_wg + wg] = make_float2(best, __int_as_float(bi));
    }
  }
};

// Cross-entropy partials of the LM head for the training layout.  Row m is
// slot j = m % B of block m / B; slots j >= 1 are scored against
// labels[(m / B) * (B - 1) + j - 1] (slot 0, the anchor, is not scored).  Per
// row, a workgroup leaves part[m][n_wg] = (max, sum of exp(z - max) over its
// columns, the label's logit if it is one of them else -inf, 0).
template <typename T, int MT>
struct EpiLMLoss {
  struct State {
    float mx[MT], sm[MT], zl[MT];
  };
  const T* W;
  int K, V;
  int n_wg;
  float4* part;
  const int32_t* labels;
  int B;
  float* dbg;          // [rows][V] or null
  __device__ void init(State& s) const {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { s.mx[mt] = -INFINITY; s.sm[mt] = 0.f; s.zl[mt] = -INFINITY; }
  }
  __device__ void rows(int tile, int r16, const T*& w0, const T*& w1) const {
    const int c0 = min(tile * 32 + r16, V - 1), c1 = min(tile * 32 + 16 + r16, V - 1);
    w0 = W + static_cast<int64_t>(c0) * K;
    w1 = W + static_cast<int64_t>(c1) * K;
  }
  __device__ void apply(State& s, int mt, int tile, int, int m, int i, bool valid, float v0,
                        float v1) const {
    const int c0 = tile * 32 + i, c1 = c0 + 16;
    if (valid && dbg) {
      if (c0 < V) dbg[static_cast<int64_t>(m) * V + c0] = v0;
      if (c1 < V) dbg[static_cast<int64_t>(m) * V + c1] = v1;
    }
    const int j = m % B;
    const int lab = valid && j > 0 ? labels[(m / B) * (B - 1) + j - 1] : -1;
#pragma unroll
    for (int q = 0; q < MT; ++q) {
      if (q != mt) continue;
      if (c0 < V) lse_merge(s.mx[q], s.sm[q], v0, 1.f);
      if (c1 < V) lse_merge(s.mx[q], s.sm[q], v1, 1.f);
      if (lab == c0) s.zl[q] = v0;
      if (lab == c1) s.zl[q] = v1;
    }
  }
  __device__ void finish(State& s, int wg, int m0, int mc) const {
    const int t = threadIdx.x, i = t & 15, rr = t >> 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float mx = s.mx[mt], sm = s.sm[mt], zl = s.zl[mt];
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const float om = __shfl_xor(mx, o, 16), os = __shfl_xor(sm, o, 16);
        zl = fmaxf(zl, __shfl_xor(zl, o, 16));
        lse_merge(mx, sm, om, os);
      }
      const int m = mt * 16 + rr;
      if (i == 0 && m < mc)
        part[static_cast<int64_t>(m0 + m) * n_wg + wg] = make_float4(mx, sm, zl, 0.f);
    }
  }
};

}  // namespace dflash
