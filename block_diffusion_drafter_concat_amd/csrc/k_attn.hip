// Block attention of the drafter: every slot of a block attends to its own
// sequence's injected context and to every slot of its own block -- no mask
// inside the block, nothing from other blocks (zhichai.net, "DFlash 的架构密码",
// 技术细节补充 / 稀疏注意力训练; zaocj.com news article on DFlash: bidirectional
// attention in a single forward pass).
//
// The block's own K/V were written by the QKV epilogue into the cache rows
// just past the committed context, so a sequence's visible keys are the
// contiguous rows [0, len + B) of its slab.
//
// Work split (HBM-bound over the K/V stream): workgroup = (context chunk,
// kv-head g, sequence b) with one wave per 16-query tile; the G*B queries of
// the kv head (G = q heads per kv head) are MFMA columns.  Every wave walks
// the whole chunk in 32-key steps with the next step's K/V fragments in
// flight; the waves of a workgroup read the same keys, so the repeats hit
// L1/L2 and HBM sees each K/V byte once.  No cross-wave merge is needed.
//   S^T[keys x queries] = K[keys x d] . Q^T   (K rows permuted so that the
//                                             C layout equals the next B layout)
//   O^T[d x queries]   += V^T[d x keys] . P^T (V^T straight from the transposed
//                                             V cache, 16 contiguous bytes/lane)
// Softmax is online in fp32 (base-2 with the scale folded in).  Chunks meet in
// the workspace in MFMA C-layout order; a merge kernel combines them in chunk
// order.
#include "kernels_attn.h"

namespace dflash {

// Softmax probabilities as MFMA B operands.  bf16: P = hi + lo with
// hi = bf16(P), lo = bf16(P - hi), two products, so P keeps ~16 significant
// bits (a single bf16 rounding of P would shift the output by ~1% after a few
// layers); fp32: P as is.
template <typename T>
__device__ __forceinline__ void pack8(Frag8<T>& f, const float* x);
template <>
__device__ __forceinline__ void pack8(Frag8<uint16_t>& f, const float* x) {
  f.v.x = f32x2_to_bf16x2(x[0], x[1]);
  f.v.y = f32x2_to_bf16x2(x[2], x[3]);
  f.v.z = f32x2_to_bf16x2(x[4], x[5]);
  f.v.w = f32x2_to_bf16x2(x[6], x[7]);
}
template <>
__device__ __forceinline__ void pack8(Frag8<float>& f, const float* x) {
  f.lo = make_float4(x[0], x[1], x[2], x[3]);
  f.hi = make_float4(x[4], x[5], x[6], x[7]);
}

// Zero the entries of a V^T fragment whose key index (first + e) is >= end.
__device__ __forceinline__ void mask_tail(Frag8<uint16_t>& f, int first, int end) {
  uint32_t w[4] = {f.v.x, f.v.y, f.v.z, f.v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (first + e >= end) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  f.v = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void mask_tail(Frag8<float>& f, int first, int end) {
  float w[8] = {f.lo.x, f.lo.y, f.lo.z, f.lo.w, f.hi.x, f.hi.y, f.hi.z, f.hi.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (first + e >= end) w[e] = 0.f;
  pack8(f, w);
}

// Output element (query row r, head dim d) of a kv head's G*B x D block goes
// to o[(b*B + j) * ldq + (g*G + h) * D + d] with r = h*B + j.
template <typename T>
__device__ __forceinline__ void store_out4(const AttnArgs& p, int b, int g, int r, int d,
                                           const float* v) {
  const int B = p.B, G = p.G, D = p.head_dim;
  const int h = r / B, j = r % B;
  T* o = static_cast<T*>(p.o) + static_cast<int64_t>(b * B + j) * p.ldq + (g * G + h) * D + d;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) stf(o + jj, v[jj]);
}

// Partial of chunk c of (b, g): O^T fragments in C-layout order
// part_o[slot][qt][dt][lane] (float4 over jj) and (max, sum) per query row.
template <typename T, int D, int NQ>
__global__ __launch_bounds__(NQ * 64) void block_attn_kernel(AttnArgs p) {
  constexpr int DS = D / 32;   // 32-wide k steps over the head dimension
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int QR = NQ * 16;  // query rows (padded)

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int qt = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int B = p.B, G = p.G, GB = G * B;
  KeySpan span;
  if (!attn_key_span(p, b, c, span)) return;
  const int kbeg = span.kbeg, kend = span.kend, n_keys = span.n_src;
  const int n_chunks_b = span.n_chunks;
  const int64_t base = span.base, cap = span.cap;
  const T* Kg = static_cast<const T*>(span.k) + static_cast<int64_t>(g) * cap * D;
  const T* Vg = static_cast<const T*>(span.v) + static_cast<int64_t>(g) * D * cap;
  const int r = qt * 16 + r16;   // this lane's query row (MFMA column)

  Frag8<T> qf[DS];
  if (r < GB) {
    const int h = r / B, j = r % B;
    const T* qrow = static_cast<const T*>(p.q) + static_cast<int64_t>(b * B + j) * p.ldq +
                    (g * G + h) * D + kg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) ld_frag(qf[ds], qrow + ds * 32);
  } else {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) zero_frag(qf[ds]);
  }

  float m_run = -1e30f, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero4();

  // K fragment rows: tile t row rr <-> key kb + (rr/4)*8 + t*4 + rr%4, so the
  // S^T C layout gives lane group kg the 8 consecutive keys kb + kg*8 .. +8.
  Frag8<T> kf[2][2][DS], vf[2][DT];
  auto load = [&](int buf, int kb) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = min(kb + (r16 >> 2) * 8 + t * 4 + (r16 & 3), n_keys - 1);
      const T* krow = Kg + (base + key) * D + kg * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) ld_frag(kf[buf][t][ds], krow + ds * 32);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      ld_frag(vf[buf][dt], Vg + static_cast<int64_t>(dt * 16 + r16) * cap + base + kb + kg * 8);
  };
  auto step = [&](int buf, int kb) {
    if (kb + 32 > kend) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) mask_tail(vf[buf][dt], kb + kg * 8, kend);
    }
    f32x4 s0 = zero4(), s1 = zero4();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s0 = mfma16(s0, kf[buf][0][ds], qf[ds]);
      s1 = mfma16(s1, kf[buf][1][ds], qf[ds]);
    }
    float x[8];
    float mx = m_run;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = (e < 4 ? s0[e] : s1[e - 4]) * p.scale_log2;
      if (kb + kg * 8 + e >= kend) v = -INFINITY;
      x[e] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float alpha = exp2f(m_run - mx);
    m_run = mx;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = exp2f(x[e] - mx);
      ls += x[e];
    }
    l_run = l_run * alpha + ls;
    Frag8<T> pf;
    pack8(pf, x);
    constexpr bool kSplitP = sizeof(T) == 2;
    Frag8<T> pl;
    if (kSplitP) {
      float lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) lo[e] = x[e] - Store<T>::load(Store<T>::make(x[e]));
      pack8(pl, lo);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = o[dt] * alpha;
      o[dt] = mfma16(o[dt], vf[buf][dt], pf);
      if (kSplitP) o[dt] = mfma16(o[dt], vf[buf][dt], pl);
    }
  };
  load(0, kbeg);
  int kb = kbeg;
  for (; kb + 32 < kend; kb += 64) {
    load(1, kb + 32);
    step(0, kb);
    if (kb + 64 < kend) load(0, kb + 64);
    step(1, kb + 32);
  }
  if (kb < kend) step(0, kb);

  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (n_chunks_b == 1) {
    if (r < GB) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float v[4] = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
        store_out4<T>(p, b, g, r, dt * 16 + kg * 4, v);
      }
    }
    return;
  }
  const int64_t slot = (static_cast<int64_t>(b) * p.n_kv + g) * p.max_chunks + c;
  float4* po = reinterpret_cast<float4*>(p.part_o) + (slot * NQ + qt) * DT * 64 + lane;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) po[dt * 64] = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  if (kg == 0) p.part_ml[slot * QR + r] = make_float2(m_run, l);
}

// bf16 variant with the K/V stream staged through LDS.  The workgroup's
// threads load each 32-key step once (K rows and V^T rows, 16-byte chunks)
// P steps ahead into registers, write it into one of two LDS slots, and the
// waves read their MFMA fragments from there.  P steps of 16 KB (head dim
// 128) per workgroup are in flight at once.  The loads go to registers and
// the slot is published with an explicit LDS wait and a plain s_barrier: the
// compiler's waits on the loads stay exact (a workgroup fence here would
// also drain every prefetch in flight).
//
// LDS slot: K [32 keys][D] with 16-byte chunk c of key k at c ^ kswz(k), and
// V^T [D][32 keys] with chunk c of row d at c ^ ((d >> 1) & 3): each group of
// 8 lanes of an MFMA fragment read (8 keys or 8 d-rows at one chunk; LDS
// serves 16-byte reads 8 lanes at a time) then hits 8 distinct bank groups.
template <int KCH>
__device__ __forceinline__ int kswz(int k) {
  return ((((k >> 3) & 3) << 2) | (k & 3)) & (KCH - 1);
}

template <int D, int NQ, int P>
__global__ __launch_bounds__(NQ * 64) void block_attn_lds_kernel(AttnArgs p) {
  using T = uint16_t;
  constexpr int DS = D / 32;   // 32-wide k steps over the head dimension
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int QR = NQ * 16;  // query rows (padded)
  constexpr int NT = NQ * 64;
  constexpr int KCH = D / 8;                   // 16-byte chunks per K row
  constexpr int SLOT_K = 32 * D;               // elements of the K part of a slot
  constexpr int SLOT = 2 * 32 * D;             // K + V^T elements per slot
  constexpr int CH = SLOT / 8;                 // 16-byte chunks per step
  constexpr int PER = (CH + NT - 1) / NT;      // chunks per thread per step
  __shared__ __align__(16) T lds[2 * SLOT];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, qt = t >> 6, lane = t & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int B = p.B, G = p.G, GB = G * B;
  KeySpan span;
  if (!attn_key_span(p, b, c, span)) return;
  const int kbeg = span.kbeg, kend = span.kend, n_keys = span.n_src;
  const int n_steps = (kend - kbeg + 31) / 32;
  const int n_chunks_b = span.n_chunks;
  const int64_t base = span.base, cap = span.cap;
  const T* Kg = static_cast<const T*>(span.k) + static_cast<int64_t>(g) * cap * D;
  const T* Vg = static_cast<const T*>(span.v) + static_cast<int64_t>(g) * D * cap;
  const int r = qt * 16 + r16;   // this lane's query row (MFMA column)

  Frag8<T> qf[DS];
  if (r < GB) {
    const int h = r / B, j = r % B;
    const T* qrow = static_cast<const T*>(p.q) + static_cast<int64_t>(b * B + j) * p.ldq +
                    (g * G + h) * D + kg * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) ld_frag(qf[ds], qrow + ds * 32);
  } else {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) zero_frag(qf[ds]);
  }

  // chunk i of a step: K (key i / KCH, chunk i % KCH) for i < 32 KCH, else
  // V^T (row d = j / 4, keys (j % 4) * 8 .. +8) with j = i - 32 KCH.  K rows
  // past the sequence's keys are clamped (their scores are masked); V^T reads
  // stay inside the sequence's slab (capacities are multiples of 32).
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  struct StepRegs {
    u32x4 v[PER];
  };
  static_assert(P == 1 || P == 2 || P == 4, "prefetch depth");
  StepRegs R0, R1, R2, R3;   // step s lives in R(s % P) (named: no stack array)
  // Every thread issues the same PER loads at every refill (chunk indices past
  // the step are clamped, and so is the step), so the compiler's count of
  // loads in flight is the same on every path and its waits stay exact.
  auto gload = [&](StepRegs& dst, int kb) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = min(t + u * NT, CH - 1);
      const T* src;
      if (i < 32 * KCH) {
        const int key = min(kb + i / KCH, n_keys - 1);
        src = Kg + (base + key) * D + (i % KCH) * 8;
      } else {
        const int jj = i - 32 * KCH;
        src = Vg + static_cast<int64_t>(jj >> 2) * cap + base + kb + (jj & 3) * 8;
      }
      dst.v[u] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  // (a clamped chunk index rewrites the last chunk with the same data)
  auto lstore = [&](const StepRegs& src, int slot) {
    T* sl = lds + slot * SLOT;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = min(t + u * NT, CH - 1);
      int off;
      if (i < 32 * KCH) {
        const int k = i / KCH, ch = i % KCH;
        off = k * D + ((ch ^ kswz<KCH>(k)) << 3);
      } else {
        const int jj = i - 32 * KCH, d = jj >> 2, ch = jj & 3;
        off = SLOT_K + d * 32 + ((ch ^ ((d >> 1) & 3)) << 3);
      }
      *reinterpret_cast<u32x4*>(sl + off) = src.v[u];
    }
  };

  float m_run = -1e30f, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero4();

  // K fragment rows: tile t2 row rr <-> key (rr/4)*8 + t2*4 + rr%4 of the
  // step, so the S^T C layout gives lane group kg the 8 consecutive keys
  // kg*8 .. +8 (the V^T fragment's keys).
  auto compute = [&](int slot, int kb) {
    const T* sl = lds + slot * SLOT;
    Frag8<T> kf[2][DS];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int k = (r16 >> 2) * 8 + t2 * 4 + (r16 & 3);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kf[t2][ds].v = *reinterpret_cast<const uint4*>(
            sl + k * D + (((ds * 4 + kg) ^ kswz<KCH>(k)) << 3));
    }
    const bool tail = kb + 32 > kend;   // uniform: the chunk's last, partial step
    f32x4 s0 = zero4(), s1 = zero4();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s0 = mfma16(s0, kf[0][ds], qf[ds]);
      s1 = mfma16(s1, kf[1][ds], qf[ds]);
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (e < 4 ? s0[e] : s1[e - 4]) * p.scale_log2;
    if (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kb + kg * 8 + e >= kend) x[e] = -INFINITY;
    }
    float mx = m_run;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // exponents are <= 0 (2^x of -inf is 0); the hardware 2^x is used as is
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = __builtin_amdgcn_exp2f(x[e] - mx);
      ls += x[e];
    }
    // rescale only when some query's running max moved (else alpha == 1)
    if (__any(mx != m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = o[dt] * alpha;
    }
    m_run = mx;
    l_run += ls;
    // V^T fragments, read once the K fragments are dead (fewer live registers:
    // two waves per SIMD)
    Frag8<T> vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = dt * 16 + r16;
      vf[dt].v = *reinterpret_cast<const uint4*>(sl + SLOT_K + d * 32 +
                                                 ((kg ^ ((d >> 1) & 3)) << 3));
    }
    if (tail) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) mask_tail(vf[dt], kb + kg * 8, kend);
    }
    // P = hi + lo in bf16 (see pack8)
    Frag8<T> pf, pl;
    pack8(pf, x);
    const uint32_t hw[4] = {pf.v.x, pf.v.y, pf.v.z, pf.v.w};
    float lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      lo[e] = x[e] - __uint_as_float((e & 1) ? (hw[e >> 1] & 0xffff0000u) : (hw[e >> 1] << 16));
    pack8(pl, lo);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = mfma16(o[dt], vf[dt], pf);
      o[dt] = mfma16(o[dt], vf[dt], pl);
    }
  };

  auto step_kb = [&](int s) { return kbeg + 32 * min(s, n_steps - 1); };
  gload(R0, step_kb(0));
  if constexpr (P > 1) gload(R1, step_kb(1));
  if constexpr (P > 2) {
    gload(R2, step_kb(2));
    gload(R3, step_kb(3));
  }
  // one step: publish its slot, refill its registers P steps ahead, compute
  auto one = [&](StepRegs& rq, int s) {
    const int kb = kbeg + 32 * s;
    lstore(rq, s & 1);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this thread's slot writes
    __builtin_amdgcn_s_barrier();          // slot s & 1 complete; slot (s+1) & 1 free
    gload(rq, step_kb(s + P));
    compute(s & 1, kb);
  };

  // whole groups of P steps (no branch between the refills, so the waits on
  // each step's registers leave the later steps' loads in flight), then the
  // last n_steps % P steps
  int s0 = 0;
  for (; s0 + P <= n_steps; s0 += P) {
    one(R0, s0);
    if constexpr (P > 1) one(R1, s0 + 1);
    if constexpr (P > 2) {
      one(R2, s0 + 2);
      one(R3, s0 + 3);
    }
  }
  if (s0 < n_steps) one(R0, s0);
  if constexpr (P > 1) if (s0 + 1 < n_steps) one(R1, s0 + 1);
  if constexpr (P > 2) if (s0 + 2 < n_steps) one(R2, s0 + 2);

  float l = l_run;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (n_chunks_b == 1) {
    if (r < GB) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float v[4] = {o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv};
        store_out4<T>(p, b, g, r, dt * 16 + kg * 4, v);
      }
    }
    return;
  }
  const int64_t slot = (static_cast<int64_t>(b) * p.n_kv + g) * p.max_chunks + c;
  float4* po = reinterpret_cast<float4*>(p.part_o) + (slot * NQ + qt) * DT * 64 + lane;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) po[dt * 64] = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  if (kg == 0) p.part_ml[slot * QR + r] = make_float2(m_run, l);
}

// One thread per (query tile, 16-row d tile, lane) of a (kv head, sequence):
// o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c over the sequence's chunks,
// in chunk order, all loads of 8 chunks issued before they are combined.
template <typename T, int D, int NQ>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs p) {
  constexpr int DT = D / 16, QR = NQ * 16;
  const int g = blockIdx.y, b = blockIdx.z;
  const int B = p.B, G = p.G, GB = G * B;
  const int n_chunks_b = attn_n_chunks(p, b);
  if (n_chunks_b <= 1) return;   // written directly by the attention kernel
  const int e = blockIdx.x * 256 + threadIdx.x;   // (qt, dt, lane)
  if (e >= NQ * DT * 64) return;
  const int lane = e & 63, dt = (e >> 6) % DT, qt = (e >> 6) / DT;
  const int r = qt * 16 + (lane & 15);
  if (r >= GB) return;
  const int64_t slot0 = (static_cast<int64_t>(b) * p.n_kv + g) * p.max_chunks;
  const float2* ml = p.part_ml + slot0 * QR + r;
  const float4* po = reinterpret_cast<const float4*>(p.part_o) + (slot0 * NQ + qt) * DT * 64 +
                     dt * 64 + lane;
  constexpr int kU = 8;
  float M = -1e30f, den = 0.f;
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < n_chunks_b; c0 += kU) {
    float2 v[kU];
    float4 w4[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = c0 + u < n_chunks_b;
      v[u] = ok ? ml[static_cast<int64_t>(c0 + u) * QR] : make_float2(-1e30f, 0.f);
      w4[u] = ok ? po[static_cast<int64_t>(c0 + u) * NQ * DT * 64] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kU; ++u) Mn = fmaxf(Mn, v[u].x);
    const float a = exp2f(M - Mn);
    den *= a;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) num[jj] *= a;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float w = exp2f(v[u].x - Mn);
      den += w * v[u].y;
      num[0] += w * w4[u].x;
      num[1] += w * w4[u].y;
      num[2] += w * w4[u].z;
      num[3] += w * w4[u].w;
    }
    M = Mn;
  }
  const float inv = 1.0f / den;
  const float out[4] = {num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
  store_out4<T>(p, b, g, r, dt * 16 + (lane >> 4) * 4, out);
}

// 32-key steps in flight per workgroup (bf16): at most 8 staged 16-byte
// chunks per thread (32 VGPRs), so that two waves fit on a SIMD; narrower
// workgroups prefetch fewer steps.
template <int D, int NQ>
constexpr int attn_prefetch() {
  constexpr int per = (2 * 32 * D / 8 + NQ * 64 - 1) / (NQ * 64);
  return 8 / per < 1 ? 1 : (8 / per > 4 ? 4 : 8 / per);
}

template <typename T, int D, int NQ>
static hipError_t launch_attn_nq(const AttnArgs& a, dim3 grid, int batch, hipStream_t st) {
  if constexpr (sizeof(T) == 2)
    block_attn_lds_kernel<D, NQ, attn_prefetch<D, NQ>()><<<grid, NQ * 64, 0, st>>>(a);
  else
    block_attn_kernel<T, D, NQ><<<grid, NQ * 64, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks <= 1) return e;
  dim3 mgrid((NQ * (D / 16) * 64 + 255) / 256, a.n_kv, batch);
  attn_merge_kernel<T, D, NQ><<<mgrid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_t(const AttnArgs& a, int nq, dim3 grid, int batch, hipStream_t st) {
  switch (nq) {
    case 1: return launch_attn_nq<T, D, 1>(a, grid, batch, st);
    case 2: return launch_attn_nq<T, D, 2>(a, grid, batch, st);
    case 3: return launch_attn_nq<T, D, 3>(a, grid, batch, st);
    case 4: return launch_attn_nq<T, D, 4>(a, grid, batch, st);
    case 5: return launch_attn_nq<T, D, 5>(a, grid, batch, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_block_attention(bool bf16, int head_dim, const AttnArgs& a, int batch,
                                  hipStream_t st) {
  const int nq = (a.G * a.B + 15) / 16;
  dim3 grid(a.max_chunks, a.n_kv, batch);
  if (bf16) {
    if (head_dim == 128) return launch_attn_t<uint16_t, 128>(a, nq, grid, batch, st);
    if (head_dim == 64) return launch_attn_t<uint16_t, 64>(a, nq, grid, batch, st);
  } else {
    if (head_dim == 128) return launch_attn_t<float, 128>(a, nq, grid, batch, st);
    if (head_dim == 64) return launch_attn_t<float, 64>(a, nq, grid, batch, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dflash
