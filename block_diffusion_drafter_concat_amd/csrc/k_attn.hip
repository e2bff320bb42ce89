// Block attention of the drafter: every slot of a block attends to its own
// sequence's injected context and to every slot of its own block -- no mask
// inside the block, nothing from other blocks (zhichai.net, "DFlash 的架构密码",
// 技术细节补充 / 稀疏注意力训练; zaocj.com news article on DFlash: bidirectional
// attention in a single forward pass).
//
// At inference the block's own K/V were written by the QKV epilogue into the
// cache rows just past the committed context, so a sequence's visible keys are
// the contiguous rows [0, len + B) of its slab.  In the training layout
// (AttnArgs::kb set) an entry's visible keys are the first len rows of its
// sequence's slab plus its block's own rows in a separate buffer, read as one
// extra chunk (KeySpan).
//
// Work split (HBM-bound over the K/V stream): workgroup = (key chunk, kv-head
// g, sequence b) with one wave per 16-query tile; the G*B queries of the kv
// head (G = q heads per kv head) are MFMA columns.
//   S^T[keys x queries] = K[keys x d] . Q^T   (K rows permuted so that the
//                                             C layout equals the next B layout)
//   O^T[d x queries]   += V^T[d x keys] . P^T (V^T rows of the transposed V
//                                             cache, 16 contiguous bytes/lane)
// Softmax is online in fp32 (base-2 with the scale folded in).  float32:
// every wave streams its fragments from global memory (repeats across waves
// hit L1/L2).  bf16: the workgroup loads each 32-key step once into an LDS
// ring with LDS-destination loads (block_attn_dma_kernel).  Chunks meet in
// the workspace in MFMA C-layout order; a merge kernel combines them.
#include <atomic>
#include <type_traits>

#include "gemm_tiled.h"   // LDS-destination load and LDS-read helpers
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

// Output element (query row r, head dim d) of a kv head's G*B x D block is
// o[m, k] with m = b*B + j, k = (g*G + h) * D + d and r = h*B + j: row-major
// (row stride ldq) or, for the output projection's weight-streaming GEMM,
// fragment-major (four columns of one aligned run of 32 stay contiguous).
template <typename T>
__device__ __forceinline__ void store_out4(const AttnArgs& p, int b, int g, int r, int d,
                                           const float* v) {
  const int B = p.B, G = p.G, D = p.head_dim;
  const int h = r / B, j = r % B;
  const int m = b * B + j, k = (g * G + h) * D + d;
  T* o = static_cast<T*>(p.o) + (p.ofrag ? frag_major(m, k, static_cast<int>(p.ldq))
                                         : static_cast<int64_t>(m) * p.ldq + k);
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

  int c, g, b;
  attn_wg_coords(p, c, g, b);
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

// LDS slot of one 32-key step: K [32 keys][D] with 16-byte chunk c of key k
// at c ^ kswz(k), and V^T [D][32 keys] with chunk c of row d at
// c ^ ((d >> 1) & 3): each group of 8 lanes of an MFMA fragment read (8 keys
// or 8 d-rows at one chunk; LDS serves 16-byte reads 8 lanes at a time) then
// hits 8 distinct bank groups.
template <int KCH>
__device__ __forceinline__ int kswz(int k) {
  return ((((k >> 3) & 3) << 2) | (k & 3)) & (KCH - 1);
}

// bf16 variant whose K/V stream goes global -> LDS with LDS-destination buffer
// loads (no staging registers, no LDS stores): a ring of NSLOT step slots per
// workgroup with NSLOT - 1 steps in flight.  48 KB of ring per workgroup
// (head dim 128: 3 slots) lets three workgroups share a CU, whose waves then
// overlap one another's softmax and MFMA latency with the loads; measured at
// 35K keys: 3 slots 27.8 us, 4 slots 29.1, 5 slots 30.4 (loads alone 23-24,
// math alone 21-22).  Slot layout
// and swizzles as above: a lane of a 1 KB load instruction
// writes LDS chunk q = 64 i + lane of the slot, so it fetches the global chunk
// that belongs there.  Fragment reads are instructions the compiler does not
// track (tile_ds_read) with explicit waits, so the loads in flight are never
// drained before an LDS read; each step: wait for this wave's loads of the
// step, barrier (every wave's loads landed; the slot of the previous step is
// free), refill that slot NSLOT - 1 steps ahead, compute.
template <int D>
constexpr int attn_dma_slots() {
  return 49152 / (2 * 32 * D * 2) > 8 ? 8 : 49152 / (2 * 32 * D * 2);
}

__device__ __forceinline__ Frag8<uint16_t> as_frag(const u32x4_t& x) {
  Frag8<uint16_t> f;
  f.v = make_uint4(x.x, x.y, x.z, x.w);
  return f;
}

template <int D, int NQ, int NSLOT>
__global__ __launch_bounds__(NQ * 64) void block_attn_dma_kernel(AttnArgs p) {
  using T = uint16_t;
  constexpr int DS = D / 32;   // 32-wide k steps over the head dimension
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int QR = NQ * 16;  // query rows (padded)
  constexpr int KCH = D / 8;                    // 16-byte chunks per K row
  constexpr int SLOT_K = 32 * D;                // elements of the K part of a slot
  constexpr int SLOT = 2 * 32 * D;              // K + V^T elements per slot
  constexpr int NIK = SLOT_K * 2 / 1024;        // 1 KB load instructions: K part
  constexpr int PERK = (NIK + NQ - 1) / NQ;     // K (and V^T) instructions per wave
  constexpr int PERW = 2 * PERK;                // per wave (extra ones repeat the last)
  constexpr int T2OFF = 4 * D * 2;              // bytes between the two K fragment tiles
  static_assert(PERW * (NSLOT - 2) < 64, "vmcnt range");
  extern __shared__ __align__(16) uint16_t lds_ring[];

  int c, g, b;
  attn_wg_coords(p, c, g, b);
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), qt = wave;
  const int r16 = lane & 15, kg = lane >> 4;
  const int B = p.B, G = p.G, GB = G * B;
  KeySpan span;
  if (!attn_key_span(p, b, c, span)) return;
  const int kbeg = span.kbeg, kend = span.kend;
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

  // per-lane byte offsets of this wave's load instructions (step-invariant):
  // K chunk (key k, chunk ch) sits at LDS chunk k*KCH + (ch ^ kswz(k)); V^T
  // chunk (row d, chunk ch) at SLOT_K/8 + d*4 + (ch ^ ((d >> 1) & 3))
  // Wave w issues K instructions w*PERK .. +PERK and the same V^T ones, so
  // which part an instruction loads is known at compile time.
  uint32_t voff[PERW];
#pragma unroll
  for (int u = 0; u < PERK; ++u) {
    const int ii = min(wave * PERK + u, NIK - 1);
    const int q = ii * 64 + lane;
    const int k = q / KCH, ch = (q % KCH) ^ kswz<KCH>(q / KCH);
    voff[u] = static_cast<uint32_t>((k * D + ch * 8) * 2);
    const int d = q >> 2, cv = (q & 3) ^ ((d >> 1) & 3);
    voff[PERK + u] = static_cast<uint32_t>((static_cast<int64_t>(d) * cap + cv * 8) * 2);
  }
  const uint64_t head_bytes = static_cast<uint64_t>(cap) * D * 2;
  // Rows past the chunk's keys (up to the step's 32) are read too: they lie
  // inside the entry's slab (capacities are multiples of 32), their scores
  // are masked and their V entries zeroed.
  auto issue = [&](int st) {
    const int kb = kbeg + 32 * min(st, n_steps - 1);   // steps past the end repeat the last
    lds_u16* sl = (lds_u16*)(lds_ring) + (st % NSLOT) * SLOT;
    const int soff_k = static_cast<int>((base + kb) * D * 2);
    const int soff_v = static_cast<int>((base + kb) * 2);
    // (the resources are locals and the offset an int: a resource temporary
    // passed to the builtin, or an unsigned array element as its offset, makes
    // the host pass drop the kernel's launch stub without a diagnostic)
    const __amdgpu_buffer_rsrc_t krs = tile_rsrc(Kg, head_bytes);
    const __amdgpu_buffer_rsrc_t vrs = tile_rsrc(Vg, head_bytes);
#pragma unroll
    for (int u = 0; u < PERK; ++u) {
      const int ii = min(wave * PERK + u, NIK - 1);
      const int vk = static_cast<int>(voff[u]), vv = static_cast<int>(voff[PERK + u]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, sl + ii * 512, 16, vk, soff_k, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, sl + SLOT_K + ii * 512, 16, vv, soff_v, 0, 0);
    }
  };

  float m_run = -1e30f, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = zero4();

  // Fragment addresses.  K tile t2 row rr <-> key (rr/4)*8 + t2*4 + rr%4, so
  // the S^T C layout gives lane group kg keys kg*8 .. +8; that key's swizzle
  // is r16 & (KCH - 1) for both tiles (tile 1 sits T2OFF bytes later).  V^T
  // row d = dt*16 + r16 has swizzle (r16 >> 1) & 3 (tile dt 1 KB later).
  const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)(lds_ring)));
  const int k0 = (r16 >> 2) * 8 + (r16 & 3);
  uint32_t koff[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
    koff[ds] = lds0 + 2 * (k0 * D + (((ds * 4 + kg) ^ (r16 & (KCH - 1))) << 3));
  const uint32_t vofs = lds0 + 2 * (SLOT_K + r16 * 32 + ((kg ^ ((r16 >> 1) & 3)) << 3));

  // tail_c: std::true_type for the chunk's last step (the only one that can
  // hold keys past kend), so full steps carry no masking code at all
  auto compute = [&](auto tail_c, int slot, int kb) {
    constexpr bool tail = decltype(tail_c)::value;
    const uint32_t sb = static_cast<uint32_t>(slot * SLOT * 2);
    u32x4_t kf0[DS], kf1[DS], vf[DT];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      kf0[ds] = tile_ds_read<0>(koff[ds] + sb);
      kf1[ds] = tile_ds_read<T2OFF>(koff[ds] + sb);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    tile_tie_all(kf0, std::make_integer_sequence<int, DS>{});
    tile_tie_all(kf1, std::make_integer_sequence<int, DS>{});
    f32x4 s0 = zero4(), s1 = zero4();
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s0 = mfma16(s0, as_frag(kf0[ds]), qf[ds]);
      s1 = mfma16(s1, as_frag(kf1[ds]), qf[ds]);
    }
    // V^T fragments now: their reads overlap the softmax
    tile_read_frags(vf, vofs + sb, std::make_integer_sequence<int, DT>{});
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (e < 4 ? s0[e] : s1[e - 4]) * p.scale_log2;
    if constexpr (tail) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kb + kg * 8 + e >= kend) x[e] = -INFINITY;
    }
    float mx = m_run;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // Lazy rescale: the reference max m_run moves only when a row's max
    // passes it by more than 8 (base 2), so the exponents stay <= 8 and the
    // accumulators (in AGPRs: a rescale moves each one out and back) are
    // touched rarely.  o and l share the reference, so o / l is unchanged.
    if (__any(mx > m_run + 8.0f)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = o[dt] * alpha;
      m_run = mx;
    }
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = __builtin_amdgcn_exp2f(x[e] - m_run);
      ls += x[e];
    }
    l_run += ls;
    Frag8<T> pf, pl;
    pack8(pf, x);
    const uint32_t hw[4] = {pf.v.x, pf.v.y, pf.v.z, pf.v.w};
    float lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      lo[e] = x[e] - __uint_as_float((e & 1) ? (hw[e >> 1] & 0xffff0000u) : (hw[e >> 1] << 16));
    pack8(pl, lo);
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the V^T fragments
    tile_tie_all(vf, std::make_integer_sequence<int, DT>{});
    Frag8<T> v[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) v[dt] = as_frag(vf[dt]);
    if constexpr (tail) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) mask_tail(v[dt], kb + kg * 8, kend);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = mfma16(o[dt], v[dt], pf);
      o[dt] = mfma16(o[dt], v[dt], pl);
    }
  };

#pragma unroll
  for (int j = 0; j < NSLOT - 1; ++j) issue(j);
  // the query fragments (loaded before the ring) are in: only ring loads may
  // stay in flight (else the compiler drains the whole ring before the loop)
  // (at most 63 in the field; the query loads are older than every ring load)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(PERW * (NSLOT - 1) > 63 ? 63 : PERW * (NSLOT - 1)));
  auto step = [&](auto tail_c, int s) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(PERW * (NSLOT - 2)));   // this wave's loads of step s
    __builtin_amdgcn_s_barrier();                                 // everyone's; slot of s-1 free
    issue(s + NSLOT - 1);
    compute(tail_c, s % NSLOT, kbeg + 32 * s);
  };
  for (int s = 0; s < n_steps - 1; ++s) step(std::false_type{}, s);
  step(std::true_type{}, n_steps - 1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may land after the workgroup ends

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

// Chunk merge.  Workgroup (query tile qt, 16-row d tile dt) of a (kv head,
// sequence): lane l owns output element (query row qt*16 + l%16, d rows
// dt*16 + (l/16)*4 .. +4); wave w folds chunks w, w + 4, w + 8, ... (8 loads
// in flight per thread) into o = sum_c 2^(m_c - M) O_c, l = sum_c 2^(m_c - M)
// l_c, and the four waves' folds meet in LDS in wave order (deterministic).
template <typename T, int D, int NQ>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs p) {
  constexpr int DT = D / 16, QR = NQ * 16;
  const int qt = blockIdx.x / DT, dt = blockIdx.x % DT, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int B = p.B, G = p.G, GB = G * B;
  const int n_chunks_b = attn_n_chunks(p, b);
  if (n_chunks_b <= 1) return;   // written directly by the attention kernel
  const int r = qt * 16 + (lane & 15);
  const int64_t slot0 = (static_cast<int64_t>(b) * p.n_kv + g) * p.max_chunks;
  const float2* ml = p.part_ml + slot0 * QR + r;
  const float4* po = reinterpret_cast<const float4*>(p.part_o) + (slot0 * NQ + qt) * DT * 64 +
                     dt * 64 + lane;
  constexpr int kU = 8;
  float M = -1e30f, den = 0.f;
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int c0 = wave; c0 < n_chunks_b; c0 += 4 * kU) {
    float2 v[kU];
    float4 w4[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + 4 * u;
      const bool ok = c < n_chunks_b;
      v[u] = ok ? ml[static_cast<int64_t>(c) * QR] : make_float2(-1e30f, 0.f);
      w4[u] = ok ? po[static_cast<int64_t>(c) * NQ * DT * 64] : make_float4(0.f, 0.f, 0.f, 0.f);
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
  __shared__ float sm[4][64][6];
  float* mine = sm[wave][lane];
  mine[0] = M;
  mine[1] = den;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) mine[2 + jj] = num[jj];
  __syncthreads();
  if (wave != 0 || r >= GB) return;
  float Mt = sm[0][lane][0];
#pragma unroll
  for (int w = 1; w < 4; ++w) Mt = fmaxf(Mt, sm[w][lane][0]);
  float dn = 0.f, nm[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float a = exp2f(sm[w][lane][0] - Mt);
    dn += a * sm[w][lane][1];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) nm[jj] += a * sm[w][lane][2 + jj];
  }
  const float inv = 1.0f / dn;
  const float out[4] = {nm[0] * inv, nm[1] * inv, nm[2] * inv, nm[3] * inv};
  store_out4<T>(p, b, g, r, dt * 16 + (lane >> 4) * 4, out);
}

template <typename T, int D, int NQ>
static hipError_t launch_attn_nq(const AttnArgs& a, dim3 grid, int batch, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    constexpr int NS = attn_dma_slots<D>();
    constexpr int lds = NS * 2 * 32 * D * 2;
    auto kern = &block_attn_dma_kernel<D, NQ, NS>;
    static std::atomic<uint64_t> lds_set{0};
    const hipError_t e0 = set_dynamic_lds_once(lds_set, reinterpret_cast<const void*>(kern), lds);
    if (e0 != hipSuccess) return e0;
    kern<<<grid, NQ * 64, lds, st>>>(a);
  } else {
    block_attn_kernel<T, D, NQ><<<grid, NQ * 64, 0, st>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks <= 1) return e;
  dim3 mgrid(NQ * (D / 16), a.n_kv, batch);
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
  const dim3 grid = a.n_order > 0 ? dim3(a.n_order * a.n_kv) : dim3(a.max_chunks, a.n_kv, batch);
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
