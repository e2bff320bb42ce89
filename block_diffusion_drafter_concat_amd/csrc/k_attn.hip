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
// kv-head g, sequence b), 4 waves, each wave takes every 4th 32-key step.
// All G*B queries of the kv-head (G = q heads per kv head) ride along as MFMA
// columns, so each K/V byte is read once per workgroup:
//   S^T[keys x queries] = K[keys x d] . Q^T   (K rows permuted so that the
//                                             C layout equals the next B layout)
//   O^T[d x queries]   += V^T[d x keys] . P^T (V^T straight from the transposed
//                                             V cache, 16 contiguous bytes/lane)
// Softmax is online in fp32 (base-2 with the scale folded in).  Chunks meet in
// the workspace; a separate merge kernel combines them in chunk order.
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
  f.v.x = static_cast<uint32_t>(f32_to_bf16(x[0])) | (static_cast<uint32_t>(f32_to_bf16(x[1])) << 16);
  f.v.y = static_cast<uint32_t>(f32_to_bf16(x[2])) | (static_cast<uint32_t>(f32_to_bf16(x[3])) << 16);
  f.v.z = static_cast<uint32_t>(f32_to_bf16(x[4])) | (static_cast<uint32_t>(f32_to_bf16(x[5])) << 16);
  f.v.w = static_cast<uint32_t>(f32_to_bf16(x[6])) | (static_cast<uint32_t>(f32_to_bf16(x[7])) << 16);
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

template <typename T, int D, int NQ>
__global__ __launch_bounds__(256) void block_attn_kernel(AttnArgs p) {
  constexpr int DS = D / 32;   // 32-wide k steps over the head dimension
  constexpr int DT = D / 16;   // 16-row tiles of O^T
  constexpr int QR = NQ * 16;  // query rows (padded)
  __shared__ float s_m[4][QR], s_l[4][QR];
  __shared__ float s_o[QR][D + 4];

  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int B = p.B, G = p.G, GB = G * B;
  const int n_keys = p.seq.len[b] + B;
  const int kbeg = c * p.chunk;
  if (kbeg >= n_keys) return;
  const int kend = min(kbeg + p.chunk, n_keys);
  const int n_chunks_b = (n_keys + p.chunk - 1) / p.chunk;
  const int64_t base = p.seq.off[b];
  const T* Kg = static_cast<const T*>(p.kc) + static_cast<int64_t>(g) * p.cap * D;
  const T* Vg = static_cast<const T*>(p.vc) + static_cast<int64_t>(g) * D * p.cap;
  const T* q = static_cast<const T*>(p.q);

  Frag8<T> qf[NQ][DS];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int r = qt * 16 + r16;
    if (r < GB) {
      const int h = r / B, j = r % B;
      const T* qrow = q + static_cast<int64_t>(b * B + j) * p.ldq + (g * G + h) * D;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) ld_frag(qf[qt][ds], qrow + ds * 32 + kg * 8);
    } else {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) zero_frag(qf[qt][ds]);
    }
  }

  float m_run[NQ], l_run[NQ];
  f32x4 o[DT][NQ];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    m_run[qt] = -1e30f;
    l_run[qt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][qt] = zero4();
  }

  for (int kb = kbeg + wave * 32; kb < kend; kb += 128) {
    Frag8<T> kf[2][DS];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int key = min(kb + (r16 >> 2) * 8 + t * 4 + (r16 & 3), n_keys - 1);
      const T* krow = Kg + (base + key) * D + kg * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) ld_frag(kf[t][ds], krow + ds * 32);
    }
    Frag8<T> vf[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      ld_frag(vf[dt], Vg + static_cast<int64_t>(dt * 16 + r16) * p.cap + base + kb + kg * 8);
    if (kb + 32 > kend) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) mask_tail(vf[dt], kb + kg * 8, kend);
    }
#pragma unroll
    for (int qt = 0; qt < NQ; ++qt) {
      f32x4 s0 = zero4(), s1 = zero4();
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        s0 = mfma16(s0, kf[0][ds], qf[qt][ds]);
        s1 = mfma16(s1, kf[1][ds], qf[qt][ds]);
      }
      // this lane: query qt*16 + r16, keys kb + kg*8 + e, e = t*4 + jj
      float x[8];
      float mx = m_run[qt];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = (e < 4 ? s0[e] : s1[e - 4]) * p.scale_log2;
        if (kb + kg * 8 + e >= kend) v = -INFINITY;
        x[e] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float alpha = exp2f(m_run[qt] - mx);
      m_run[qt] = mx;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = exp2f(x[e] - mx);
        ls += x[e];
      }
      l_run[qt] = l_run[qt] * alpha + ls;
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
        o[dt][qt] = o[dt][qt] * alpha;
        o[dt][qt] = mfma16(o[dt][qt], vf[dt], pf);
        if (kSplitP) o[dt][qt] = mfma16(o[dt][qt], vf[dt], pl);
      }
    }
  }

  // ---- waves of this workgroup meet in LDS
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    float l = l_run[qt];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (kg == 0) {
      s_m[wave][qt * 16 + r16] = m_run[qt];
      s_l[wave][qt * 16 + r16] = l;
    }
  }
  __syncthreads();
  float scale_w[NQ];
#pragma unroll
  for (int qt = 0; qt < NQ; ++qt) {
    const int r = qt * 16 + r16;
    const float M = fmaxf(fmaxf(s_m[0][r], s_m[1][r]), fmaxf(s_m[2][r], s_m[3][r]));
    scale_w[qt] = exp2f(m_run[qt] - M);
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float& dst = s_o[qt * 16 + r16][dt * 16 + kg * 4 + jj];
            const float v = o[dt][qt][jj] * scale_w[qt];
            dst = (w == 0) ? v : dst + v;
          }
    }
    __syncthreads();
  }

  const int t = threadIdx.x;
  T* out = static_cast<T*>(p.o);
  if (n_chunks_b == 1) {
    for (int e = t; e < GB * D; e += 256) {
      const int r = e / D, dd = e % D;
      const float M = fmaxf(fmaxf(s_m[0][r], s_m[1][r]), fmaxf(s_m[2][r], s_m[3][r]));
      const float L = s_l[0][r] * exp2f(s_m[0][r] - M) + s_l[1][r] * exp2f(s_m[1][r] - M) +
                      s_l[2][r] * exp2f(s_m[2][r] - M) + s_l[3][r] * exp2f(s_m[3][r] - M);
      const int h = r / B, j = r % B;
      stf(out + static_cast<int64_t>(b * B + j) * p.ldq + (g * G + h) * D + dd, s_o[r][dd] / L);
    }
    return;
  }

  // ---- several chunks: publish this chunk's (unnormalised O, max, sum); the
  // merge kernel combines the chunks of a (sequence, kv head) in chunk order
  const int64_t slot = (static_cast<int64_t>(b) * p.n_kv + g) * p.max_chunks;
  float* po = p.part_o + (slot + c) * (QR * D);
  float2* pml = p.part_ml + (slot + c) * QR;
  for (int e = t; e < GB * D; e += 256) po[e] = s_o[e / D][e % D];
  for (int r = t; r < GB; r += 256) {
    const float M = fmaxf(fmaxf(s_m[0][r], s_m[1][r]), fmaxf(s_m[2][r], s_m[3][r]));
    const float L = s_l[0][r] * exp2f(s_m[0][r] - M) + s_l[1][r] * exp2f(s_m[1][r] - M) +
                    s_l[2][r] * exp2f(s_m[2][r] - M) + s_l[3][r] * exp2f(s_m[3][r] - M);
    pml[r] = make_float2(M, L);
  }
}

// One workgroup per (row block of 256 output elements, kv head, sequence):
// o = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c over the sequence's chunks.
template <typename T, int D, int QR>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnArgs p) {
  const int g = blockIdx.y, b = blockIdx.z;
  const int B = p.B, G = p.G, GB = G * B;
  const int n_keys = p.seq.len[b] + B;
  const int n_chunks_b = (n_keys + p.chunk - 1) / p.chunk;
  if (n_chunks_b <= 1) return;   // written directly by the attention kernel
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= GB * D) return;
  const int r = e / D, dd = e % D;
  const int64_t slot = (static_cast<int64_t>(b) * p.n_kv + g) * p.max_chunks;
  const float2* ml = p.part_ml + slot * QR + r;
  const float* po = p.part_o + slot * (QR * D) + e;
  // all loads of a group of 8 chunks are issued before they are combined
  constexpr int kU = 8;
  float M = -1e30f, num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < n_chunks_b; c0 += kU) {
    float2 v[kU];
    float o[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = c0 + u < n_chunks_b;
      v[u] = ok ? ml[(c0 + u) * QR] : make_float2(-1e30f, 0.f);
      o[u] = ok ? po[static_cast<int64_t>(c0 + u) * QR * D] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int u = 0; u < kU; ++u) Mn = fmaxf(Mn, v[u].x);
    const float a = exp2f(M - Mn);
    num *= a;
    den *= a;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const float w = exp2f(v[u].x - Mn);
      num += w * o[u];
      den += w * v[u].y;
    }
    M = Mn;
  }
  const int h = r / B, j = r % B;
  stf(static_cast<T*>(p.o) + static_cast<int64_t>(b * B + j) * p.ldq + (g * G + h) * D + dd,
      num / den);
}

template <typename T, int D, int NQ>
static hipError_t launch_attn_nq(const AttnArgs& a, dim3 grid, int batch, hipStream_t st) {
  block_attn_kernel<T, D, NQ><<<grid, 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_chunks <= 1) return e;
  dim3 mgrid((a.G * a.B * D + 255) / 256, a.n_kv, batch);
  attn_merge_kernel<T, D, NQ * 16><<<mgrid, 256, 0, st>>>(a);
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
