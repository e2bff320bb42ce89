// Small memory-bound kernels of the drafter pass: block embedding, residual
// RMSNorm, the QKV finish of batched blocks, LM-head argmax finalize and
// greedy verification.
#include <algorithm>
#include "kernels.h"

namespace dflash {

// ------------------------------------------------------------------ embed
// One workgroup per block slot m = b*B + j.  Slot 0 of a block holds the anchor
// (the previous cycle's bonus token), the others the mask token (zhichai.net,
// "DFlash 的架构密码", 训练策略 1: every block starts at a verified token).
// The shared target embedding supplies the rows (same page, 训练策略 3).
template <typename T, int PER>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ embed, int H, int V,
                                                    const int32_t* __restrict__ anchors,
                                                    int mask_id, int B, float* __restrict__ x,
                                                    const T* __restrict__ gain,
                                                    T* __restrict__ u, float eps, int frag) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int b = m / B, j = m % B;
  // an anchor outside [0, V) is clamped into range rather than read out of bounds
  const int tok = (j == 0) ? min(max(anchors[b], 0), V - 1) : mask_id;
  const T* src = embed + static_cast<size_t>(tok) * H;
  float* dst = x + static_cast<size_t>(m) * H;
  float v[PER][4];
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = (q * 256 + threadIdx.x) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[q][e] = (c < H) ? ldf(src + c + e) : 0.f;
      ss += v[q][e] * v[q][e];
    }
    if (c < H) *reinterpret_cast<float4*>(dst + c) = make_float4(v[q][0], v[q][1], v[q][2], v[q][3]);
  }
  // the first layer's attention RMSNorm of this row (gains loaded before the
  // reduction, so their latency overlaps it)
  float4 gq[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = (q * 256 + threadIdx.x) * 4;
    gq[q] = c < H ? ld4(gain + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = (q * 256 + threadIdx.x) * 4;
    if (c < H) {
      // four columns of one aligned run of 32: contiguous in either layout
      T* o = u + (frag ? frag_major(m, c, H) : static_cast<int64_t>(m) * H + c);
      st4(o, make_float4(v[q][0] * r * gq[q].x, v[q][1] * r * gq[q].y, v[q][2] * r * gq[q].z,
                         v[q][3] * r * gq[q].w));
    }
  }
}

hipError_t launch_embed(bool bf16, const void* embed, int H, int V, const int32_t* anchors,
                        int mask_id, int batch, int B, float* x, const void* gain, void* u,
                        float eps, hipStream_t st, bool frag) {
  if (H > 8192 || H % 4 || (frag && H % 32)) return hipErrorInvalidValue;
  dim3 grid(batch * B), block(256);
  const int per = (H + 1023) / 1024;
#define DF_EMB(TT, P)                                                                          \
  embed_kernel<TT, P><<<grid, block, 0, st>>>(static_cast<const TT*>(embed), H, V, anchors,    \
                                              mask_id, B, x,                                   \
                                              static_cast<const TT*>(gain), static_cast<TT*>(u), \
                                              eps, frag ? 1 : 0)
  if (bf16) {
    if (per <= 1) DF_EMB(uint16_t, 1); else if (per <= 2) DF_EMB(uint16_t, 2);
    else if (per <= 4) DF_EMB(uint16_t, 4); else DF_EMB(uint16_t, 8);
  } else {
    if (per <= 1) DF_EMB(float, 1); else if (per <= 2) DF_EMB(float, 2);
    else if (per <= 4) DF_EMB(float, 4); else DF_EMB(float, 8);
  }
#undef DF_EMB
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// Row m: v = x[m] (if x) + sum over splits s of part[s][m] (in split order);
// x[m] = v (if x); out[m] = v / sqrt(mean(v^2) + eps) * g (if out; row-major,
// or fragment-major for a weight-streaming GEMM that reads it next).
// The split-K partials of the producing GEMM meet here, together with the
// residual add, so no GEMM has to wait on another workgroup.  RMSNorm:
// zhichai.net, "DFlash 的架构密码", 技术细节补充 / 投影层 for the fusion norm;
// the same form for the layer norms.  One workgroup per row, H <= 8192,
// float32 statistics with a fixed reduction order.
template <typename T, int PER, int NS>
__global__ __launch_bounds__(256) void resid_rmsnorm_kernel(float* __restrict__ x,
                                                            const float* __restrict__ part,
                                                            int n_split, int64_t split_stride,
                                                            const T* __restrict__ gain,
                                                            T* __restrict__ out, int H, float eps,
                                                            int frag) {
  __shared__ float red[4];
  const int m = blockIdx.x;
  constexpr int kMaxSplit = NS;
  // every load of the row is issued before any arithmetic (latency-bound)
  float4 v[PER];
  float4 p[kMaxSplit][PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = (q * 256 + threadIdx.x) * 4;
    v[q] = (x && c < H) ? *reinterpret_cast<const float4*>(x + static_cast<int64_t>(m) * H + c)
                        : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s)
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int c = (q * 256 + threadIdx.x) * 4;
      p[s][q] = (s < n_split && c < H)
                    ? *reinterpret_cast<const float4*>(part + s * split_stride +
                                                      static_cast<int64_t>(m) * H + c)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    float4 a = v[q];
#pragma unroll
    for (int s = 0; s < kMaxSplit; ++s) {
      a.x += p[s][q].x; a.y += p[s][q].y; a.z += p[s][q].z; a.w += p[s][q].w;
    }
    v[q] = a;
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    const int c = (q * 256 + threadIdx.x) * 4;
    if (x && n_split > 0 && c < H)
      *reinterpret_cast<float4*>(x + static_cast<int64_t>(m) * H + c) = a;
  }
  if (!out) return;
  float4 gq[PER];   // gains, loaded before the reduction
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = (q * 256 + threadIdx.x) * 4;
    gq[q] = c < H ? ld4(gain + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float r = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int c = (q * 256 + threadIdx.x) * 4;
    if (c < H) {
      T* o = out + (frag ? frag_major(m, c, H) : static_cast<int64_t>(m) * H + c);
      st4(o, make_float4(v[q].x * r * gq[q].x, v[q].y * r * gq[q].y, v[q].z * r * gq[q].z,
                         v[q].w * r * gq[q].w));
    }
  }
}

template <typename T>
static hipError_t launch_rn(float* x, const float* part, int n_split, int64_t split_stride,
                            const void* gain, void* out, int rows, int H, float eps,
                            hipStream_t st, int frag) {
  const T* g = static_cast<const T*>(gain);
  T* o = static_cast<T*>(out);
  const int per = (H + 1023) / 1024;
#define DF_RN(P, S) resid_rmsnorm_kernel<T, P, S><<<rows, 256, 0, st>>>(x, part, n_split, split_stride, g, o, H, eps, frag)
  if (n_split <= 4) {
    if (per <= 1) DF_RN(1, 4);
    else if (per <= 2) DF_RN(2, 4);
    else if (per <= 4) DF_RN(4, 4);
    else DF_RN(8, 4);
  } else {
    if (per <= 1) DF_RN(1, 8);
    else if (per <= 2) DF_RN(2, 8);
    else if (per <= 4) DF_RN(4, 8);
    else return hipErrorInvalidValue;
  }
#undef DF_RN
  return hipGetLastError();
}

hipError_t launch_resid_rmsnorm(bool bf16, float* x, const float* part, int n_split,
                                int64_t split_stride, const void* gain, void* out, int rows,
                                int H, float eps, hipStream_t st, bool frag) {
  if (rows <= 0) return hipSuccess;
  if (H > 8192 || H % 4 || n_split > 8 || (frag && H % 32)) return hipErrorInvalidValue;
  const int f = frag ? 1 : 0;
  return bf16 ? launch_rn<uint16_t>(x, part, n_split, split_stride, gain, out, rows, H, eps, st, f)
              : launch_rn<float>(x, part, n_split, split_stride, gain, out, rows, H, eps, st, f);
}

// ------------------------------------------------------------------ LM-head argmax
// Row m (block slot j = m % B >= 1): fold the per-workgroup (value, lowest
// column) partials of the LM-head GEMM into the draft id of that slot.
__global__ __launch_bounds__(256) void lm_argmax_finalize_kernel(const float2* __restrict__ part,
                                                                 int n_wg, int B,
                                                                 const int32_t* __restrict__ anchors,
                                                                 int V,
                                                                 int32_t* __restrict__ draft) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int m = blockIdx.x, j = m % B;
  if (j == 0) return;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  const float2* pr = part + static_cast<int64_t>(m) * n_wg;
  constexpr int kU = 8;
  for (int w0 = threadIdx.x; w0 < n_wg; w0 += 256 * kU) {
    float2 q[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int w = w0 + u * 256;
      q[u] = w < n_wg ? pr[w] : make_float2(-INFINITY, __int_as_float(0x7fffffff));
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int qi = __float_as_int(q[u].y);
      if (better(q[u].x, qi, best, bi)) { best = q[u].x; bi = qi; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
  }
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], best, bi)) { best = sv[w]; bi = si[w]; }
    // a block whose anchor lies outside [0, V) was embedded from a clamped
    // row; its drafts are refused (-1) rather than passed off as a draft
    const int32_t a = anchors ? anchors[m / B] : 0;
    draft[(m / B) * (B - 1) + (j - 1)] = (a >= 0 && a < V) ? bi : -1;
  }
}

// ------------------------------------------------------------ training loss
// Row m (slot j = m % B >= 1 of block m / B): fold the per-workgroup
// (max, sum, label logit) partials of the LM head into the slot's
// cross-entropy  log(sum_v exp(z_v)) - z_label  (zhichai.net, "DFlash 的架构
// 密码", 训练策略 2: the loss of the draft slots).  Fixed fold order.
__global__ __launch_bounds__(256) void lm_loss_finalize_kernel(const float4* __restrict__ part,
                                                               int n_wg, int B,
                                                               float* __restrict__ slot_loss) {
  __shared__ float sm_m[4], sm_s[4], sm_z[4];
  const int m = blockIdx.x, j = m % B;
  if (j == 0) return;
  float mx = -INFINITY, sm = 0.f, zl = -INFINITY;
  const float4* pr = part + static_cast<int64_t>(m) * n_wg;
  constexpr int kU = 8;
  for (int w0 = threadIdx.x; w0 < n_wg; w0 += 256 * kU) {
    float4 q[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int w = w0 + u * 256;
      q[u] = w < n_wg ? pr[w] : make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      lse_merge(mx, sm, q[u].x, q[u].y);
      zl = fmaxf(zl, q[u].z);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(mx, o, 64), os = __shfl_xor(sm, o, 64);
    zl = fmaxf(zl, __shfl_xor(zl, o, 64));
    lse_merge(mx, sm, om, os);
  }
  if ((threadIdx.x & 63) == 0) {
    sm_m[threadIdx.x >> 6] = mx;
    sm_s[threadIdx.x >> 6] = sm;
    sm_z[threadIdx.x >> 6] = zl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w) {
      lse_merge(mx, sm, sm_m[w], sm_s[w]);
      zl = fmaxf(zl, sm_z[w]);
    }
    slot_loss[(m / B) * (B - 1) + (j - 1)] = mx + logf(sm) - zl;
  }
}

// loss = sum w_j * slot_loss / sum w_j over every scored slot of n_blocks
// blocks, w_j = exp(-(j-1)/gamma) for slot j = 1..B-1 (zhichai.net, "DFlash
// 的架构密码", 训练策略 2: earlier slots weigh more).  One workgroup, fixed
// order.
__global__ __launch_bounds__(256) void loss_reduce_kernel(const float* __restrict__ slot_loss,
                                                          int n, int B, float inv_gamma,
                                                          float* __restrict__ loss) {
  __shared__ float sa[4], sb[4];
  float a = 0.f, wsum = 0.f;
  for (int e = threadIdx.x; e < n * (B - 1); e += 256) {
    const int k = e % (B - 1);   // slot j = k + 1
    const float w = expf(-static_cast<float>(k) * inv_gamma);
    a += w * slot_loss[e];
    wsum += w;
  }
  a = wave_sum(a);
  wsum = wave_sum(wsum);
  if ((threadIdx.x & 63) == 0) {
    sa[threadIdx.x >> 6] = a;
    sb[threadIdx.x >> 6] = wsum;
  }
  __syncthreads();
  if (threadIdx.x == 0) loss[0] = ((sa[0] + sa[1]) + (sa[2] + sa[3])) / ((sb[0] + sb[1]) + (sb[2] + sb[3]));
}

hipError_t launch_lm_loss(const float4* part, int n_wg, int rows, int B, float gamma,
                          float* slot_loss, float* loss, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  lm_loss_finalize_kernel<<<rows, 256, 0, st>>>(part, n_wg, B, slot_loss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  loss_reduce_kernel<<<1, 256, 0, st>>>(slot_loss, rows / B, B, 1.0f / gamma, loss);
  return hipGetLastError();
}

// ------------------------------------------------------------ QKV finish
// Block row m = b * B + j of a batch whose QKV projection left ks fp32
// partial slabs [ks][M][qd + 2 kvd]: sum the slabs, rotate q and k at the
// block position len[b] + j (pairs (c, c + d/2) of a head), store q to its
// buffer and k, v to the layer's cache at row off[b] + len[b] + j (V
// transposed; with block_rows, to rows b * kTrainSlab + j of a training
// layout's block buffer instead).
//   - q/k part: the first rows * ry workgroups, ry per row splitting its
//     rotation pairs (few rows still spread over the GPU);
//   - v part: one workgroup per (block, 64 value columns).  The transposed V
//     cache keeps a column's positions contiguous, so the tile goes through
//     LDS: loaded along columns (coalesced slab reads), stored along the
//     block's slots (one 32-byte run per column for B = 16) instead of one
//     scattered 2-byte store per value.
constexpr int kQkvMaxSplit = 8;   // K-split slabs the finishing kernel sums
constexpr int kQkvVCols = 64;     // value columns per v-part workgroup
template <typename T>
__global__ __launch_bounds__(256) void qkv_finish_kernel(const float* __restrict__ part, int ks,
                                                         int64_t slab, int qd, int kvd, int d,
                                                         int B, int rows, int ry,
                                                         T* __restrict__ q, int64_t ldq,
                                                         T* __restrict__ kc, T* __restrict__ vc,
                                                         int64_t cap, RopeFreq freq, SeqTable seq,
                                                         bool block_rows) {
  const int nq = qd + 2 * kvd, half = d / 2;
  const int wg = blockIdx.x;
  if (wg < rows * ry) {
    const int m = wg / ry, yy = wg % ry, b = m / B, j = m % B;
    const int pos = seq_len_of(seq, b) + j;
    // training layout: the block's K/V go to its own rows of the block buffer
    const int64_t row = block_rows ? static_cast<int64_t>(b) * kTrainSlab + j : seq.off[b] + pos;
    const float* pr = part + static_cast<int64_t>(m) * nq;
    const int n_pairs = (qd + kvd) / 2;   // rotation pairs of [q heads | k heads]
    for (int p = yy * 256 + threadIdx.x; p < n_pairs; p += ry * 256) {
      const int c = p % half, col = (p / half) * d + c;
      // every slab's value is loaded before the sums (in slab order) start
      float a0[kQkvMaxSplit], a1[kQkvMaxSplit];
#pragma unroll
      for (int s2 = 0; s2 < kQkvMaxSplit; ++s2) {
        a0[s2] = s2 < ks ? pr[s2 * slab + col] : 0.f;
        a1[s2] = s2 < ks ? pr[s2 * slab + col + half] : 0.f;
      }
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < kQkvMaxSplit; ++s2)
        if (s2 < ks) {
          x0 += a0[s2];
          x1 += a1[s2];
        }
      float cs, sn;
      rope_cos_sin(pos, c, freq, cs, sn);
      T* dst = col < qd ? q + static_cast<int64_t>(m) * ldq + col
                        : kc + (static_cast<int64_t>((col - qd) / d) * cap + row) * d + c;
      stf(dst, x0 * cs - x1 * sn);
      stf(dst + half, x1 * cs + x0 * sn);
    }
    return;
  }
  // v part: block b, value columns [c0, c0 + 64)
  __shared__ float tile[16][kQkvVCols + 1];
  const int vt = wg - rows * ry, n_ct = (kvd + kQkvVCols - 1) / kQkvVCols;
  const int b = vt / n_ct, c0 = (vt % n_ct) * kQkvVCols;
  const int t = threadIdx.x;
  {
    const int col = t % kQkvVCols, jr = t / kQkvVCols;   // 4 slots per pass
    for (int j = jr; j < B; j += 256 / kQkvVCols) {
      float x = 0.f;
      if (c0 + col < kvd) {
        const float* pr = part + static_cast<int64_t>(b * B + j) * nq + qd + kvd + c0 + col;
        float a[kQkvMaxSplit];
#pragma unroll
        for (int s2 = 0; s2 < kQkvMaxSplit; ++s2) a[s2] = s2 < ks ? pr[s2 * slab] : 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kQkvMaxSplit; ++s2)
          if (s2 < ks) x += a[s2];
      }
      tile[j][col] = x;
    }
  }
  __syncthreads();
  const int64_t row0 = block_rows ? static_cast<int64_t>(b) * kTrainSlab
                                  : seq.off[b] + seq_len_of(seq, b);
  const int j = t % 16, cr = t / 16;   // 16 columns per pass
  if (j < B)
    for (int col = cr; col < kQkvVCols && c0 + col < kvd; col += 16)
      stf(vc + static_cast<int64_t>(c0 + col) * cap + row0 + j, tile[j][col]);
}

hipError_t launch_qkv_finish(bool bf16, const float* part, int ks, int64_t slab, int rows, int qd,
                             int kvd, int d, int B, void* q, int64_t ldq, void* kc, void* vc,
                             int64_t cap, const RopeFreq& freq, const SeqTable& seq,
                             hipStream_t st, bool block_rows) {
  if (rows <= 0) return hipSuccess;
  if (ks < 1 || ks > kQkvMaxSplit || B > 16 || rows % B) return hipErrorInvalidValue;
  // enough q/k workgroups to cover the GPU when rows are few
  const int n_pairs = (qd + kvd) / 2;
  const int ry = std::max(1, std::min((n_pairs + 255) / 256, 1024 / rows));
  const int n_vwg = (rows / B) * ((kvd + kQkvVCols - 1) / kQkvVCols);
  const dim3 grid(rows * ry + n_vwg);
  if (bf16)
    qkv_finish_kernel<uint16_t><<<grid, 256, 0, st>>>(
        part, ks, slab, qd, kvd, d, B, rows, ry, static_cast<uint16_t*>(q), ldq,
        static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vc), cap, freq, seq, block_rows);
  else
    qkv_finish_kernel<float><<<grid, 256, 0, st>>>(part, ks, slab, qd, kvd, d, B, rows, ry,
                                                   static_cast<float*>(q), ldq,
                                                   static_cast<float*>(kc),
                                                   static_cast<float*>(vc), cap, freq, seq,
                                                   block_rows);
  return hipGetLastError();
}

hipError_t launch_lm_argmax_finalize(const float2* part, int n_wg, int rows, int B,
                                     const int32_t* anchors, int V, int32_t* draft,
                                     hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  lm_argmax_finalize_kernel<<<rows, 256, 0, st>>>(part, n_wg, B, anchors, V, draft);
  return hipGetLastError();
}

// ------------------------------------------------------------------ verify
// Stage 1: workgroup (row, chunk) finds the largest logit of one column chunk
// of one target row and its lowest column.  Stage 2: one wave per sequence
// combines the chunks of its B rows and scans for the first draft that
// disagrees (zhichai.net, "DFlash 的架构密码", 训练策略 1; ai-stack.site,
// "DFlash：基于块扩散的闪存推测解码方法", 实践 2 and 实践 5).
//
// Stage 1 is a pure stream of the logits: chunks are sized so that the whole
// grid is about one resident round (kVerifyWGs workgroups of 256 threads, 8
// per CU), each thread's 16-byte loads go out in groups of kVerifyBurst
// before any compare, and chunk boundaries are multiples of 8 columns, so a
// 16-byte load never straddles two chunks or the row end when V % 8 == 0.
constexpr int kVerifyWGs = 2048;
constexpr int kVerifyMinChunk = 2048;
constexpr int kVerifyBurst = 2;
struct ArgPart {
  float v;
  int i;
};

// Columns per chunk for `rows` target rows of V columns (a multiple of 8).
static int verify_chunk_cols(int rows, int V) {
  const int target = max(1, (kVerifyWGs + rows - 1) / max(rows, 1));
  int chunk = (V + target - 1) / target;
  chunk = (chunk + 7) / 8 * 8;
  return max(chunk, kVerifyMinChunk);
}

template <typename T, bool kVec>
__global__ __launch_bounds__(256) void verify_chunk_kernel(const T* __restrict__ logits, int V,
                                                           int chunk_cols,
                                                           ArgPart* __restrict__ part,
                                                           int n_chunks) {
  const int row = blockIdx.x / n_chunks, chunk = blockIdx.x - row * n_chunks;
  const T* r = logits + static_cast<int64_t>(row) * V;
  const int c0 = chunk * chunk_cols;
  const int c1 = min(V, c0 + chunk_cols);
  float best = -INFINITY;
  int bi = 0x7fffffff;
  constexpr int kPer = 16 / sizeof(T);
  if (kVec) {
    // every thread walks its columns in increasing order, so ">" keeps the lowest
    for (int cb = c0 + static_cast<int>(threadIdx.x) * kPer; cb < c1;
         cb += 256 * kPer * kVerifyBurst) {
      uint4 buf[kVerifyBurst];
#pragma unroll
      for (int u = 0; u < kVerifyBurst; ++u) {
        const int c = cb + u * 256 * kPer;
        if (c < c1) buf[u] = *reinterpret_cast<const uint4*>(r + c);
      }
#pragma unroll
      for (int u = 0; u < kVerifyBurst; ++u) {
        const int c = cb + u * 256 * kPer;
        if (c < c1) {
          const T* e = reinterpret_cast<const T*>(&buf[u]);
#pragma unroll
          for (int q = 0; q < kPer; ++q) {
            const float v = Store<T>::load(e[q]);
            if (v > best) { best = v; bi = c + q; }
          }
        }
      }
    }
  } else {
    for (int c = c0 + threadIdx.x; c < c1; c += 256) {
      const float v = ldf(r + c);
      if (v > best) { best = v; bi = c; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
  }
  __shared__ float sv[4];
  __shared__ int si[4];
  if ((threadIdx.x & 63) == 0) { sv[threadIdx.x >> 6] = best; si[threadIdx.x >> 6] = bi; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], best, bi)) { best = sv[w]; bi = si[w]; }
    part[blockIdx.x] = ArgPart{best, bi};
  }
}

// One workgroup per sequence, wave j folds the chunks of row j into the
// target's token t_j and compares it with draft j (loaded before the fold, so
// its latency overlaps); thread 0 then counts the leading matches.
__global__ __launch_bounds__(1024) void verify_scan_kernel(const ArgPart* __restrict__ part,
                                                           int n_chunks, int B,
                                                           const int32_t* __restrict__ drafts,
                                                           int32_t* __restrict__ accept,
                                                           int32_t* __restrict__ bonus) {
  __shared__ int s_t[16];
  __shared__ int s_match[16];
  const int b = blockIdx.x, j = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (j < B) {
    const int dj = j < B - 1 ? drafts[static_cast<int64_t>(b) * (B - 1) + j] : -1;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    const ArgPart* p = part + static_cast<int64_t>(b * B + j) * n_chunks;
    for (int c = lane; c < n_chunks; c += 64) {
      const ArgPart q = p[c];
      if (better(q.v, q.i, best, bi)) { best = q.v; bi = q.i; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
    }
    if (lane == 0) {
      s_t[j] = bi;
      s_match[j] = j < B - 1 && bi == dj;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < B - 1 && s_match[a]) ++a;
    accept[b] = a;
    bonus[b] = s_t[a];
  }
}

// rows * n_chunks <= rows * ceil(kVerifyWGs / rows) <= rows + kVerifyWGs, an
// upper bound that grows with the row count (so a workspace sized for the
// largest batch and block serves every smaller call).
size_t verify_ws_bytes(int batch, int B, int V) {
  (void)V;
  return (static_cast<size_t>(batch) * B + kVerifyWGs) * sizeof(ArgPart);
}

hipError_t launch_verify(const void* logits, bool bf16, const int32_t* drafts, int batch, int B,
                         int V, int32_t* accept, int32_t* bonus, void* ws, hipStream_t st) {
  const int rows = batch * B;
  const int chunk = verify_chunk_cols(rows, V);
  const int n_chunks = (V + chunk - 1) / chunk;
  ArgPart* part = static_cast<ArgPart*>(ws);
  const unsigned grid = static_cast<unsigned>(rows) * n_chunks;
  const bool vec = V % 8 == 0;
  if (bf16) {
    auto p = static_cast<const uint16_t*>(logits);
    if (vec) verify_chunk_kernel<uint16_t, true><<<grid, 256, 0, st>>>(p, V, chunk, part, n_chunks);
    else verify_chunk_kernel<uint16_t, false><<<grid, 256, 0, st>>>(p, V, chunk, part, n_chunks);
  } else {
    auto p = static_cast<const float*>(logits);
    if (vec) verify_chunk_kernel<float, true><<<grid, 256, 0, st>>>(p, V, chunk, part, n_chunks);
    else verify_chunk_kernel<float, false><<<grid, 256, 0, st>>>(p, V, chunk, part, n_chunks);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  verify_scan_kernel<<<batch, 64 * B, 0, st>>>(part, n_chunks, B, drafts, accept, bonus);
  return hipGetLastError();
}

// ------------------------------------------------------------------ lengths
// Device-resident step: after the accepted rows of each sequence were
// appended, len[b] += accept[b] + 1 (the anchor and its accepted drafts).  A
// length that would pass len_max stays where it is and sets status[0] = 1, so
// no later kernel of the loop indexes past the capacity the host checked.
__global__ __launch_bounds__(64) void advance_lengths_kernel(int32_t* __restrict__ len,
                                                             const int32_t* __restrict__ accept,
                                                             int n, int B, int len_max,
                                                             int32_t* __restrict__ status) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= n) return;
  const int a = min(max(accept[b], 0), B - 1);
  const int cur = min(max(len[b], 0), len_max);
  const int nl = cur + a + 1;
  if (nl > len_max) {
    status[0] = 1;
    len[b] = cur;
  } else {
    len[b] = nl;
  }
}

hipError_t launch_advance_lengths(int32_t* len, const int32_t* accept, int n, int B, int len_max,
                                  int32_t* status, hipStream_t st) {
  advance_lengths_kernel<<<(n + 63) / 64, 64, 0, st>>>(len, accept, n, B, len_max, status);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bf16 rounding
// The float32 -> bf16 rounding every kernel here stores with, exposed for
// its test: packed = 0 takes the scalar conversion (f32_to_bf16), packed = 1
// the pair conversion (f32x2_to_bf16x2) on elements (2i, 2i+1).
__global__ __launch_bounds__(256) void bf16_round_kernel(const float* __restrict__ in,
                                                         uint16_t* __restrict__ out, int64_t n,
                                                         int packed) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  if (packed) {
    const float2* in2 = reinterpret_cast<const float2*>(in);
    uint32_t* out2 = reinterpret_cast<uint32_t*>(out);
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n / 2; i += stride) {
      const float2 v = in2[i];
      out2[i] = f32x2_to_bf16x2(v.x, v.y);
    }
  } else {
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += stride) out[i] = f32_to_bf16(in[i]);
  }
}

hipError_t launch_bf16_round(const float* in, uint16_t* out, int64_t n, int packed,
                             hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t work = packed ? n / 2 : n;
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((work + 255) / 256, 8192));
  bf16_round_kernel<<<grid, 256, 0, st>>>(in, out, n, packed);
  return hipGetLastError();
}

// Weight packing: a row-major [N, K] bf16 matrix into fragment-major order
// (frag_major(); rows padded with zeros to a multiple of 16), 16 bytes per
// thread: consecutive threads write consecutive bytes of the destination and
// read 64-byte row pieces of the source.
__global__ __launch_bounds__(256) void pack_frag_kernel(const uint16_t* __restrict__ src, int N,
                                                        int K, uint16_t* __restrict__ dst,
                                                        int64_t chunks) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t kb_per_row = K / 32;
  for (int64_t q = blockIdx.x * 256 + threadIdx.x; q < chunks; q += stride) {
    // chunk q = 8 elements at dst[8q]: block q / 64 (16 rows x 32 columns),
    // row (q % 64) / 4 of the block, columns 8 (q % 4) .. + 8
    const int64_t blk = q >> 6;
    const int r = static_cast<int>((q >> 2) & 15), c8 = static_cast<int>(q & 3) * 8;
    const int64_t n = (blk / kb_per_row) * 16 + r;
    const int64_t k = (blk % kb_per_row) * 32 + c8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) v = *reinterpret_cast<const uint4*>(src + n * K + k);
    *reinterpret_cast<uint4*>(dst + q * 8) = v;
  }
}

hipError_t launch_pack_frag(const uint16_t* src, int N, int K, uint16_t* dst, hipStream_t st) {
  if (N <= 0 || K <= 0 || K % 32) return hipErrorInvalidValue;
  const int64_t chunks = static_cast<int64_t>((N + 15) / 16) * 16 * (K / 8);
  const unsigned grid = static_cast<unsigned>(std::min<int64_t>((chunks + 255) / 256, 16384));
  pack_frag_kernel<<<grid, 256, 0, st>>>(src, N, K, dst, chunks);
  return hipGetLastError();
}

}  // namespace dflash
