// Stochastic drafting and lossless verification (speculative sampling).
//
// The pages: candidates are accepted or rejected by the target's probability
// distribution and a rejected one is resampled, so the output keeps the
// target's distribution (ai-stack.site, "DFlash：基于块扩散的闪存推测解码方法",
// FAQ 4 and the workflow answer's step 3); the rule is the textbook one that
// page points to.  Both distributions are softmax(logits / T) at one
// temperature T > 0.  Every random number is a caller input.
//
//   sample:  draft of slot j >= 1 = argmax_v (z_v / T - log(-log u_v))
//            (Gumbel-max: a draw from softmax(z / T)), lowest index on ties.
//   verify:  draft k (slot k+1, token x) is kept while r_k * p_{k+1}(x) <
//            q_k(x); the first rejected position a draws its token from
//            (q_a - p_{a+1})_+, a fully kept block draws a bonus from q_{B-1}:
//            the smallest column whose cumulative weight exceeds u * total.
//
// Every reduction runs in a fixed order: the result depends only on the inputs.
#include <algorithm>

#include "kernels.h"

namespace dflash {

constexpr int kSampleChunk = 8192;   // columns per workgroup of the chunked passes
struct SArg {
  float v;
  int i;
};

// x[i] = row[c + i] * scale for i < 32 (-inf past V).  With kVec (rows
// 16-byte aligned) and a whole run inside the row: 16-byte loads.
template <typename T, bool kVec>
__device__ __forceinline__ void load_run32(const T* __restrict__ row, int c, int V, float scale,
                                           float* x) {
  constexpr int kPer = 16 / sizeof(T);
  if (kVec && c + 32 <= V) {
#pragma unroll
    for (int i = 0; i < 32; i += kPer) {
      T buf[kPer];
      *reinterpret_cast<uint4*>(buf) = *reinterpret_cast<const uint4*>(row + c + i);
#pragma unroll
      for (int e = 0; e < kPer; ++e) x[i + e] = Store<T>::load(buf[e]) * scale;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = c + i < V ? ldf(row + c + i) * scale : -INFINITY;
  }
}

// ------------------------------------------------------------ Gumbel-max
// Workgroup (chunk, draft row): the best noisy logit of one column chunk;
// thread t takes the 32 columns c0 + 32 t .. +32 (16-byte loads).
template <bool kVec>
__global__ __launch_bounds__(256) void gumbel_chunk_kernel(const float* __restrict__ logits,
                                                          const float* __restrict__ uni, int B,
                                                          int V, float inv_t,
                                                          SArg* __restrict__ part, int n_chunks) {
  const int chunk = blockIdx.x, row = blockIdx.y;    // row = n * (B - 1) + (j - 1)
  const int n = row / (B - 1), j = row % (B - 1) + 1;
  const float* z = logits + (static_cast<int64_t>(n) * B + j) * V;
  const float* u = uni + static_cast<int64_t>(row) * V;
  const int c = chunk * kSampleChunk + threadIdx.x * 32;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  if (c < V) {
    float zs[32], us[32];
    load_run32<float, kVec>(z, c, V, inv_t, zs);
    load_run32<float, kVec>(u, c, V, 1.0f, us);
#pragma unroll
    for (int i = 0; i < 32; ++i) {   // increasing columns: ">" keeps the lowest
      if (c + i >= V) break;
      const float v = zs[i] - __logf(-__logf(us[i]));
      if (v > best) { best = v; bi = c + i; }
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
    part[static_cast<int64_t>(row) * n_chunks + chunk] = SArg{best, bi};
  }
}

// One wave per draft row folds its chunks.
__global__ __launch_bounds__(64) void gumbel_final_kernel(const SArg* __restrict__ part,
                                                         int n_chunks, int32_t* __restrict__ ids) {
  const int row = blockIdx.x, lane = threadIdx.x;
  float best = -INFINITY;
  int bi = 0x7fffffff;
  for (int c = lane; c < n_chunks; c += 64) {
    const SArg q = part[static_cast<int64_t>(row) * n_chunks + c];
    if (better(q.v, q.i, best, bi)) { best = q.v; bi = q.i; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
  }
  if (lane == 0) ids[row] = bi;
}

// ------------------------------------------------------------ verify
// Workgroup (chunk, row, side): (max, sum of exp(x - max)) of x = logits / T
// over one column chunk.  side 0: target rows [N*B][V] (bf16 or fp32); side 1:
// drafter rows (fp32).  Thread t keeps columns c0 + 32 t .. +32 in registers
// (16-byte loads): the chunk's max first, then one exponential per column.
template <typename T, bool kVecT, bool kVecD>
__global__ __launch_bounds__(256) void lse_chunk_kernel(const T* __restrict__ tgt,
                                                       const float* __restrict__ drf, int V,
                                                       float inv_t, float2* __restrict__ part,
                                                       int rows, int n_chunks) {
  const int chunk = blockIdx.x, row = blockIdx.y, side = blockIdx.z, t = threadIdx.x;
  const int c = chunk * kSampleChunk + t * 32;
  float x[32];
  if (c >= V) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = -INFINITY;
  } else if (side == 0) {
    load_run32<T, kVecT>(tgt + static_cast<int64_t>(row) * V, c, V, inv_t, x);
  } else {
    load_run32<float, kVecD>(drf + static_cast<int64_t>(row) * V, c, V, inv_t, x);
  }
  __shared__ float red[4];
  float m = x[0];
#pragma unroll
  for (int i = 1; i < 32; ++i) m = fmaxf(m, x[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));   // chunk max (finite: c0 < V)
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) s += expf(x[i] - m);
  s = wave_sum(s);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  if (t == 0)
    part[(static_cast<int64_t>(side) * rows + row) * n_chunks + chunk] =
        make_float2(m, (red[0] + red[1]) + (red[2] + red[3]));
}

// Per sequence, the outcome of the accept walk and what the sampling passes need.
struct VerifyRec {
  int a;          // drafts kept
  int resid;      // 1: draw from (q_a - p_{a+1})_+, 0: draw from q_a (bonus)
  float mt, st;   // log-sum-exp parts of target row a (x / T)
  float md, sd;   // ... of drafter row a + 1 (resid only)
};

// One workgroup per sequence, wave j folds the chunks of target row j and
// drafter row j; thread 0 walks the drafts.
template <typename T>
__global__ __launch_bounds__(1024) void verify_walk_kernel(
    const T* __restrict__ tgt, const float* __restrict__ drf, const float2* __restrict__ part,
    int rows, int n_chunks, int B, int V, float inv_t, const int32_t* __restrict__ drafts,
    const float* __restrict__ r, int32_t* __restrict__ accept, VerifyRec* __restrict__ rec) {
  __shared__ float s_mt[16], s_st[16], s_md[16], s_sd[16];
  const int n = blockIdx.x, j = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (j < B) {
#pragma unroll
    for (int side = 0; side < 2; ++side) {
      const float2* pp = part + (static_cast<int64_t>(side) * rows + n * B + j) * n_chunks;
      float m = -INFINITY, s = 0.f;
      for (int c = lane; c < n_chunks; c += 64) lse_merge(m, s, pp[c].x, pp[c].y);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(m, o, 64), os = __shfl_xor(s, o, 64);
        lse_merge(m, s, om, os);
      }
      if (lane == 0) {
        if (side == 0) { s_mt[j] = m; s_st[j] = s; }
        else { s_md[j] = m; s_sd[j] = s; }
      }
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int32_t* d = drafts + static_cast<int64_t>(n) * (B - 1);
  const float* rr = r + static_cast<int64_t>(n) * (B - 1);
  int a = 0;
  while (a < B - 1) {
    const int x = d[a];
    const float q = expf(ldf(tgt + (static_cast<int64_t>(n) * B + a) * V + x) * inv_t - s_mt[a]) / s_st[a];
    const float p = expf(drf[(static_cast<int64_t>(n) * B + a + 1) * V + x] * inv_t - s_md[a + 1]) /
                    s_sd[a + 1];
    if (rr[a] * p < q) ++a;
    else break;
  }
  accept[n] = a;
  VerifyRec v;
  v.a = a;
  v.resid = a < B - 1 ? 1 : 0;
  v.mt = s_mt[a];
  v.st = s_st[a];
  v.md = v.resid ? s_md[a + 1] : 0.f;
  v.sd = v.resid ? s_sd[a + 1] : 1.f;
  rec[n] = v;
}

// Weight of column c of sequence n's sampling row (see VerifyRec), from the
// scaled logits xt (target row a) and xd (drafter row a + 1).
__device__ __forceinline__ float sample_weight_x(const VerifyRec& v, float xt, float xd) {
  const float q = expf(xt - v.mt) / v.st;
  if (!v.resid) return q;
  return fmaxf(q - expf(xd - v.md) / v.sd, 0.f);
}
template <typename T>
__device__ __forceinline__ float sample_weight(const T* __restrict__ tgt,
                                               const float* __restrict__ drf, const VerifyRec& v,
                                               int n, int B, int V, float inv_t, int c) {
  const float xt = ldf(tgt + (static_cast<int64_t>(n) * B + v.a) * V + c) * inv_t;
  const float xd = v.resid ? drf[(static_cast<int64_t>(n) * B + v.a + 1) * V + c] * inv_t : 0.f;
  return sample_weight_x(v, xt, xd);
}

// Sum of the weights of the 32 columns c .. c + 32 (past V: 0), in column
// order; the 256 of a chunk are then added in thread order.  Both sampling
// passes use this order.
template <typename T, bool kVecT, bool kVecD>
__device__ __forceinline__ float thread_run_sum(const T* tgt, const float* drf,
                                                const VerifyRec& v, int n, int B, int V,
                                                float inv_t, int c) {
  float xt[32], xd[32];
  load_run32<T, kVecT>(tgt + (static_cast<int64_t>(n) * B + v.a) * V, c, V, inv_t, xt);
  if (v.resid) load_run32<float, kVecD>(drf + (static_cast<int64_t>(n) * B + v.a + 1) * V, c, V,
                                        inv_t, xd);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (c + i < V) s += sample_weight_x(v, xt[i], v.resid ? xd[i] : 0.f);
  return s;
}

// Workgroup (chunk, sequence): total weight of the chunk.
template <typename T, bool kVecT, bool kVecD>
__global__ __launch_bounds__(256) void sample_sum_kernel(const T* __restrict__ tgt,
                                                        const float* __restrict__ drf,
                                                        const VerifyRec* __restrict__ rec, int B,
                                                        int V, float inv_t,
                                                        float* __restrict__ csum, int n_chunks) {
  __shared__ float sv[256];
  const int chunk = blockIdx.x, n = blockIdx.y, t = threadIdx.x;
  const VerifyRec v = rec[n];
  const int c0 = chunk * kSampleChunk + t * 32;
  sv[t] = c0 < V ? thread_run_sum<T, kVecT, kVecD>(tgt, drf, v, n, B, V, inv_t, c0) : 0.f;
  __syncthreads();
  if (t == 0) {
    float s = 0.f;
    for (int i = 0; i < 256; ++i) s += sv[i];
    csum[static_cast<int64_t>(n) * n_chunks + chunk] = s;
  }
}

// One workgroup per sequence: the chunk where the running total passes
// u * total, then the thread run, then the column.  A target past every
// column of the chosen chunk (rounding between the two passes) takes the
// chunk's last column of positive weight.
template <typename T, bool kVecT, bool kVecD>
__global__ __launch_bounds__(256) void sample_pick_kernel(const T* __restrict__ tgt,
                                                         const float* __restrict__ drf,
                                                         const VerifyRec* __restrict__ rec, int B,
                                                         int V, float inv_t,
                                                         const float* __restrict__ csum,
                                                         int n_chunks, const float* __restrict__ u,
                                                         int32_t* __restrict__ next_tok) {
  __shared__ float sv[256];
  __shared__ int s_chunk;
  __shared__ float s_base, s_target;
  const int n = blockIdx.x, t = threadIdx.x;
  const VerifyRec v = rec[n];
  if (t == 0) {
    const float* cs = csum + static_cast<int64_t>(n) * n_chunks;
    float tot = 0.f;
    for (int c = 0; c < n_chunks; ++c) tot += cs[c];
    const float target = u[n] * tot;
    float base = 0.f;
    int chosen = n_chunks - 1;
    for (int c = 0; c < n_chunks; ++c) {
      if (base + cs[c] > target) { chosen = c; break; }
      if (c < n_chunks - 1) base += cs[c];
    }
    // skip trailing empty chunks the fallback could land on
    while (chosen > 0 && cs[chosen] <= 0.f) { --chosen; base -= cs[chosen]; }
    s_chunk = chosen;
    s_base = base;
    s_target = target;
  }
  __syncthreads();
  const int chunk = s_chunk;
  const int c0 = chunk * kSampleChunk + t * 32;
  sv[t] = c0 < V ? thread_run_sum<T, kVecT, kVecD>(tgt, drf, v, n, B, V, inv_t, c0) : 0.f;
  __syncthreads();
  if (t == 0) {
    float acc = s_base;
    int run = -1, last_pos = -1;
    for (int i = 0; i < 256; ++i) {
      if (sv[i] > 0.f) last_pos = i;
      if (run < 0 && acc + sv[i] > s_target) run = i;
      if (run < 0) acc += sv[i];
    }
    int col = -1;
    if (run >= 0) {
      const int r0 = chunk * kSampleChunk + run * (kSampleChunk / 256);
      const int r1 = min(V, r0 + kSampleChunk / 256);
      float a2 = acc;
      int lastc = -1;
      for (int c = r0; c < r1; ++c) {
        const float w = sample_weight(tgt, drf, v, n, B, V, inv_t, c);
        if (w > 0.f) lastc = c;
        if (a2 + w > s_target) { col = c; break; }
        a2 += w;
      }
      if (col < 0) col = lastc;
    }
    if (col < 0 && last_pos >= 0) {   // rounding left the target past the chunk
      const int r0 = chunk * kSampleChunk + last_pos * (kSampleChunk / 256);
      const int r1 = min(V, r0 + kSampleChunk / 256);
      for (int c = r0; c < r1; ++c)
        if (sample_weight(tgt, drf, v, n, B, V, inv_t, c) > 0.f) col = c;
    }
    next_tok[n] = col < 0 ? 0 : col;
  }
}

size_t stochastic_ws_bytes(int batch, int B, int V) {
  const size_t nc = (static_cast<size_t>(V) + kSampleChunk - 1) / kSampleChunk;
  const size_t gumbel = static_cast<size_t>(batch) * (B - 1) * nc * sizeof(SArg);
  const size_t verify = 2 * static_cast<size_t>(batch) * B * nc * sizeof(float2) +
                        static_cast<size_t>(batch) * nc * sizeof(float) +
                        static_cast<size_t>(batch) * sizeof(VerifyRec) + 256;
  return std::max(gumbel, verify);
}

hipError_t launch_sample_drafts(const float* logits, int batch, int B, int V, float temperature,
                                const float* uniforms, int32_t* ids, void* ws, hipStream_t st) {
  const int nc = (V + kSampleChunk - 1) / kSampleChunk;
  SArg* part = static_cast<SArg*>(ws);
  const bool vec = V % 4 == 0;   // fp32 rows 16-byte aligned
  if (vec)
    gumbel_chunk_kernel<true><<<dim3(nc, batch * (B - 1)), 256, 0, st>>>(
        logits, uniforms, B, V, 1.0f / temperature, part, nc);
  else
    gumbel_chunk_kernel<false><<<dim3(nc, batch * (B - 1)), 256, 0, st>>>(
        logits, uniforms, B, V, 1.0f / temperature, part, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gumbel_final_kernel<<<batch * (B - 1), 64, 0, st>>>(part, nc, ids);
  return hipGetLastError();
}

template <typename T>
static hipError_t verify_stochastic_t(const T* tgt, const float* drf, const int32_t* drafts,
                                      int batch, int B, int V, float temperature, const float* r,
                                      const float* u, int32_t* accept, int32_t* next_tok,
                                      void* ws, hipStream_t st) {
  const int nc = (V + kSampleChunk - 1) / kSampleChunk, rows = batch * B;
  const float inv_t = 1.0f / temperature;
  char* w = static_cast<char*>(ws);
  float2* part = reinterpret_cast<float2*>(w);
  w += 2 * static_cast<size_t>(rows) * nc * sizeof(float2);
  float* csum = reinterpret_cast<float*>(w);
  w += static_cast<size_t>(batch) * nc * sizeof(float);
  w = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(w) + 15) & ~uintptr_t{15});
  VerifyRec* rec = reinterpret_cast<VerifyRec*>(w);
  // 16-byte loads when both row strides keep 16-byte alignment
  const bool vec = (static_cast<size_t>(V) * sizeof(T)) % 16 == 0 && V % 4 == 0;
  if (vec)
    lse_chunk_kernel<T, true, true><<<dim3(nc, rows, 2), 256, 0, st>>>(tgt, drf, V, inv_t, part,
                                                                       rows, nc);
  else
    lse_chunk_kernel<T, false, false><<<dim3(nc, rows, 2), 256, 0, st>>>(tgt, drf, V, inv_t, part,
                                                                         rows, nc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  verify_walk_kernel<T><<<batch, 64 * B, 0, st>>>(tgt, drf, part, rows, nc, B, V, inv_t, drafts,
                                                  r, accept, rec);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (vec) {
    sample_sum_kernel<T, true, true><<<dim3(nc, batch), 256, 0, st>>>(tgt, drf, rec, B, V, inv_t,
                                                                      csum, nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    sample_pick_kernel<T, true, true><<<batch, 256, 0, st>>>(tgt, drf, rec, B, V, inv_t, csum, nc,
                                                             u, next_tok);
  } else {
    sample_sum_kernel<T, false, false><<<dim3(nc, batch), 256, 0, st>>>(tgt, drf, rec, B, V,
                                                                        inv_t, csum, nc);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    sample_pick_kernel<T, false, false><<<batch, 256, 0, st>>>(tgt, drf, rec, B, V, inv_t, csum,
                                                               nc, u, next_tok);
  }
  return hipGetLastError();
}

hipError_t launch_verify_stochastic(const void* target_logits, bool bf16, const float* draft_logits,
                                    const int32_t* drafts, int batch, int B, int V,
                                    float temperature, const float* r, const float* u,
                                    int32_t* accept, int32_t* next_tok, void* ws, hipStream_t st) {
  if (bf16)
    return verify_stochastic_t(static_cast<const uint16_t*>(target_logits), draft_logits, drafts,
                               batch, B, V, temperature, r, u, accept, next_tok, ws, st);
  return verify_stochastic_t(static_cast<const float*>(target_logits), draft_logits, drafts, batch,
                             B, V, temperature, r, u, accept, next_tok, ws, st);
}

}  // namespace dflash
