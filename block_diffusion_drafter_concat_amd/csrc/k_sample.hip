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
// Every exponential of this path (chunk sums, accept tests, sampling weights)
// is the hardware one (exp2 of x * log2 e, relative error ~1e-6 for the
// arguments that matter): with the library exponential the 78 M per-column
// evaluations of a batch-16 call cost as much VALU time as the logits stream.
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
  for (int i = 0; i < 32; ++i) s += __expf(x[i] - m);
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
// drafter row j; thread k tests draft k; thread 0 walks the outcomes.
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
  // every draft's accept test at once (thread k takes draft k; a draft id
  // outside [0, V) is never accepted and its loads use a clamped column), then
  // thread 0 keeps the drafts up to the first rejection
  __shared__ int s_ok[16];
  const int32_t* d = drafts + static_cast<int64_t>(n) * (B - 1);
  const float* rr = r + static_cast<int64_t>(n) * (B - 1);
  if (threadIdx.x < B - 1) {
    const int k = threadIdx.x;
    const int x0 = d[k];
    const int x = min(max(x0, 0), V - 1);
    const float xt = ldf(tgt + (static_cast<int64_t>(n) * B + k) * V + x) * inv_t;
    const float xd = drf[(static_cast<int64_t>(n) * B + k + 1) * V + x] * inv_t;
    const float q = __expf(xt - s_mt[k]) / s_st[k];
    const float p = __expf(xd - s_md[k + 1]) / s_sd[k + 1];
    s_ok[k] = (x0 == x) && (rr[k] * p < q);
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int a = 0;
  while (a < B - 1 && s_ok[a]) ++a;
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
  const float q = __expf(xt - v.mt) / v.st;
  if (!v.resid) return q;
  return fmaxf(q - __expf(xd - v.md) / v.sd, 0.f);
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

// Inclusive prefix sum over the 256 threads of a workgroup in a fixed order:
// a shuffle scan inside each wave, then the totals of the earlier waves added
// left to right.  The chunk total of sample_sum_kernel and the running totals
// of sample_pick_kernel both come from this one routine on the same values,
// so thread 255's result is the chunk total bit for bit.
__device__ __forceinline__ float block_incl_scan256(float x, float* s_wt /* [4] */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) s_wt[w] = x;
  __syncthreads();
  float off = 0.f;
  for (int k = 0; k < w; ++k) off += s_wt[k];
  __syncthreads();
  return off + x;
}

// Workgroup (chunk, sequence): total weight of the chunk.
template <typename T, bool kVecT, bool kVecD>
__global__ __launch_bounds__(256) void sample_sum_kernel(const T* __restrict__ tgt,
                                                        const float* __restrict__ drf,
                                                        const VerifyRec* __restrict__ rec, int B,
                                                        int V, float inv_t,
                                                        float* __restrict__ csum, int n_chunks) {
  __shared__ float s_wt[4];
  const int chunk = blockIdx.x, n = blockIdx.y, t = threadIdx.x;
  const VerifyRec v = rec[n];
  const int c0 = chunk * kSampleChunk + t * 32;
  const float x = c0 < V ? thread_run_sum<T, kVecT, kVecD>(tgt, drf, v, n, B, V, inv_t, c0) : 0.f;
  const float incl = block_incl_scan256(x, s_wt);
  if (t == 255) csum[static_cast<int64_t>(n) * n_chunks + chunk] = incl;
}

// One workgroup per sequence: the chunk where the running total passes
// u * total (thread 0, chunk sums in order), then the thread run (the first
// run of positive weight whose running total passes the target, from the
// workgroup scan), then the column (the first positive-weight column whose
// running total inside the run passes it, from a wave scan).  A target past
// every column of the chosen run (rounding between the two passes) takes the
// run's last column of positive weight; past every run of the chunk, the
// chunk's last column of positive weight.
template <typename T, bool kVecT, bool kVecD>
__global__ __launch_bounds__(256) void sample_pick_kernel(const T* __restrict__ tgt,
                                                         const float* __restrict__ drf,
                                                         const VerifyRec* __restrict__ rec, int B,
                                                         int V, float inv_t,
                                                         const float* __restrict__ csum,
                                                         int n_chunks, const float* __restrict__ u,
                                                         int32_t* __restrict__ next_tok) {
  constexpr int kRun = kSampleChunk / 256;   // columns per thread run
  __shared__ float s_cs[256];
  __shared__ float s_incl[256];
  __shared__ float s_wt[4];
  __shared__ int s_first[4], s_lastp[4];
  __shared__ int s_chunk;
  __shared__ float s_base, s_target;
  const int n = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const VerifyRec v = rec[n];
  const float* cs = csum + static_cast<int64_t>(n) * n_chunks;
  // chunk sums through LDS when they fit (one per thread), else read in place
  const bool staged = n_chunks <= 256;
  if (staged) s_cs[t] = t < n_chunks ? cs[t] : 0.f;
  __syncthreads();
  if (t == 0) {
    auto chunk_sum = [&](int c) { return staged ? s_cs[c] : cs[c]; };
    float tot = 0.f;
    for (int c = 0; c < n_chunks; ++c) tot += chunk_sum(c);
    const float target = u[n] * tot;
    float base = 0.f;
    int chosen = n_chunks - 1;
    for (int c = 0; c < n_chunks; ++c) {
      if (base + chunk_sum(c) > target) { chosen = c; break; }
      if (c < n_chunks - 1) base += chunk_sum(c);
    }
    // skip trailing empty chunks the fallback could land on
    while (chosen > 0 && chunk_sum(chosen) <= 0.f) { --chosen; base -= chunk_sum(chosen); }
    s_chunk = chosen;
    s_base = base;
    s_target = target;
  }
  __syncthreads();
  const int chunk = s_chunk;
  const float base = s_base, target = s_target;
  const int c0 = chunk * kSampleChunk + t * kRun;
  const float x = c0 < V ? thread_run_sum<T, kVecT, kVecD>(tgt, drf, v, n, B, V, inv_t, c0) : 0.f;
  const float incl = block_incl_scan256(x, s_wt);
  s_incl[t] = incl;
  // first run whose running total passes the target; last run of positive weight
  const uint64_t hit = __ballot(x > 0.f && base + incl > target);
  const uint64_t pos = __ballot(x > 0.f);
  if (lane == 0) {
    s_first[wv] = hit ? wv * 64 + __ffsll(static_cast<unsigned long long>(hit)) - 1 : 256;
    s_lastp[wv] = pos ? wv * 64 + 63 - __clzll(static_cast<long long>(pos)) : -1;
  }
  __syncthreads();
  if (t >= 64) return;
  int run = min(min(s_first[0], s_first[1]), min(s_first[2], s_first[3]));
  run = run < 256 ? run : -1;
  const int last_pos = max(max(s_lastp[0], s_lastp[1]), max(s_lastp[2], s_lastp[3]));
  // wave 0: lanes 0..31 weigh the columns of the chosen run, lanes 32..63
  // those of the last run of positive weight
  const int rsel = lane < kRun ? run : last_pos;
  const int c = chunk * kSampleChunk + rsel * kRun + (lane % kRun);
  const float w = (rsel >= 0 && c < V) ? sample_weight(tgt, drf, v, n, B, V, inv_t, c) : 0.f;
  float wi = lane < kRun ? w : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(wi, o, 64);
    if (lane >= o) wi += y;
  }
  const float a2 = base + (run > 0 ? s_incl[run - 1] : 0.f);
  const uint64_t chit = __ballot(lane < kRun && run >= 0 && w > 0.f && a2 + wi > target);
  const uint64_t rpos = __ballot(lane < kRun && w > 0.f);
  const uint64_t lpos = __ballot(lane >= kRun && w > 0.f);
  if (lane == 0) {
    int col = -1;
    if (run >= 0) {
      const int r0 = chunk * kSampleChunk + run * kRun;
      if (chit) col = r0 + __ffsll(static_cast<unsigned long long>(chit)) - 1;
      else if (rpos) col = r0 + 63 - __clzll(static_cast<long long>(rpos));
    }
    if (col < 0 && last_pos >= 0 && lpos)   // rounding left the target past the chunk
      col = chunk * kSampleChunk + last_pos * kRun + (63 - __clzll(static_cast<long long>(lpos))) - kRun;
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
