// Weight-streaming GEMM for few rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Shape of the problem on the drafter's decode path: M = batch * B <= 256 rows
// of activations against weight matrices of 10^7..10^9 bytes, so the weight
// stream from HBM sets the time.  Design for CDNA4:
//   - A workgroup (4 waves) owns one "pair tile": two 16-row groups of W
//     (w0, w1) whose outputs the epilogue needs together -- the two halves of a
//     RoPE head, a gate row and its up row, or just 32 consecutive rows.
//   - The 4 waves split K; each streams its W rows straight from HBM into MFMA
//     B fragments (16 bytes per lane, 64 contiguous bytes per row and
//     instruction), double-buffered U steps deep to keep bytes in flight.
//   - A (the small activation matrix) is read from L2 in A-fragment layout and
//     may be split over several slabs along K (the fusion input needs no
//     concatenation copy).
//   - Partial sums of the 4 waves meet in LDS (fixed order); an optional split
//     of K over `ksplit` workgroups meets in a workspace, summed in split order
//     by the last workgroup to arrive, so results do not depend on timing.
//   - The epilogue receives, per output row m and column i in 0..15, the pair
//     (v0, v1) = (out[m, w0 row i], out[m, w1 row i]).
#pragma once

#include "device_common.h"

namespace dflash {

template <typename T>
struct AOperand {
  const T* slab[6];   // K is split into slabs of slab_k columns each
  int64_t lda;        // row stride of every slab, elements
  int slab_k;
  int M;              // rows of the whole problem (the epilogue's row index space)
  int m0, mc;         // this launch covers rows [m0, m0 + mc), mc <= 16 * MT
};

template <typename T>
__device__ __forceinline__ const T* a_ptr(const AOperand<T>& A, int row, int k) {
  const int s = k / A.slab_k;
  return A.slab[s] + static_cast<int64_t>(row) * A.lda + (k - s * A.slab_k);
}

template <typename T, int MT, int U, class Epi>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(AOperand<T> A, int K, int ksplit,
                                                          float* __restrict__ part,
                                                          int* __restrict__ counters, Epi epi) {
  __shared__ float red[4][2][256];
  __shared__ int s_last;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kg = lane >> 4;

  const T* w0;
  const T* w1;
  epi.rows(tile, r16, w0, w1);
  const int kper = K / (4 * ksplit);
  const int kbeg = (split * 4 + wave) * kper;
  w0 += kbeg + kg * 8;
  w1 += kbeg + kg * 8;
  int arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = A.m0 + min(mt * 16 + r16, A.mc - 1);

  f32x4 acc0[MT], acc1[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) { acc0[mt] = zero4(); acc1[mt] = zero4(); }

  Frag8<T> b0[2][U], b1[2][U], a[2][MT][U];
  auto load = [&](int buf, int k) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      ld_frag(b0[buf][u], w0 + k + u * 32);
      ld_frag(b1[buf][u], w1 + k + u * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        ld_frag(a[buf][mt][u], a_ptr(A, arow[mt], kbeg + k + u * 32 + kg * 8));
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc0[mt] = mfma16(acc0[mt], a[buf][mt][u], b0[buf][u]);
        acc1[mt] = mfma16(acc1[mt], a[buf][mt][u], b1[buf][u]);
      }
  };
  const int step = 32 * U;
  load(0, 0);
  int k = 0;
  for (; k + 2 * step <= kper; k += 2 * step) {
    load(1, k + step);
    compute(0);
    if (k + 2 * step < kper) load(0, k + 2 * step);
    compute(1);
  }
  if (k < kper) compute(0);

  // waves meet in LDS (fixed order): lane holds rows kg*4+jj, column r16
  const int t = threadIdx.x;
  float v0[MT], v1[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      red[wave][0][(kg * 4 + jj) * 16 + r16] = acc0[mt][jj];
      red[wave][1][(kg * 4 + jj) * 16 + r16] = acc1[mt][jj];
    }
    __syncthreads();
    v0[mt] = (red[0][0][t] + red[1][0][t]) + (red[2][0][t] + red[3][0][t]);
    v1[mt] = (red[0][1][t] + red[1][1][t]) + (red[2][1][t] + red[3][1][t]);
    __syncthreads();
  }

  if (ksplit > 1) {
    float2* my = reinterpret_cast<float2*>(part) +
                 (static_cast<int64_t>(tile) * ksplit + split) * (MT * 256);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) my[mt * 256 + t] = make_float2(v0[mt], v1[mt]);
    __threadfence();
    __syncthreads();
    if (t == 0) s_last = (atomicAdd(&counters[tile], 1) == ksplit - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float2* all = reinterpret_cast<const float2*>(part) +
                        static_cast<int64_t>(tile) * ksplit * (MT * 256);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float s0 = 0.f, s1 = 0.f;
      for (int s = 0; s < ksplit; ++s) {
        const float2 p = all[static_cast<int64_t>(s) * (MT * 256) + mt * 256 + t];
        s0 += p.x;
        s1 += p.y;
      }
      v0[mt] = s0;
      v1[mt] = s1;
    }
  }

  // element t of a 16x16 tile: row t/16, column t%16
  const int i = t & 15, rr = t >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = mt * 16 + rr;
    epi.apply(tile, A.m0 + m, i, m < A.mc, v0[mt], v1[mt]);
  }
  epi.tail(tile, A.m0, A.mc);
}

}  // namespace dflash
