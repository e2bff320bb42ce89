// Weight-streaming GEMM for few rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Shape of the problem on the drafter's decode path: M = batch * B <= 128 rows
// per launch against weight matrices of 10^7..10^9 bytes, so the weight
// stream from HBM sets the time.  Design for CDNA4:
//   - A workgroup (NW waves) owns one "pair tile" at a time: two 16-row
//     groups of W (w0, w1) whose outputs the epilogue needs together -- the
//     two halves of a RoPE head, a gate row and its up row, or just 32
//     consecutive rows.  It may walk several consecutive tiles.
//   - The NW waves split K; each streams its W rows straight from HBM into
//     MFMA B fragments (16 bytes per lane, 64 contiguous bytes per row and
//     instruction), double-buffered U steps deep to keep bytes in flight.
//   - A (the small activation matrix) is read from L2 in A-fragment layout and
//     may be split over several slabs along K (the fusion input needs no
//     concatenation copy).
//   - Partial sums of the waves meet in LDS in a fixed order.  A split of K
//     over `ksplit` workgroups (grid.y) never meets inside this kernel: each
//     split hands its fp32 partial to the epilogue (which stores it), and the
//     next kernel -- which needs whole rows anyway -- sums the splits in
//     order.  No workgroup waits on another, so no device-wide fence is ever
//     issued (on gfx950 each such fence writes back the XCD's L2).
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

template <typename T, int MT, int U, int NW, class Epi>
__global__ __launch_bounds__(NW * 64) void skinny_gemm_kernel(AOperand<T> A, int K, int n_tiles,
                                                              int tiles_per_wg, Epi epi) {
  __shared__ float red[NW][2][256];
  const int split = blockIdx.y, ksplit = gridDim.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int kper = K / (NW * ksplit);
  const int kbeg = (split * NW + wave) * kper;
  int arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = A.m0 + min(mt * 16 + r16, A.mc - 1);
  const int t = threadIdx.x;
  const int i = t & 15, rr = t >> 4;   // element t of a 16x16 tile: row t/16, column t%16

  typename Epi::State es;
  epi.init(es);
  const int tile_first = blockIdx.x * tiles_per_wg;
  const int tile_end = min(n_tiles, tile_first + tiles_per_wg);
  for (int tile = tile_first; tile < tile_end; ++tile) {
    const T* w0;
    const T* w1;
    epi.rows(tile, r16, w0, w1);
    w0 += kbeg + kg * 8;
    w1 += kbeg + kg * 8;

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
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        red[wave][0][(kg * 4 + jj) * 16 + r16] = acc0[mt][jj];
        red[wave][1][(kg * 4 + jj) * 16 + r16] = acc1[mt][jj];
      }
      __syncthreads();
      if (t < 256) {
        float v0 = 0.f, v1 = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          v0 += red[w][0][t];
          v1 += red[w][1][t];
        }
        const int m = mt * 16 + rr;
        epi.apply(es, mt, tile, split, A.m0 + m, i, m < A.mc, v0, v1);
      }
      __syncthreads();
    }
  }
  if (t < 256) epi.finish(es, blockIdx.x, A.m0, A.mc);
}

}  // namespace dflash
