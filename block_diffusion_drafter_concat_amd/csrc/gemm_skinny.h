// Weight-streaming GEMM for few rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Shape of the problem on the drafter's decode path: M = batch * B <= 128 rows
// per launch against weight matrices of 10^7..10^9 bytes, so the weight
// stream from HBM sets the time.  Design for CDNA4:
//   - A workgroup (NW waves) owns PT "pair tiles" at a time: each two 16-row
//     groups of W (w0, w1) whose outputs the epilogue needs together -- the
//     two halves of a RoPE head, a gate row and its up row, or just 32
//     consecutive rows.  The PT pair tiles share each A fragment, so PT = 2
//     halves the A reads per weight byte (measured: the per-step A reads from
//     L2 cost 15-25% of the weight-stream rate).  A workgroup may walk several
//     such steps.
//   - The NW waves split K; each streams its W rows straight from HBM into
//     MFMA B fragments (16 bytes per lane, 64 contiguous bytes per row and
//     instruction), double-buffered U steps deep to keep bytes in flight.
//   - A (the small activation matrix) is read from L2 in A-fragment layout and
//     may be split over several slabs along K (SLABS; the fusion input needs
//     no concatenation copy).  The slab of a 32-column step is picked with
//     scalar arithmetic, so its pointer is one scalar load, not a per-lane
//     load that every A fragment would wait behind; a one-slab A (SLABS =
//     false) needs no pick at all.  An A written by the
//     drafter's own kernels is stored fragment-major (frag_major()): each
//     fragment load is then one contiguous 16 x 32 run instead of 16 row
//     pieces, which measured 10-15% faster on the M = 16 shapes.
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
  int64_t lda;        // row stride of every slab, elements (fragment-major: the row length K)
  int frag;           // 1: one slab, stored fragment-major (frag_major())
  int slab_k;
  int M;              // rows of the whole problem (the epilogue's row index space)
  int m0, mc;         // this launch covers rows [m0, m0 + mc), mc <= 16 * MT
};

template <typename T, int MT, int U, int NW, int PT, class Epi, bool SLABS>
__global__ __launch_bounds__(NW * 64) void skinny_gemm_kernel(AOperand<T> A, int K, int n_tiles,
                                                              int tiles_per_wg, Epi epi) {
  __shared__ float red[NW][2][256];
  const int split = blockIdx.y, ksplit = gridDim.y;
  // the wave index is uniform: k offsets and the slab choice stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int kper = K / (NW * ksplit);
  const int kbeg = (split * NW + wave) * kper;
  // slab of column kk (uniform, a multiple of 32; so is slab_k, and the 32
  // columns of a step never straddle two slabs): floor(kk / slab_k) through a
  // 40-bit reciprocal, exact while kk * slab_k < 2^40 (host-checked)
  const uint64_t slab_magic = (uint64_t{1} << 40) / static_cast<uint64_t>(A.slab_k) + 1;
  // elements between two 32-column steps of one row: 32 row-major, one
  // 16 x 32 chunk fragment-major
  const int kstep = A.frag ? 512 : 32;
  const T* aslab0 = A.slab[0];
  int64_t aoff[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = A.m0 + min(mt * 16 + r16, A.mc - 1);
    aoff[mt] = (A.frag ? static_cast<int64_t>(row >> 4) * 16 * A.lda + (row & 15) * 32
                       : static_cast<int64_t>(row) * A.lda) + kg * 8;
  }
  const int t = threadIdx.x;
  const int i = t & 15, rr = t >> 4;   // element t of a 16x16 tile: row t/16, column t%16

  typename Epi::State es;
  epi.init(es);
  // a step of the walk covers PT consecutive pair tiles, which share every
  // A fragment (PT = 2 halves the A loads per weight byte)
  const int n_steps = (n_tiles + PT - 1) / PT;
  const int st_first = blockIdx.x * tiles_per_wg;
  const int st_end = min(n_steps, st_first + tiles_per_wg);
  for (int sw = st_first; sw < st_end; ++sw) {
    const T* w0[PT];
    const T* w1[PT];
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      // a missing last tile re-reads the previous one; its sums are dropped
      epi.rows(min(sw * PT + p, n_tiles - 1), r16, w0[p], w1[p]);
      w0[p] += kbeg + kg * 8;
      w1[p] += kbeg + kg * 8;
    }

    f32x4 acc0[PT][MT], acc1[PT][MT];
#pragma unroll
    for (int p = 0; p < PT; ++p)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) { acc0[p][mt] = zero4(); acc1[p][mt] = zero4(); }

    Frag8<T> b0[2][PT][U], b1[2][PT][U], a[2][MT][U];
    auto load = [&](int buf, int k) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int p = 0; p < PT; ++p) {
          ld_frag(b0[buf][p][u], w0[p] + k + u * 32);
          ld_frag(b1[buf][p][u], w1[p] + k + u * 32);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kk = kbeg + k + u * 32;
        // one slab (every A but the fusion input): no slab pick, so no scalar
        // load of the slab pointer sits on the step's critical path
        const int sl = SLABS ? static_cast<int>((static_cast<uint64_t>(kk) * slab_magic) >> 40) : 0;
        const T* as = (SLABS ? A.slab[sl] : aslab0) +
                      static_cast<int64_t>((kk - sl * A.slab_k) >> 5) * kstep;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ld_frag(a[buf][mt][u], as + aoff[mt]);
      }
    };
    auto compute = [&](int buf) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int p = 0; p < PT; ++p) {
            acc0[p][mt] = mfma16(acc0[p][mt], a[buf][mt][u], b0[buf][p][u]);
            acc1[p][mt] = mfma16(acc1[p][mt], a[buf][mt][u], b1[buf][p][u]);
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
    for (int p = 0; p < PT; ++p) {
      const int tile = sw * PT + p;
      if (tile >= n_tiles) break;   // uniform over the workgroup
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          red[wave][0][(kg * 4 + jj) * 16 + r16] = acc0[p][mt][jj];
          red[wave][1][(kg * 4 + jj) * 16 + r16] = acc1[p][mt][jj];
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
  }
  if (t < 256) epi.finish(es, blockIdx.x, A.m0, A.mc);
}

}  // namespace dflash
