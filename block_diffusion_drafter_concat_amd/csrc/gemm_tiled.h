// LDS-tiled bf16 MFMA GEMM for many rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Used where M is large enough that the problem is compute-bound (fusion and
// injection over a prefill of T context rows).  Design for CDNA4 (gfx950):
//   - workgroup tile 256 x 256 (rows of A x rows of W), 4 waves in a 2 x 2
//     grid, each wave 128 x 128 = 8 x 8 MFMA tiles of 16 x 16 (fp32
//     accumulators, 256 per lane, held in AGPRs);
//   - K in stages of 64: both operand tiles (2 x 32 KB) go through LDS, double
//     buffered; the next stage is loaded into registers while the current one
//     feeds the MFMAs.  16-byte chunks are XOR-swizzled by row so that the
//     fragment reads (16 rows x 16 bytes per instruction) hit distinct banks;
//   - tiles are walked in an XCD-aware order: workgroup w runs on XCD w % 8,
//     so consecutive tile indices are given to the same XCD, and inside an
//     XCD's range tiles go in groups of 4 row-tiles, so the A and W tiles a
//     group shares stay in that XCD's L2;
//   - grid.y selects an output part (e.g. a layer's K or V projection), grid.z
//     a K split whose fp32 partial the consumer sums;
//   - the accumulators leave through LDS in four 64-row slices, so the
//     epilogue sees whole rows of the 256-column tile and can store them
//     coalesced (and RoPE pairs (c, c + d/2) of a head are both at hand).
#pragma once

#include "device_common.h"
#include "gemm_skinny.h"

namespace dflash {

constexpr int kTBM = 256, kTBN = 256, kTBK = 64;

// Row r, 16-byte chunk c (of 8 per 64-element row) of a 256 x 64 LDS tile.
__device__ __forceinline__ int swz(int r, int c) { return r * 64 + ((c ^ (r & 7)) << 3); }

// One 64-row slice of a finished 256 x 256 tile in LDS, as the epilogue sees
// it: local row lr < 32 is output row mA + lr, lr >= 32 is mB + lr - 32;
// column c is output column n0 + c.
constexpr int kCtStride = kTBN + 4;   // padded fp32 row stride (no bank conflicts)
constexpr int kTiledEpiLds = 1024;
struct TiledSlice {
  const float* c;
  int mA, mB, M, n0, N, part, split;
  __device__ int row(int lr) const { return lr < 32 ? mA + lr : mB + lr - 32; }
  __device__ float at(int lr, int col) const { return c[lr * kCtStride + col]; }
};
static_assert(64 * kCtStride * 4 + kTiledEpiLds <= 2 * 2 * kTBM * kTBK * 2, "slice fits in LDS");

template <class Epi>
__global__ __launch_bounds__(256) void tiled_gemm_kernel(AOperand<uint16_t> A, int N, int K,
                                                         int tiles_m, int tiles_n, Epi epi) {
  const int part = blockIdx.y;    // output part (uniform per workgroup)
  const int split = blockIdx.z;   // K split
  extern __shared__ __align__(16) uint16_t lds[];   // [2][A 256x64 | W 256x64]
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int r16 = lane & 15, kg = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- XCD-aware tile order: workgroup w runs on XCD w % 8; XCD x owns the
  // contiguous tile range [start(x), start(x) + count(x)) (a bijection)
  const int n_tiles = tiles_m * tiles_n;
  const int w = blockIdx.x;
  const int xcd = w % 8, local = w / 8;
  const int base_cnt = n_tiles / 8, extra = n_tiles % 8;
  const int tile = xcd * base_cnt + min(xcd, extra) + local;
  // tiles are visited in groups of 4 row-tiles sweeping all column tiles
  constexpr int kGroup = 4;
  const int group_size = kGroup * tiles_n;
  const int g0 = (tile / group_size) * kGroup;
  const int gm = min(kGroup, tiles_m - g0);
  const int in_g = tile % group_size;
  const int tm = g0 + in_g % gm;
  const int tn = in_g / gm;
  const int m0 = tm * kTBM, n0 = tn * kTBN;

  const int kper = K / gridDim.z;
  const int kbeg = split * kper;

  // ---- global -> register staging: thread t moves chunks (row t/8 + 32 i,
  // chunk t%8) of both operand tiles; row offsets and W row pointers are fixed
  // for the whole K loop.
  const int srow = t >> 3, schunk = t & 7;
  int64_t aoff[8];
  const uint16_t* wp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    aoff[i] = static_cast<int64_t>(min(m0 + srow + 32 * i, A.M - 1)) * A.lda + schunk * 8;
    wp[i] = epi.wrow(part, min(n0 + srow + 32 * i, N - 1)) + schunk * 8;
  }
  int lw_off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lw_off[i] = swz(srow + 32 * i, schunk);

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = zero4();

  const int n_stages = kper / kTBK;
  uint4 ra0, ra1, ra2, ra3, ra4, ra5, ra6, ra7;
  uint4 rw0, rw1, rw2, rw3, rw4, rw5, rw6, rw7;
#define DF_GLOAD(k0)                                                                      \
  {                                                                                       \
    const int s_ = (k0) / A.slab_k;                                                       \
    const uint16_t* ab_ = A.slab[s_] + ((k0) - s_ * A.slab_k);                            \
    ra0 = *reinterpret_cast<const uint4*>(ab_ + aoff[0]);                                 \
    ra1 = *reinterpret_cast<const uint4*>(ab_ + aoff[1]);                                 \
    ra2 = *reinterpret_cast<const uint4*>(ab_ + aoff[2]);                                 \
    ra3 = *reinterpret_cast<const uint4*>(ab_ + aoff[3]);                                 \
    ra4 = *reinterpret_cast<const uint4*>(ab_ + aoff[4]);                                 \
    ra5 = *reinterpret_cast<const uint4*>(ab_ + aoff[5]);                                 \
    ra6 = *reinterpret_cast<const uint4*>(ab_ + aoff[6]);                                 \
    ra7 = *reinterpret_cast<const uint4*>(ab_ + aoff[7]);                                 \
    rw0 = *reinterpret_cast<const uint4*>(wp[0] + (k0));                                  \
    rw1 = *reinterpret_cast<const uint4*>(wp[1] + (k0));                                  \
    rw2 = *reinterpret_cast<const uint4*>(wp[2] + (k0));                                  \
    rw3 = *reinterpret_cast<const uint4*>(wp[3] + (k0));                                  \
    rw4 = *reinterpret_cast<const uint4*>(wp[4] + (k0));                                  \
    rw5 = *reinterpret_cast<const uint4*>(wp[5] + (k0));                                  \
    rw6 = *reinterpret_cast<const uint4*>(wp[6] + (k0));                                  \
    rw7 = *reinterpret_cast<const uint4*>(wp[7] + (k0));                                  \
  }
#define DF_LSTORE(buf)                                                                    \
  {                                                                                       \
    uint16_t* la_ = lds + (buf) * (2 * kTBM * kTBK);                                      \
    uint16_t* lw_ = la_ + kTBM * kTBK;                                                    \
    *reinterpret_cast<uint4*>(la_ + lw_off[0]) = ra0;                                     \
    *reinterpret_cast<uint4*>(la_ + lw_off[1]) = ra1;                                     \
    *reinterpret_cast<uint4*>(la_ + lw_off[2]) = ra2;                                     \
    *reinterpret_cast<uint4*>(la_ + lw_off[3]) = ra3;                                     \
    *reinterpret_cast<uint4*>(la_ + lw_off[4]) = ra4;                                     \
    *reinterpret_cast<uint4*>(la_ + lw_off[5]) = ra5;                                     \
    *reinterpret_cast<uint4*>(la_ + lw_off[6]) = ra6;                                     \
    *reinterpret_cast<uint4*>(la_ + lw_off[7]) = ra7;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[0]) = rw0;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[1]) = rw1;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[2]) = rw2;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[3]) = rw3;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[4]) = rw4;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[5]) = rw5;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[6]) = rw6;                                     \
    *reinterpret_cast<uint4*>(lw_ + lw_off[7]) = rw7;                                     \
  }
  DF_GLOAD(kbeg);
  DF_LSTORE(0);
  __syncthreads();
  for (int st = 0; st < n_stages; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < n_stages;
    if (more) DF_GLOAD(kbeg + (st + 1) * kTBK);
    const uint16_t* la = lds + buf * (2 * kTBM * kTBK);
    const uint16_t* lw = la + kTBM * kTBK;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      Frag8<uint16_t> af[8], bf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        af[i].v = *reinterpret_cast<const uint4*>(la + swz(wm * 128 + i * 16 + r16, kk * 4 + kg));
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bf[j].v = *reinterpret_cast<const uint4*>(lw + swz(wn * 128 + j * 16 + r16, kk * 4 + kg));
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(acc[i][j], af[i], bf[j]);
    }
    // the other buffer was last read in the previous stage, which every
    // thread finished before the previous barrier
    if (more) DF_LSTORE(buf ^ 1);
    __syncthreads();
  }
#undef DF_GLOAD
#undef DF_LSTORE

  // ---- epilogue: slice q holds rows {32 q + r, 128 + 32 q + r : r < 32} of
  // the tile as C[64][kCtStride] fp32 (local row lr = wm * 32 + r).  C tile
  // (i, j) lane holds rows i*16 + kg*4 + jj, column j*16 + r16.
  float* ct = reinterpret_cast<float*>(lds);
  void* ext = ct + 64 * kCtStride;   // epilogue's own LDS (kTiledEpiLds bytes)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          ct[(wm * 32 + ii * 16 + kg * 4 + jj) * kCtStride + wn * 128 + j * 16 + r16] =
              acc[2 * q + ii][j][jj];
    __syncthreads();
    const TiledSlice sl{ct, m0 + 32 * q, m0 + 128 + 32 * q, A.M, n0, N, part, split};
    epi.store(sl, ext, t);
    __syncthreads();
  }
}

constexpr size_t kTiledLds = 2 * 2 * kTBM * kTBK * sizeof(uint16_t);   // 128 KB

// ------------------------------------------------------------- epilogues

// out[split][m][n] (float32 partial sums) over W rows 0..N-1; N % 4 == 0.
struct TEpiStoreF32 {
  const uint16_t* W;
  int K;
  float* out;
  int64_t ldo, slab_rows;
  __device__ const uint16_t* wrow(int, int n) const { return W + static_cast<int64_t>(n) * K; }
  __device__ void store(const TiledSlice& s, void*, int t) const {
    const int c4 = (t & 63) * 4;
    if (s.n0 + c4 >= s.N) return;
    for (int lr = t >> 6; lr < 64; lr += 4) {
      const int m = s.row(lr);
      if (m >= s.M) continue;
      const float4 v = *reinterpret_cast<const float4*>(s.c + lr * kCtStride + c4);
      *reinterpret_cast<float4*>(out + (s.split * slab_rows + m) * ldo + s.n0 + c4) = v;
    }
  }
};

// KV injection over rows of context features.  Part p = 2 * layer + (0: K,
// 1: V); its N = Hkv * d columns are that layer's k (or v) projection.  K
// gets RoPE at the row's position (the pair partner of column c is c + d/2);
// V is stored transposed.  A tile's 256 columns hold whole heads.
struct TEpiInject {
  const uint16_t* wk[kMaxLayers];
  const uint16_t* wv[kMaxLayers];
  uint16_t* kc[kMaxLayers];
  uint16_t* vc[kMaxLayers];
  int K, d;
  int64_t cap;
  RopeFreq freq;
  SeqTable seq;
  __device__ const uint16_t* wrow(int part, int n) const {
    const uint16_t* w = (part & 1) ? wv[part >> 1] : wk[part >> 1];
    return w + static_cast<int64_t>(n) * K;
  }
  __device__ void store(const TiledSlice& s, void* ext, int t) const {
    // per local row: position and cache row (rows are grouped by sequence)
    int* pos_t = static_cast<int*>(ext);
    int64_t* row_t = reinterpret_cast<int64_t*>(pos_t + 64);
    if (t < 64) {
      const int m = min(s.row(t), s.M - 1);
      int pos = 0;
      int64_t off = 0;
      for (int b = 0; b < seq.n; ++b)
        if (m >= seq.row0[b]) {
          pos = seq.pos0[b] + (m - seq.row0[b]);
          off = seq.off[b];
        }
      pos_t[t] = pos;
      row_t[t] = off + pos;
    }
    __syncthreads();
    if ((s.part & 1) == 0) {
      uint16_t* kd = kc[s.part >> 1];
      const int half = d / 2;
      const int q = t & 127;                    // RoPE pair of the tile
      const int hl = q / half, c = q % half;    // head inside the tile, pair index
      const int col = hl * d + c;
      const int head = (s.n0 + col) / d;
      if (s.n0 + col >= s.N) return;
      const double inv = freq.inv[c];
      for (int lr = t >> 7; lr < 64; lr += 2) {
        if (s.row(lr) >= s.M) continue;
        float cs, sn;
        rope_cos_sin(pos_t[lr], inv, cs, sn);
        const float x0 = s.at(lr, col), x1 = s.at(lr, col + half);
        uint16_t* dst = kd + (static_cast<int64_t>(head) * cap + row_t[lr]) * d + c;
        stf(dst, x0 * cs - x1 * sn);
        stf(dst + half, x1 * cs + x0 * sn);
      }
    } else {
      uint16_t* vt = vc[s.part >> 1];
      const int lr = t & 63;
      if (s.row(lr) >= s.M) return;
      const int64_t r = row_t[lr];
      for (int col = t >> 6; col < kTBN && s.n0 + col < s.N; col += 4)
        stf(vt + static_cast<int64_t>(s.n0 + col) * cap + r, s.at(lr, col));
    }
  }
};

}  // namespace dflash
