// LDS-tiled bf16 MFMA GEMM for many rows: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Used where M is large enough that the problem is compute-bound (fusion and
// injection over a prefill of T context rows).  Design for CDNA4 (gfx950):
//   - workgroup tile 256 x 256 (rows of A x rows of W), 4 waves in a 2 x 2
//     grid, each wave 128 x 128 = 8 x 8 MFMA tiles of 16 x 16 (fp32
//     accumulators, 256 per lane, held in AGPRs);
//   - K in stages of 64: both operand tiles (2 x 32 KB) go through LDS, double
//     buffered; the next stage is loaded straight into LDS (buffer loads with
//     the LDS-destination bit, no staging registers) while the current one
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
// it.  Local rows come in runs of `run` rows, one run per wave row; run r
// starts at output row m_base + r * wave_rows.  Column c is output column
// n0 + c.
constexpr int kCtStride = kTBN + 4;   // padded fp32 row stride (no bank conflicts)
constexpr int kTiledEpiLds = 1024;
struct TiledSlice {
  const float* c;
  int m_base, run, wave_rows, M, n0, N, part, split;
  __device__ int row(int lr) const { return m_base + (lr / run) * wave_rows + lr % run; }
  __device__ float at(int lr, int col) const { return c[lr * kCtStride + col]; }
};
static_assert(64 * kCtStride * 4 + kTiledEpiLds <= 2 * 2 * kTBM * kTBK * 2, "slice fits in LDS");

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n),
                                           0x00020000);
}

// WM x WN waves; wave (wm, wn) owns rows wm * 256/WM and columns
// wn * 256/WN of the tile as MI x NJ MFMA tiles of 16 x 16.
template <int WM, int WN, class Epi>
__global__ __launch_bounds__(WM * WN * 64) void tiled_gemm_kernel(AOperand<uint16_t> A, int N,
                                                                  int K, int tiles_m,
                                                                  int tiles_n, Epi epi) {
  constexpr int NWAVES = WM * WN, NT = NWAVES * 64;
  constexpr int RW = kTBM / WM, CW = kTBN / WN;   // wave tile
  constexpr int MI = RW / 16, NJ = CW / 16;
  constexpr int LI = 32 / NWAVES;                 // loads per wave per operand
  static_assert(MI % 4 == 0, "four epilogue slices per wave row");
  const int part = blockIdx.y;    // output part (uniform per workgroup)
  const int split = blockIdx.z;   // K split
  extern __shared__ __align__(16) uint16_t lds[];   // [2][A 256x64 | W 256x64]
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int r16 = lane & 15, kg = lane >> 4;
  const int wm = wave / WN, wn = wave % WN;

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

  // ---- global -> LDS without registers (buffer_load ... lds).  One wave
  // instruction fills 1 KB of LDS: 8 tile rows of 8 16-byte chunks, lane l
  // landing at chunk l of the run.  Instruction i of wave w covers tile rows
  // 8 (w LI + i) .. +8; lane l takes row 8 (w LI + i) + l / 8 and, so that the
  // XOR swizzle holds, global chunk (l % 8) ^ (l / 8).  Rows past M or N
  // read as zero through the buffer range check.
  const int lrow = 8 * LI * wave + (lane >> 3);
  const int gchunk = (lane & 7) ^ (lane >> 3);
  const uint32_t a_voff = static_cast<uint32_t>(lrow * A.lda * 2 + gchunk * 16);
  const uint32_t w_voff = static_cast<uint32_t>(lrow * K * 2 + gchunk * 16);
  const uint32_t a_istep = static_cast<uint32_t>(8 * A.lda * 2);
  const uint32_t w_istep = static_cast<uint32_t>(8 * K * 2);
  const __amdgpu_buffer_rsrc_t wrs =
      tile_rsrc(epi.wbase(part) + static_cast<int64_t>(n0) * K,
                static_cast<uint64_t>(N - n0) * static_cast<uint64_t>(K) * 2);
  const uint64_t a_bytes = static_cast<uint64_t>(A.M - m0) * static_cast<uint64_t>(A.lda) * 2;
  auto issue = [&](int k0, int buf) {
    const int s = k0 / A.slab_k;
    const int col = k0 - s * A.slab_k;
    const __amdgpu_buffer_rsrc_t ars =
        tile_rsrc(A.slab[s] + static_cast<int64_t>(m0) * A.lda, a_bytes);
    lds_u16* la = (lds_u16*)(lds) + buf * (2 * kTBM * kTBK) + wave * (LI * 512);
    lds_u16* lw = la + kTBM * kTBK;
#pragma unroll
    for (int i = 0; i < LI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, la + i * 512, 16, a_voff,
                                               i * a_istep + col * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < LI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, lw + i * 512, 16, w_voff,
                                               i * w_istep + k0 * 2, 0, 0);
  };

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = zero4();

  // One stage: read this wave's fragments of both k halves, then (when there
  // is a next stage) start its loads into the other buffer -- after the reads
  // in program order, so no LDS read waits on them -- then the MFMAs.  The
  // other buffer was last read in the previous stage, which every thread
  // finished before the previous barrier.
  auto stage = [&](int buf, bool next, int k_next) {
    const uint16_t* la = lds + buf * (2 * kTBM * kTBK);
    const uint16_t* lw = la + kTBM * kTBK;
    Frag8<uint16_t> af[2][MI], bf[2][NJ];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[kk][i].v =
            *reinterpret_cast<const uint4*>(la + swz(wm * RW + i * 16 + r16, kk * 4 + kg));
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bf[kk][j].v =
            *reinterpret_cast<const uint4*>(lw + swz(wn * CW + j * 16 + r16, kk * 4 + kg));
    }
    if (next) issue(k_next, buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma16(acc[i][j], af[kk][i], bf[kk][j]);
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this wave's next-stage loads
    __syncthreads();
  };

  const int n_stages = kper / kTBK;
  issue(kbeg, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  __syncthreads();
  for (int st = 0; st + 1 < n_stages; ++st) stage(st & 1, true, kbeg + (st + 1) * kTBK);
  stage((n_stages - 1) & 1, false, 0);

  // ---- epilogue: four slices of 64 rows.  Slice q takes MFMA rows
  // i in [q MI/4, (q+1) MI/4) of every wave: local row lr = wm * 4 MI +
  // (i - q MI/4) * 16 + kg * 4 + jj, stored as C[64][kCtStride] fp32.  C tile
  // (i, j) lane holds rows i*16 + kg*4 + jj, column j*16 + r16.
  constexpr int QI = MI / 4, RUN = 16 * QI;
  float* ct = reinterpret_cast<float*>(lds);
  void* ext = ct + 64 * kCtStride;   // epilogue's own LDS (kTiledEpiLds bytes)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
#pragma unroll
    for (int ii = 0; ii < QI; ++ii)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          ct[(wm * RUN + ii * 16 + kg * 4 + jj) * kCtStride + wn * CW + j * 16 + r16] =
              acc[q * QI + ii][j][jj];
    __syncthreads();
    const TiledSlice sl{ct, m0 + q * RUN, RUN, RW, A.M, n0, N, part, split};
    epi.store(sl, ext, t, NT);
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
  __device__ const uint16_t* wbase(int) const { return W; }
  __device__ void store(const TiledSlice& s, void*, int t, int nt) const {
    const int c4 = (t & 63) * 4;
    if (s.n0 + c4 >= s.N) return;
    for (int lr = t >> 6; lr < 64; lr += nt >> 6) {
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
  __device__ const uint16_t* wbase(int part) const {
    return (part & 1) ? wv[part >> 1] : wk[part >> 1];
  }
  __device__ void store(const TiledSlice& s, void* ext, int t, int nt) const {
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
      for (int lr = t >> 7; lr < 64; lr += nt >> 7) {
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
      for (int col = t >> 6; col < kTBN && s.n0 + col < s.N; col += nt >> 6)
        stf(vt + static_cast<int64_t>(s.n0 + col) * cap + r, s.at(lr, col));
    }
  }
};

}  // namespace dflash
