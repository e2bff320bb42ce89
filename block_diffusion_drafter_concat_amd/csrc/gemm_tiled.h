// LDS-tiled bf16 MFMA GEMM: out[m, n] = sum_k A[m, k] * W[n, k].
//
// Used wherever the rows are many enough for the MFMA units to matter: the
// fusion and injection GEMMs over a prefill, and the layer GEMMs and LM head
// of a batch of blocks (M = 64 .. 256 rows).  Design for CDNA4 (gfx950):
//   - workgroup tile BM x BN (rows of A x rows of W), WM x WN waves, each wave
//     (BM/WM) x (BN/WN) as 16 x 16 MFMA tiles with fp32 accumulators;
//   - K in stages of 32: both operand tiles go through a ring of 4-5 LDS
//     slots, NS - 1 stages in flight.  Stages are loaded straight into LDS
//     (buffer loads with the LDS-destination bit, no staging registers) while
//     the current one feeds the MFMAs.  16-byte chunks are XOR-swizzled by
//     row so that the fragment reads (16 rows x 16 bytes per instruction)
//     hit distinct banks.  The next stage's fragment reads and the loads are
//     issued between the current stage's MFMAs in a fixed interleave;
//   - every 16-row load instruction of the W tile has its own buffer resource,
//     from the epilogue's W-row map, so one tile can draw rows from several
//     matrices (q/k/v, gate/up pairs) and rows past a matrix's end read zero;
//   - either operand may be stored row-major or fragment-major (blocks of 16
//     rows x 32 columns, 1 KB each, k fastest: frag_major()).  A load
//     instruction covers 16 rows x 32 columns either way; fragment-major it
//     reads one contiguous 1 KB block instead of 16 row pieces of 64 bytes
//     at the row stride (measured on MI355X: 61 -> 102 GB/s per compute unit
//     from L2 at one workgroup per CU, and fewer stalls on the stage barrier
//     for rows streamed from HBM).  The drafter's own activations are stored
//     that way; weights are when the caller has packed them;
//   - tiles are walked in an XCD-aware order: workgroup w runs on XCD w % 8,
//     so consecutive tile indices are given to the same XCD, and inside an
//     XCD's range tiles go in groups of 4 row-tiles, so the A and W tiles a
//     group shares stay in that XCD's L2;
//   - grid.y selects an output part (e.g. a layer's K or V projection), grid.z
//     a K split whose fp32 partial the consumer sums;
//   - the accumulators leave through LDS in 64-row slices, so the epilogue
//     sees whole rows of the tile and can store them coalesced (and RoPE
//     pairs (c, c + d/2) of a head are both at hand).
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "gemm_skinny.h"

namespace dflash {

constexpr int kTBK = 32;             // k per stage
constexpr int kTiledEpiLds = 1024;   // epilogue's own LDS after the C slice
constexpr int kLdsMax = 160 * 1024;  // LDS of one gfx950 workgroup

// LDS ring slots: 5 when they fit in the workgroup's LDS (3 stages in
// flight ahead of the one being read), else 4.
constexpr int tiled_stages(int BM, int BN) {
  return 5 * (BM + BN) * kTBK * 2 <= kLdsMax ? 5 : 4;
}

// Row r, 16-byte chunk c (of 4 per 32-element row) of an LDS operand tile, in
// elements: chunk c sits at c ^ ((r >> 1) & 3).  A 16-byte-per-lane LDS read
// is served 8 lanes (128 bytes) at a time; the 8 rows of such a group (one
// chunk each, rows 64 bytes apart) then land on 8 distinct 16-byte bank
// groups (measured: no bank-conflict cycles).
__device__ __forceinline__ int swz(int r, int c) { return r * 32 + ((c ^ ((r >> 1) & 3)) << 3); }

// Dynamic LDS of one launch: the stage ring of both operand tiles.
constexpr size_t tiled_lds_bytes(int BM, int BN) {
  return static_cast<size_t>(tiled_stages(BM, BN)) * (BM + BN) * kTBK * sizeof(uint16_t);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits for vmcnt <= n (n < 64) and nothing else
// (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

// LDS fragment read issued as an instruction the compiler does not track:
// the LDS-destination loads of later stages are then never waited for here
// (the compiler would otherwise drain them before every LDS read).  The
// caller waits for the result explicitly (tile_lgkm_wait).
template <int OFF>
__device__ __forceinline__ u32x4_t tile_ds_read(uint32_t addr) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
  return v;
}
// Fragment reads at 1 KB strides from one address (fragment i at i KB).
template <int... I>
__device__ __forceinline__ void tile_read_frags(u32x4_t* dst, uint32_t addr,
                                                std::integer_sequence<int, I...>) {
  ((dst[I] = tile_ds_read<I * 1024>(addr)), ...);
}
// An empty asm that claims to modify x: no use of x can move above it.
__device__ __forceinline__ void tile_tie(u32x4_t& x) { asm volatile("" : "+v"(x)); }
template <int... I>
__device__ __forceinline__ void tile_tie_all(u32x4_t* r, std::integer_sequence<int, I...>) {
  (tile_tie(r[I]), ...);
}

// One 64-row slice of a finished tile in LDS, as the epilogue sees it.  Local
// rows come in runs of `run` rows, one run per wave row; run r starts at
// output row m_base + r * wave_rows.  Column c < bn is output column n0 + c.
struct TiledSlice {
  const float* c;
  int ld;   // fp32 row stride of c
  int m_base, run, wave_rows, M, n0, N, bn, part, split, tile_n;
  __device__ int row(int lr) const { return m_base + (lr / run) * wave_rows + lr % run; }
  __device__ float at(int lr, int col) const { return c[lr * ld + col]; }
};

// W rows [n, n + 8) of part p: where they start and how many are real.
struct WRows {
  const uint16_t* p;
  int valid;
};

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n),
                                           0x00020000);
}

// f(integral_constant<int, I>) for I = 0 .. N-1, in order (compile-time indices).
template <class F, int... I>
__device__ __forceinline__ void tiled_static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void tiled_static_for(F&& f) {
  tiled_static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// wfrag: the W rows the epilogue maps are fragment-major (rows padded with
// zeros to a multiple of 16; the block of a 16-aligned row n starts at n K,
// where row-major row n starts, so the row maps serve both layouts).  A
// fragment-major A has one slab (slab_k == K).
template <int BM, int BN, int WM, int WN, class Epi>
__global__ __launch_bounds__(WM * WN * 64) void tiled_gemm_kernel(AOperand<uint16_t> A, int N,
                                                                  int K, int tiles_m,
                                                                  int tiles_n, int wfrag,
                                                                  Epi epi) {
  constexpr int NWAVES = WM * WN, NT = NWAVES * 64;
  constexpr int RW = BM / WM, CW = BN / WN;   // wave tile
  constexpr int MI = RW / 16, NJ = CW / 16;
  constexpr int NSL = BM / 64, RUN = RW / NSL, QI = RUN / 16;  // epilogue slices
  constexpr int CT_LD = BN + 4;               // padded fp32 row stride of a C slice
  static_assert(BM % 64 == 0 && RUN % 16 == 0 && RUN * WM == 64, "64-row slices");
  static_assert(64 * CT_LD * 4 + kTiledEpiLds <= tiled_lds_bytes(BM, BN), "slice fits in LDS");

  const int part = blockIdx.y;    // output part (uniform per workgroup)
  const int split = blockIdx.z;   // K split
  extern __shared__ __align__(16) uint16_t lds[];   // [2][A BMx64 | W BNx64]
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
  const int m0 = tm * BM, n0 = tn * BN;

  const int kper = K / gridDim.z;
  const int kbeg = split * kper;

  // ---- global -> LDS without registers (buffer_load ... lds).  One wave
  // instruction fills 1 KB of LDS: 16 tile rows of 4 16-byte chunks, lane l
  // landing at chunk l of the run.  Lane l takes row l / 4 of the run and,
  // so that the swizzle holds, global chunk (l % 4) ^ ((l / 8) & 3).  Each
  // instruction has its own buffer resource starting at its first row and
  // covering its rows that exist; the range check covers the VGPR (row,
  // chunk) and SGPR (k) offsets together, so rows past M (or past a W
  // matrix's end) read as zero.
  constexpr int LA = BM / 16 / NWAVES, LW = BN / 16 / NWAVES;   // loads per wave per stage
  static_assert(LA * 16 * NWAVES == BM && LW * 16 * NWAVES == BN, "whole load instructions");
  constexpr int STAGE = (BM + BN) * kTBK;   // elements of one ring slot
  constexpr int NS = tiled_stages(BM, BN);  // ring slots; NS - 1 stages in flight
  const int lrow = lane >> 2;
  const int gchunk = (lane & 3) ^ ((lane >> 3) & 3);
  // lane offset inside an instruction's 16 rows, and bytes per column of the
  // k offset: row-major, row lrow at the row stride and 2; fragment-major,
  // byte lrow * 64 of the 1 KB block and 32 (one block per 32 columns)
  const uint32_t a_voff = static_cast<uint32_t>((A.frag ? 64 : A.lda * 2) * lrow + gchunk * 16);
  const uint32_t w_voff = static_cast<uint32_t>((wfrag ? 64 : K * 2) * lrow + gchunk * 16);
  const uint32_t a_kb = A.frag ? 32 : 2, w_kb = wfrag ? 32 : 2;
  // bytes a 16-row run of row length ld may read: rows [0, valid) row-major;
  // the whole block fragment-major (its rows past the end hold zeros or
  // unused values)
  auto run_bytes = [](int valid, int ld, int frag) -> uint64_t {
    if (valid <= 0) return 0;
    return static_cast<uint64_t>(frag || valid > 16 ? 16 : valid) * ld * 2;
  };
  const int a_row0 = m0 + 16 * LA * wave;   // rows of A this wave loads
  const uint16_t* wptr[LW];   // first W row of each load instruction
  uint64_t wbytes[LW];
#pragma unroll
  for (int i = 0; i < LW; ++i) {
    const WRows wr = epi.wrows(part, n0 + 16 * (wave * LW + i), N);
    wptr[i] = wr.p;
    wbytes[i] = run_bytes(wr.valid, K, wfrag);
  }
  const int n_stages = kper / kTBK;
  // Loads are issued for stages 0, 1, 2, ... in order; the next stage's slab,
  // column and ring slot advance incrementally (stages past the last re-load
  // the last one, never read, so every step issues the same loads).  The
  // division below runs on the vector ALU: its results are marked uniform.
  int nx_stage = 0, nx_slot = 0, nx_k = kbeg;
  int nx_slab = __builtin_amdgcn_readfirstlane(kbeg / A.slab_k);
  int nx_col = __builtin_amdgcn_readfirstlane(kbeg - nx_slab * A.slab_k);
  const uint16_t* nx_sp = A.slab[nx_slab];   // reloaded only when the slab changes
  // A's buffer resources of the next loads (built where the step starts, so
  // that the scalar read of a new slab pointer is waited for before any of
  // the step's LDS reads is in flight)
  auto a_rsrc = [&](__amdgpu_buffer_rsrc_t* ars) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r0 = a_row0 + 16 * i;
      ars[i] = tile_rsrc(nx_sp + static_cast<int64_t>(min(r0, A.M)) * A.lda,
                         run_bytes(A.M - r0, A.lda, A.frag));
    }
  };
  auto load_one = [&](auto ic, const __amdgpu_buffer_rsrc_t* ars) {
    constexpr int i = decltype(ic)::value;
    lds_u16* slot = (lds_u16*)(lds) + nx_slot * STAGE;
    if constexpr (i < LA) {
      lds_u16* la = slot + wave * (LA * 512);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ars[i], la + i * 512, 16, a_voff, nx_col * a_kb,
                                               0, 0);
    } else {
      lds_u16* lw = slot + BM * kTBK + wave * (LW * 512);
      // (bound to a local: a resource temporary passed straight to the builtin
      // makes the host pass drop the kernel's launch stub)
      const __amdgpu_buffer_rsrc_t wrs = tile_rsrc(wptr[i - LA], wbytes[i - LA]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, lw + (i - LA) * 512, 16, w_voff, nx_k * w_kb,
                                               0, 0);
    }
  };
  auto advance = [&]() {
    nx_slot = nx_slot + 1 == NS ? 0 : nx_slot + 1;
    if (++nx_stage < n_stages) {
      nx_k += kTBK;
      nx_col += kTBK;
      if (nx_col == A.slab_k) {
        nx_col = 0;
        ++nx_slab;
        nx_sp = A.slab[nx_slab];
      }
    }
  };
  auto issue = [&]() {
    __amdgpu_buffer_rsrc_t ars[LA];
    a_rsrc(ars);
    tiled_static_for<LA + LW>([&](auto ic) { load_one(ic, ars); });
    advance();
  };

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = zero4();

  // Fragments of one stage: A rows wm*RW + i*16 + r16, W rows wn*CW + j*16 +
  // r16, chunk kg.  Fragment i sits 1 KB after fragment i - 1 (16 rows of
  // 64 bytes; the swizzle depends on r16 only), so each operand needs one
  // address and immediate offsets.
  struct Frags {
    u32x4_t a[MI], b[NJ];
  };
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u16*)(lds)));
  const uint32_t fa_off = lds_base + 2 * swz(wm * RW + r16, kg);
  const uint32_t fb_off = lds_base + 2 * (BM * kTBK + swz(wn * CW + r16, kg));
  auto read_frags = [&](Frags& f, int slot) {
    const uint32_t sb = static_cast<uint32_t>(slot * STAGE * 2);
    const uint32_t aa = fa_off + sb, ba = fb_off + sb;
    tile_read_frags(f.a, aa, std::make_integer_sequence<int, MI>{});
    tile_read_frags(f.b, ba, std::make_integer_sequence<int, NJ>{});
  };
  // wait for this wave's fragment reads; the fragments are operands, so no
  // use of them can be placed before the wait
  auto lgkm_wait = [&](Frags& f) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    tile_tie_all(f.a, std::make_integer_sequence<int, MI>{});
    tile_tie_all(f.b, std::make_integer_sequence<int, NJ>{});
  };
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        Frag8<uint16_t> fa, fb;
        fa.v = __builtin_bit_cast(uint4, f.a[i]);
        fb.v = __builtin_bit_cast(uint4, f.b[j]);
        acc[i][j] = mfma16(acc[i][j], fa, fb);
      }
  };
  // vmcnt(n) for n < 64 (lgkmcnt and expcnt not waited)
  constexpr int kVm = LA + LW;   // this wave's loads per stage
  static_assert(kVm * (tiled_stages(BM, BN) - 1) < 64, "vmcnt field");

  // Pipeline.  Before step st: stages st+1 .. st+NS-1 in flight, fragments
  // of st in registers (read from slot st % NS during step st-1, and waited
  // for there).  Step st: wait for stage st+1 (the later ones stay in
  // flight), barrier (stage st+1 complete; every wave is past its reads of
  // slot st % NS), then the MFMAs of st with the fragment reads of st+1 and
  // the loads of stage st+NS into that slot issued between them, then wait
  // for the fragment reads -- so values that cross the loop edge are always
  // complete.  Every slot but the one just freed holds a stage in flight or
  // unread: NS-1 stages of prefetch.
  constexpr int kAhead = NS - 1;                     // stages in flight before a wait
#pragma unroll
  for (int q = 0; q < NS; ++q) issue();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((NS - 1) * kVm));   // stage 0 landed
  __builtin_amdgcn_s_barrier();
  Frags f0, f1;
  // ring slot of the stage whose fragments are read next (stays on the last
  // stage's slot once past it)
  int rd_slot = 0, rd_stage = 0;
  auto next_read = [&]() {
    if (rd_stage + 1 < n_stages) {
      ++rd_stage;
      rd_slot = rd_slot + 1 == NS ? 0 : rd_slot + 1;
    }
    return rd_slot;
  };
  read_frags(f0, rd_slot);
  lgkm_wait(f0);
  // One step: the MFMAs of `cur`, with the fragment reads of the next stage
  // (into `nxt`) and then this step's loads spread evenly between all but the
  // last two of them (op o goes before MFMA o * SPREAD / NO), so that MFMAs
  // keep issuing while the LDS and memory queues take the rest.  Issuing the
  // reads all at once ahead of the MFMAs measured 5-6 % slower (2048- and
  // 8192-row fusion, 2048-row injection): the eight waves' reads then queue
  // at the LDS together and each wave's MFMAs wait behind its own reads.
  constexpr int NM = MI * NJ, NR = MI + NJ, NO = NR + kVm;
  constexpr int SPREAD = NM > 2 ? NM - 2 : 1;
  auto step = [&](Frags& cur, Frags& nxt) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm((kAhead - 1) * kVm));
    __builtin_amdgcn_s_barrier();
    const uint32_t sb = static_cast<uint32_t>(next_read() * STAGE * 2);
    const uint32_t aa = fa_off + sb, ba = fb_off + sb;
    __amdgpu_buffer_rsrc_t ars[LA];
    a_rsrc(ars);
    __builtin_amdgcn_sched_barrier(0);
    tiled_static_for<NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      tiled_static_for<NO>([&](auto oc) {
        constexpr int o = decltype(oc)::value;
        if constexpr (o * SPREAD / NO == m) {
          if constexpr (o < MI) {
            nxt.a[o] = tile_ds_read<o * 1024>(aa);
          } else if constexpr (o < NR) {
            nxt.b[o - MI] = tile_ds_read<(o - MI) * 1024>(ba);
          } else {
            load_one(std::integral_constant<int, o - NR>{}, ars);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      });
      constexpr int i = m / NJ, j = m % NJ;
      Frag8<uint16_t> fa, fb;
      fa.v = __builtin_bit_cast(uint4, cur.a[i]);
      fb.v = __builtin_bit_cast(uint4, cur.b[j]);
      acc[i][j] = mfma16(acc[i][j], fa, fb);
      __builtin_amdgcn_sched_barrier(0);
    });
    advance();
    lgkm_wait(nxt);
  };
  int st = 0;
  for (; st + 2 <= n_stages; st += 2) {
    step(f0, f1);
    step(f1, f0);
  }
  if (st < n_stages) mfmas(f0);   // odd stage count: the last stage
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));   // no load may land in the epilogue's LDS
  __syncthreads();

  // ---- epilogue: NSL slices of 64 rows.  Slice q takes MFMA rows
  // i in [q QI, (q+1) QI) of every wave: local row lr = wm * RUN +
  // (i - q QI) * 16 + kg * 4 + jj, stored as C[64][CT_LD] fp32.  C tile
  // (i, j) lane holds rows i*16 + kg*4 + jj, column j*16 + r16.
  float* ct = reinterpret_cast<float*>(lds);
  void* ext = ct + 64 * CT_LD;   // epilogue's own LDS (kTiledEpiLds bytes)
#pragma unroll
  for (int q = 0; q < NSL; ++q) {
#pragma unroll
    for (int ii = 0; ii < QI; ++ii)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          ct[(wm * RUN + ii * 16 + kg * 4 + jj) * CT_LD + wn * CW + j * 16 + r16] =
              acc[q * QI + ii][j][jj];
    __syncthreads();
    const TiledSlice sl{ct, CT_LD, m0 + q * RUN, RUN, RW, A.M, n0, N, BN, part, split, tn};
    epi.store(sl, ext, t, NT);
    __syncthreads();
  }
}

// ------------------------------------------------------------- epilogues
// Rows of a 64-row slice a wave reduces together in the training-loss epilogue.
constexpr int kTileRows = 8;
// Each epilogue maps W rows (wrows) and stores one slice (store); store is
// called by every thread of the workgroup and may use __syncthreads.

// One W matrix [N, K] (row n at W + n K).
__device__ __forceinline__ WRows wrows_single(const uint16_t* W, int K, int n, int N) {
  return WRows{W + static_cast<int64_t>(min(n, N)) * K, max(N - n, 0)};
}

// Coalesced fp32 store of a slice: out[row][n0 + c], 4 columns per thread.
__device__ __forceinline__ void store_slice_f32(const TiledSlice& s, float* out, int64_t ldo,
                                                int t, int nt) {
  const int tpr = s.bn / 4;   // threads per row
  const int c4 = (t % tpr) * 4;
  if (s.n0 + c4 >= s.N) return;
  for (int lr = t / tpr; lr < 64; lr += nt / tpr) {
    const int m = s.row(lr);
    if (m >= s.M) continue;
    const float4 v = *reinterpret_cast<const float4*>(s.c + lr * s.ld + c4);
    *reinterpret_cast<float4*>(out + static_cast<int64_t>(m) * ldo + s.n0 + c4) = v;
  }
}

// out[split][m][n] (float32 partial sums, slabs of slab_rows rows); N % 4 == 0.
struct TEpiStoreF32 {
  const uint16_t* W;
  int K;
  float* out;
  int64_t ldo, slab_rows;
  __device__ WRows wrows(int, int n, int N) const { return wrows_single(W, K, n, N); }
  __device__ void store(const TiledSlice& s, void*, int t, int nt) const {
    store_slice_f32(s, out + s.split * slab_rows * ldo, ldo, t, nt);
  }
};

// The rows of q, k and v stacked ([qd | kvd | kvd]): the QKV projection of a
// batch of blocks as fp32 partial slabs out[split][m][qd + 2 kvd].
struct TEpiQKVParts {
  const uint16_t* wq;
  const uint16_t* wk;
  const uint16_t* wv;
  int K, qd, kvd;
  float* out;
  int64_t ldo, slab_rows;
  __device__ WRows wrows(int, int n, int) const {
    if (n < qd) return wrows_single(wq, K, n, qd);
    if (n < qd + kvd) return wrows_single(wk, K, n - qd, kvd);
    return wrows_single(wv, K, n - qd - kvd, kvd);
  }
  __device__ void store(const TiledSlice& s, void*, int t, int nt) const {
    store_slice_f32(s, out + s.split * slab_rows * ldo, ldo, t, nt);
  }
};

// SwiGLU of a batch of blocks: the columns [0, bn/2) of tile tn are gate rows
// tn*bn/2 .. +bn/2, the columns [bn/2, bn) the up rows with the same indices;
// the epilogue writes h[m][tn*bn/2 + c] = silu(g) * u in bf16, row-major or
// fragment-major.
struct TEpiSwiGLUPair {
  const uint16_t* wg;
  const uint16_t* wu;
  int K, F, bn;
  uint16_t* h;
  int64_t ldh;   // row stride of h; fragment-major: its row length
  int frag;      // h fragment-major (the down projection's A operand)
  __device__ WRows wrows(int, int n, int) const {
    const int half = bn / 2, tn = n / bn, r = n % bn;
    const int f = tn * half + (r < half ? r : r - half);
    return wrows_single(r < half ? wg : wu, K, f, F);
  }
  __device__ void store(const TiledSlice& s, void*, int t, int nt) const {
    const int half = s.bn / 2, f0 = s.tile_n * half;
    const int c = t % half;
    if (f0 + c >= F) return;
    for (int lr = t / half; lr < 64; lr += nt / half) {
      const int m = s.row(lr);
      if (m >= s.M) continue;
      const float g = s.at(lr, c), u = s.at(lr, c + half);
      const int j = f0 + c;
      stf(h + (frag ? frag_major(m, j, static_cast<int>(ldh)) : static_cast<int64_t>(m) * ldh + j),
          g / (1.0f + expf(-g)) * u);
    }
  }
};

// LM head of a batch of blocks: per row, the largest logit among the tile's
// columns and its lowest column index -> part[m][tile] (value, index bits),
// reduced over tiles by the finalize kernel; optionally every logit.
// A launch may cover vocabulary rows [n_base, V) only (the tail of a split
// LM head); its tile i writes partial part_base + i of each row.
struct TEpiArgmax {
  const uint16_t* W;
  int K, V, n_parts;
  float2* part;
  float* dbg;   // [M][V] or null
  int n_base, part_base;
  __device__ WRows wrows(int, int n, int) const { return wrows_single(W, K, n_base + n, V); }
  __device__ void store(const TiledSlice& s, void*, int t, int nt) const {
    const int lane = t & 63, wave = t >> 6, nw = nt >> 6;
    for (int lr = wave; lr < 64; lr += nw) {   // one wave per row
      const int m = s.row(lr);
      if (m >= s.M) continue;
      float best = -INFINITY;
      int bi = 0x7fffffff;
      for (int c = lane; c < s.bn; c += 64) {
        const int n = n_base + s.n0 + c;
        if (n >= V) break;
        const float v = s.at(lr, c);
        if (dbg) dbg[static_cast<int64_t>(m) * V + n] = v;
        if (v > best) { best = v; bi = n; }   // columns grow: ">" keeps the lowest
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(best, o, 64);
        const int oi = __shfl_xor(bi, o, 64);
        if (better(ov, oi, best, bi)) { best = ov; bi = oi; }
      }
      if (lane == 0)
        part[static_cast<int64_t>(m) * n_parts + part_base + s.tile_n] =
            make_float2(best, __int_as_float(bi));
    }
  }
};

// Training-layout LM head: per row, over this tile's columns, the max logit,
// the sum of exp(z - max) and the label's logit (or -inf) ->
// part[m][n_parts] as float4 (max, sum, label logit, 0).  Row m is slot
// j = m % B of block m / B; slot 0 (the anchor) has no label.
struct TEpiLoss {
  const uint16_t* W;
  int K, V, n_parts, B;
  float4* part;
  const int32_t* labels;
  float* dbg;   // [M][V] or null
  int n_base, part_base;   // as in TEpiArgmax
  __device__ WRows wrows(int, int n, int) const { return wrows_single(W, K, n_base + n, V); }
  __device__ void store(const TiledSlice& s, void*, int t, int nt) const {
    const int lane = t & 63, wave = t >> 6, nw = nt >> 6;
    // one wave per row; a wave's rows (wave, wave + nw, ...) go kTileRows at
    // a time so that the rows' butterflies interleave (one row after another
    // left each level's LDS-permute latency exposed: training-layout LM head
    // 1431 -> 1331 us; the argmax epilogue measured slower that way, 376-382
    // -> 385-389 us at batch 16 over three alternated runs, and keeps one row
    // at a time)
    for (int lr0 = wave; lr0 < 64; lr0 += kTileRows * nw) {
      float mx[kTileRows], zl[kTileRows], sm[kTileRows];
#pragma unroll
      for (int q = 0; q < kTileRows; ++q) {
        mx[q] = -INFINITY;
        zl[q] = -INFINITY;
        const int lr = lr0 + q * nw;
        if (lr >= 64) continue;
        const int m = s.row(lr);
        if (m >= s.M) continue;
        const int j = m % B;
        const int lab = j > 0 ? labels[(m / B) * (B - 1) + j - 1] : -1;
        for (int c = lane; c < s.bn; c += 64) {
          const int n = n_base + s.n0 + c;
          if (n >= V) break;
          const float v = s.at(lr, c);
          if (dbg) dbg[static_cast<int64_t>(m) * V + n] = v;
          mx[q] = fmaxf(mx[q], v);
          if (n == lab) zl[q] = v;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
        for (int q = 0; q < kTileRows; ++q) {
          mx[q] = fmaxf(mx[q], __shfl_xor(mx[q], o, 64));
          zl[q] = fmaxf(zl[q], __shfl_xor(zl[q], o, 64));
        }
      }
#pragma unroll
      for (int q = 0; q < kTileRows; ++q) {
        sm[q] = 0.f;
        const int lr = lr0 + q * nw;
        if (lr >= 64 || s.row(lr) >= s.M) continue;
        for (int c = lane; c < s.bn; c += 64) {
          if (n_base + s.n0 + c >= V) break;
          sm[q] += expf(s.at(lr, c) - mx[q]);
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
#pragma unroll
        for (int q = 0; q < kTileRows; ++q) sm[q] += __shfl_xor(sm[q], o, 64);
      }
      if (lane == 0) {
#pragma unroll
        for (int q = 0; q < kTileRows; ++q) {
          const int lr = lr0 + q * nw;
          if (lr >= 64) continue;
          const int m = s.row(lr);
          if (m >= s.M) continue;
          part[static_cast<int64_t>(m) * n_parts + part_base + s.tile_n] =
              make_float4(mx[q], sm[q], zl[q], 0.f);
        }
      }
    }
  }
};

// KV injection over rows of context features.  Part p = 2 * layer + (0: K,
// 1: V); its N = Hkv * d columns are that layer's k (or v) projection.  K
// gets RoPE at the row's position (the pair partner of column c is c + d/2);
// V is stored transposed.  A tile's columns hold whole heads (bn % d == 0).
// A launch may cover parts [part_base, part_base + gridDim.y) only.
struct TEpiInject {
  const uint16_t* wk[kMaxLayers];
  const uint16_t* wv[kMaxLayers];
  uint16_t* kc[kMaxLayers];
  uint16_t* vc[kMaxLayers];
  int K, d;
  int64_t cap;
  RopeFreq freq;
  SeqTable seq;
  int part_base;
  __device__ WRows wrows(int part, int n, int N) const {
    part += part_base;
    return wrows_single((part & 1) ? wv[part >> 1] : wk[part >> 1], K, n, N);
  }
  __device__ void store(const TiledSlice& s, void* ext, int t, int nt) const {
    // per local row: position and cache row (rows are grouped by sequence)
    int* pos_t = static_cast<int*>(ext);
    int64_t* row_t = reinterpret_cast<int64_t*>(pos_t + 64);
    if (t < 64) {
      // rows past M, and rows a sequence does not append, store nothing
      const int m = s.row(t);
      int b = 0, pos = 0;
      const bool keep = m < s.M && inject_row(seq, m, b, pos);
      pos_t[t] = pos;
      row_t[t] = keep ? seq.off[b] + pos : -1;
    }
    __syncthreads();
    const int part = s.part + part_base;
    if ((part & 1) == 0) {
      uint16_t* kd = kc[part >> 1];
      const int half = d / 2, pairs = s.bn / 2;
      const int q = t % pairs;                  // RoPE pair of the tile
      const int hl = q / half, c = q % half;    // head inside the tile, pair index
      const int col = hl * d + c;
      const int head = (s.n0 + col) / d;
      if (s.n0 + col >= s.N) return;
      const double inv = freq.inv[c];
      for (int lr = t / pairs; lr < 64; lr += nt / pairs) {
        if (row_t[lr] < 0) continue;
        float cs, sn;
        rope_cos_sin(pos_t[lr], inv, cs, sn);
        const float x0 = s.at(lr, col), x1 = s.at(lr, col + half);
        uint16_t* dst = kd + (static_cast<int64_t>(head) * cap + row_t[lr]) * d + c;
        stf(dst, x0 * cs - x1 * sn);
        stf(dst + half, x1 * cs + x0 * sn);
      }
    } else {
      uint16_t* vt = vc[part >> 1];
      const int lr = t & 63;
      const int64_t r = row_t[lr];
      if (r < 0) return;
      for (int col = t >> 6; col < s.bn && s.n0 + col < s.N; col += nt >> 6)
        stf(vt + static_cast<int64_t>(s.n0 + col) * cap + r, s.at(lr, col));
    }
  }
};

}  // namespace dflash
