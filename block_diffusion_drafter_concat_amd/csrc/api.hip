// C ABI front end of libdflash: argument checks, workspace layout and the
// launch sequence of every call.  All checks run before the first launch, so a
// rejected call has no side effects.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <atomic>
#include <mutex>
#include <new>

#include <hip/hip_ext.h>

#include "../../include/dflash.h"
#include "gemm_epilogues.h"
#include "gemm_skinny.h"
#include "gemm_tiled.h"
#include "kernels.h"
#include "kernels_attn.h"

using namespace dflash;

struct dflash_handle {
  dflash_config cfg;
  dflash_weights w;
  dflash_layer_weights layers[DFLASH_MAX_LAYERS];
  dflash_timing_point timing[32];
  int n_timing;
  // fragment-major copies of the bf16 GEMM weights in caller memory
  // (dflash_pack_weights): the LDS-tiled GEMMs read these while `packed`
  bool packed;
  dflash_layer_weights pk_layers[DFLASH_MAX_LAYERS];   // wq, wk, wv, wo, wg, wu, wd
  const void* pk_fc;
  const void* pk_lm;
};

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline dflash_status hip_status(hipError_t e) { return e == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP; }
#define DF_HIP(expr)                                     \
  do {                                                   \
    hipError_t e_ = (expr);                              \
    if (e_ != hipSuccess) return DFLASH_ERR_HIP;         \
  } while (0)

// Attention split: chunks per (sequence, kv head) at most kMaxAttnChunks, and
// at most kAttnSlotBudget partial slots over the whole batch (or two chunks
// per (sequence, kv head) if the batch is larger).  The bf16 block-attention
// kernel fits three workgroups on a compute unit, so kAttnConcurrent (3 x 256
// CUs) of them run at once; attn_chunk() picks the chunk length.
constexpr int kMaxAttnChunks = 128;
constexpr int kAttnSlotBudget = 2048;
constexpr int kAttnConcurrent = 768;
constexpr int kAttnWgOverhead = 64;   // fixed cost of a workgroup, in keys
int64_t attn_slots(int batch, int n_kv) {
  const int64_t all = static_cast<int64_t>(batch) * n_kv;
  // at least two per entry: a training-layout block always has its own chunk
  // besides at least one context chunk
  return std::min<int64_t>(all * kMaxAttnChunks, std::max<int64_t>(kAttnSlotBudget, 2 * all));
}
// Keys per attention workgroup: a multiple of 128, at most max_c chunks per
// (sequence, kv head), chosen to minimise an estimated makespan in units of
// keys.  A workgroup costs (its keys + kAttnWgOverhead); the dispatcher hands
// workgroups, in grid order, to the first of kAttnConcurrent free places.
//  - Near-uniform batch (longest <= 1.25 x shortest): every workgroup is a
//    full chunk, so the work runs in whole rounds:
//        ceil(workgroups / kAttnConcurrent) * (chunk + overhead).
//  - Ragged batch: one round costs the longest job; over several rounds the
//    late workgroups fill the gaps that short ones leave, and the remaining
//    imbalance shrinks as the workgroups grow more numerous:
//        total / kAttnConcurrent + 0.215 * (chunk + overhead) * kAttnConcurrent / workgroups
//    (the 0.215 fitted to the ragged batch-16 workload, contexts 512..8192).
// Ties go to the longer chunk (fewer partials to merge).
int attn_chunk(const int32_t* keys, int nb, int n_kv, int max_keys, int max_c) {
  int lo = 128, min_keys = max_keys;
  while ((max_keys + lo - 1) / lo > max_c) lo += 128;
  for (int b = 0; b < nb; ++b) min_keys = std::min(min_keys, static_cast<int>(keys[b]));
  const bool uniform = 4 * static_cast<int64_t>(max_keys) <= 5 * static_cast<int64_t>(min_keys);
  const int hi = std::max(lo, (max_keys + 127) / 128 * 128);
  int best = hi;
  double best_cost = -1.0;
  for (int c = hi; c >= lo; c -= 128) {
    int64_t wgs = 0, work = 0;
    for (int b = 0; b < nb; ++b) {
      const int64_t n = (keys[b] + c - 1) / c;
      wgs += n;
      work += keys[b] + n * kAttnWgOverhead;
    }
    wgs *= n_kv;
    work *= n_kv;
    const double job = c + kAttnWgOverhead;
    double cost;
    if (uniform) cost = static_cast<double>((wgs + kAttnConcurrent - 1) / kAttnConcurrent) * job;
    else if (wgs <= kAttnConcurrent) cost = job;
    else cost = static_cast<double>(work) / kAttnConcurrent + 0.215 * job * kAttnConcurrent / wgs;
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = c;
    }
  }
  return best;
}

// Longest-first order for a ragged batch (host-held lengths, inference).
// Workgroups go, in grid order, to the first of kAttnConcurrent free places;
// listing every full chunk first and then the partial last chunks, largest
// first, is a longest-first list schedule, in which the short jobs fill the
// gaps the long ones leave.  attn_lpt_cost() is that schedule's makespan in
// keys (a workgroup costs its keys + kAttnWgOverhead): after the full chunks
// the places sit at two load levels; the partial chunks then go one by one to
// the least loaded place (a heap).  *n_items = (sequence, chunk) entries.
// extra > 0 (training layout): every entry has one more chunk of `extra` keys
// (its block's own keys) after its context chunks.
double attn_lpt_cost(const int32_t* keys, int nb, int n_kv, int chunk, int extra, int* n_items) {
  int64_t full = 0;
  int items = 0, np = 0;
  int part[2 * DFLASH_MAX_BATCH];
  for (int b = 0; b < nb; ++b) {
    const int nf = keys[b] / chunk, r = keys[b] - nf * chunk;
    full += nf;
    items += nf + (r > 0 ? 1 : 0);
    if (r > 0) part[np++] = r;
    if (extra > 0) {
      ++items;
      part[np++] = extra;
    }
  }
  *n_items = items;
  std::sort(part, part + np, std::greater<int>());
  const int64_t F = full * n_kv, S = kAttnConcurrent;
  const double job = chunk + kAttnWgOverhead;
  const int64_t q = F / S, rem = F % S;
  double load[kAttnConcurrent];   // a min-heap of the places' loads
  for (int64_t i = 0; i < S; ++i) load[i] = static_cast<double>(i < rem ? q + 1 : q) * job;
  std::make_heap(load, load + S, std::greater<double>());
  for (int k = 0; k < np; ++k)
    for (int g = 0; g < n_kv; ++g) {
      std::pop_heap(load, load + S, std::greater<double>());
      load[S - 1] += part[k] + kAttnWgOverhead;
      std::push_heap(load, load + S, std::greater<double>());
    }
  return *std::max_element(load, load + S);
}

// For a ragged batch: the chunk length (a multiple of 128, at most max_c
// chunks per entry, at most kAttnOrderMax entries) that minimises that
// makespan, and the order (full chunks by sequence, then the partial ones --
// and the block chunks of the training layout -- by size, largest first, ties
// by sequence).  Near-uniform batches keep the grid order and attn_chunk's
// choice.
void attn_plan_order(const int32_t* keys, int nb, int n_kv, int max_keys, int max_c, int extra,
                     int* chunk, AttnArgs* aa) {
  if (max_c < 1) return;
  int min_keys = max_keys;
  for (int b = 0; b < nb; ++b) min_keys = std::min(min_keys, static_cast<int>(keys[b]));
  if (4 * static_cast<int64_t>(max_keys) <= 5 * static_cast<int64_t>(min_keys)) return;
  int lo = 128;
  while ((max_keys + lo - 1) / lo > max_c) lo += 128;
  // fewer than kAttnOrderMax entries needs chunk >= sum(keys) / kAttnOrderMax
  int64_t total = 0;
  for (int b = 0; b < nb; ++b) total += keys[b];
  const int64_t need = (total + kAttnOrderMax - 1) / kAttnOrderMax;
  lo = std::max<int64_t>(lo, (need + 127) / 128 * 128);
  const int hi = std::max(lo, (max_keys + 127) / 128 * 128);
  // at most 64 candidates, evenly spaced (host time stays well under a ms)
  const int step = std::max(128, ((hi - lo) / 64 + 127) / 128 * 128);
  int best = -1;
  double best_cost = 0.0;
  for (int c = hi; c >= lo; c -= step) {
    int items = 0;
    const double cost = attn_lpt_cost(keys, nb, n_kv, c, extra, &items);
    if (items > kAttnOrderMax) continue;
    if (best < 0 || cost < best_cost) {
      best = c;
      best_cost = cost;
    }
  }
  if (best < 0) return;
  *chunk = best;
  int n = 0;
  for (int b = 0; b < nb; ++b)
    for (int c = 0; c < keys[b] / best; ++c) aa->order[n++] = static_cast<uint16_t>(b * 128 + c);
  // the rest: (size, entry, chunk), largest first, then by entry
  struct Rest {
    int size, b, c;
  };
  Rest rest[2 * DFLASH_MAX_BATCH];
  int np = 0;
  for (int b = 0; b < nb; ++b) {
    const int nf = keys[b] / best, r = keys[b] - nf * best;
    if (r > 0) rest[np++] = Rest{r, b, nf};
    if (extra > 0) rest[np++] = Rest{extra, b, nf + (r > 0 ? 1 : 0)};
  }
  std::stable_sort(rest, rest + np, [](const Rest& x, const Rest& y) { return x.size > y.size; });
  for (int k = 0; k < np; ++k) aa->order[n++] = static_cast<uint16_t>(rest[k].b * 128 + rest[k].c);
  aa->n_order = n;
}

// Rows per launch of the weight-streaming GEMM.
constexpr int kMaxRowsPerLaunch = 128;
// LM-head tiles (32 vocabulary rows each) walked by one workgroup.
constexpr int kLmTilesPerWg = 1;

struct Dims {
  int L, H, Hq, Hkv, d, F, V, nf, G, qd, kvd;
};
Dims dims(const dflash_config& c) {
  Dims r;
  r.L = c.n_layers; r.H = c.hidden; r.Hq = c.n_q_heads; r.Hkv = c.n_kv_heads; r.d = c.head_dim;
  r.F = c.ffn; r.V = c.vocab; r.nf = c.n_feat_layers; r.G = c.n_q_heads / c.n_kv_heads;
  r.qd = c.n_q_heads * c.head_dim; r.kvd = c.n_kv_heads * c.head_dim;
  return r;
}

struct GemmPlan {
  int tiles_qkv, tiles_o, tiles_gu, tiles_d, tiles_lm, tiles_fc, tiles_inj;
  int ks_o, ks_d;      // K-splits of the O and down projections (partials -> next norm)
  int ks_qkv;          // K-split of the bf16 QKV projection (partials -> RoPE finish)
  int wg_lm;           // LM-head workgroups
};

// K-split of a partial-product GEMM: enough workgroups (>= 512) to keep bytes
// in flight on 256 CUs while every wave still streams >= 256 k (4 waves).
int pick_ksplit(int n_tiles, int K) {
  int ks = 1;
  while (ks < 8 && n_tiles * ks < 512 && K % (4 * ks * 2 * 32) == 0 && K / (4 * ks * 2) >= 256)
    ks *= 2;
  return ks;
}
// Rows from which bf16 fusion / injection use the LDS-tiled GEMM, and its
// tile for them (8 waves, 2 x 4: two per SIMD, 128 accumulators each).
constexpr int kTiledMinRows = 129;
constexpr int kPreBM = 256, kPreBN = 256;
// Block rows (batch x slots) from which a bf16 draft runs its layer GEMMs and
// LM head on the LDS-tiled GEMM instead of the weight-streaming one.
constexpr int kMidMinRows = 64;

// Mid-M plan: K splits of the partial-slab GEMMs.  A split is taken while the
// workgroups stay under ~1.25 per compute unit and the fp32 partial slabs it
// adds stay under half the weight bytes.
struct MidPlan {
  int ks_qkv, ks_o, ks_d;
};
int mid_ksplit(int64_t tiles, int K, int64_t w_bytes, int64_t slab_bytes, int max_ks = 8) {
  int ks = 1;
  while (ks < max_ks && tiles * ks * 2 <= 320 && K % (ks * 2 * kTBK) == 0 &&
         ks * 2 * slab_bytes <= w_bytes / 2)
    ks *= 2;
  return ks;
}
MidPlan mid_plan(const Dims& D, int M) {
  const int64_t nq = D.qd + 2 * D.kvd;
  MidPlan p;
  p.ks_qkv = mid_ksplit((nq + 127) / 128, D.H, nq * D.H * 2, static_cast<int64_t>(M) * nq * 4);
  // the residual-norm kernel sums up to 8 slabs for H <= 4096, 4 above
  const int max_rn = D.H <= 4096 ? 8 : 4;
  // the O projection takes 128-row tiles above 128 rows (launch_mid_o)
  const int tm_o = M > 128 ? (M + 127) / 128 : 1;
  p.ks_o = mid_ksplit(tm_o * ((D.H + 127) / 128), D.qd, static_cast<int64_t>(D.H) * D.qd * 2,
                      static_cast<int64_t>(M) * D.H * 4, max_rn);
  p.ks_d = mid_ksplit((D.H + 127) / 128, D.F, static_cast<int64_t>(D.H) * D.F * 2,
                      static_cast<int64_t>(M) * D.H * 4, max_rn);
  return p;
}

// Fusion K-split.  Weight-streaming path: only for short incremental calls.
// Tiled path: split until the 256 x 256 tiles times the split fill the 256
// compute units once (at most 8 partial slabs, whole 64-wide k stages).
int fuse_ksplit(const dflash_handle* h, int64_t T) {
  const Dims D = dims(h->cfg);
  const int K = D.nf * D.H;
  if (h->cfg.dtype == DFLASH_BF16 && T >= kTiledMinRows) {
    const int64_t tiles = ((T + kPreBM - 1) / kPreBM) * ((D.H + kPreBN - 1) / kPreBN);
    const int max_ks = D.H <= 4096 ? 8 : 4;   // partial slabs the norm kernel sums
    int ks = 1;
    while (ks < max_ks && 2 * ks * tiles <= 256 && K % (2 * ks * kTBK) == 0) ks *= 2;
    return ks;
  }
  return T <= 64 ? pick_ksplit(D.H / 32, K) : 1;
}

// Largest ks * T over every call size T <= t_max (ks is constant where the
// row-tile count is, so only the largest T of each such range matters).
int64_t fuse_part_rows(const dflash_handle* h, int64_t t_max) {
  int64_t best = 0;
  auto consider = [&](int64_t T) {
    T = T < t_max ? T : t_max;
    if (T > 0) best = std::max(best, fuse_ksplit(h, T) * T);
  };
  consider(64);
  consider(kTiledMinRows - 1);
  for (int64_t tm = 1; (tm - 1) * kPreBM < t_max; ++tm) consider(tm * kPreBM);
  consider(t_max);
  return best;
}

GemmPlan gemm_plan(const Dims& D) {
  GemmPlan g;
  g.tiles_qkv = (D.qd + 2 * D.kvd) / 32;
  g.tiles_o = D.H / 32;
  g.tiles_gu = D.F / 16;
  g.tiles_d = D.H / 32;
  g.tiles_lm = (D.V + 31) / 32;
  g.tiles_fc = D.H / 32;
  g.tiles_inj = D.L * 2 * D.kvd / 32;
  g.ks_o = pick_ksplit(g.tiles_o, D.qd);
  g.ks_d = pick_ksplit(g.tiles_d, D.F);
  g.ks_qkv = pick_ksplit(g.tiles_qkv, D.H);
  g.wg_lm = (g.tiles_lm + kLmTilesPerWg - 1) / kLmTilesPerWg;
  return g;
}

// ------------------------------------------------------------- workspace
// Every call lays out its own scratch from offset 0 with sizes that grow with
// (batch, block, tokens); dflash_workspace_size takes the largest.
struct Layout {
  size_t x_off, u_off, q_off, o_off, h_off, part_off, qkvp_off, lm_off, bkv_off, ao_off, aml_off,
      ver_off;
  size_t total;
};

Layout layout(const dflash_handle* h, int max_batch, int max_block, int64_t max_tokens) {
  const Dims D = dims(h->cfg);
  const size_t es = h->cfg.dtype == DFLASH_BF16 ? 2 : 4;
  const size_t M = static_cast<size_t>(max_batch) * max_block;
  const size_t T = static_cast<size_t>(max_tokens > 0 ? max_tokens : 1);
  const GemmPlan g = gemm_plan(D);
  Layout L{};
  size_t off = 0;
  L.x_off = off;    off += align_up(M * D.H * 4);
  // u and h may be stored fragment-major: whole 16-row groups
  const size_t M16 = (M + 15) / 16 * 16;
  L.u_off = off;    off += align_up(M16 * D.H * es);
  L.q_off = off;    off += align_up(M * D.qd * es);
  L.o_off = off;    off += align_up(M16 * D.qd * es);
  L.h_off = off;    off += align_up(M16 * D.F * es);
  // K-split partial slabs: O / down projections [ks][M][H], fusion [ks][T][H]
  size_t part = static_cast<size_t>(g.ks_o > g.ks_d ? g.ks_o : g.ks_d) * M * D.H * 4;
  const size_t pf = static_cast<size_t>(fuse_part_rows(h, static_cast<int64_t>(T))) * D.H * 4;
  part = pf > part ? pf : part;
  size_t qkvp = 0;
  if (h->cfg.dtype == DFLASH_BF16 && M >= static_cast<size_t>(kMidMinRows)) {
    // the mid-M path at every row count up to M (splits shrink as M grows)
    for (size_t m = kMidMinRows; m <= M; ++m) {
      const MidPlan mp = mid_plan(D, static_cast<int>(m));
      part = std::max(part, static_cast<size_t>(std::max(mp.ks_o, mp.ks_d)) * m * D.H * 4);
      qkvp = std::max(qkvp, static_cast<size_t>(mp.ks_qkv) * m * (D.qd + 2 * D.kvd) * 4);
    }
  }
  {
    // the training layout's QKV on the weight-streaming split path: bf16
    // below the mid-M path, float32 at any row count
    const size_t ms = h->cfg.dtype == DFLASH_BF16 ? std::min(M, static_cast<size_t>(kMidMinRows - 1)) : M;
    qkvp = std::max(qkvp, static_cast<size_t>(g.ks_qkv) * ms * (D.qd + 2 * D.kvd) * 4);
  }
  L.part_off = off; off += align_up(part);
  L.qkvp_off = off; off += align_up(qkvp);
  L.lm_off = off;   off += align_up(M * g.wg_lm * 16);   // argmax: 8 B, training loss: 16 B
  // training layout: block K and V^T, kTrainSlab rows per block
  L.bkv_off = off;  off += align_up(2 * static_cast<size_t>(D.Hkv) * max_batch * kTrainSlab * D.d * es);
  const size_t qr = static_cast<size_t>((D.G * max_block + 15) / 16 * 16);
  const size_t slots = static_cast<size_t>(attn_slots(max_batch, D.Hkv));
  L.ao_off = off;  off += align_up(slots * qr * D.d * 4);
  L.aml_off = off; off += align_up(slots * qr * 8);
  L.ver_off = off; off += align_up(verify_ws_bytes(max_batch, max_block, D.V));
  L.total = off;
  return L;
}

// Record the caller's timing event for (section, layer), if one is set.
hipError_t mark(const dflash_handle* h, int section, int layer, bool stop, hipStream_t st) {
  for (int i = 0; i < h->n_timing; ++i) {
    const dflash_timing_point& p = h->timing[i];
    if (p.section == section && (p.layer == layer || layer < 0)) {
      hipError_t e = hipEventRecord(static_cast<hipEvent_t>(stop ? p.ev_stop : p.ev_start), st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}
#define DF_MARK(sec, layer, stop) DF_HIP(mark(h, sec, layer, stop, st))

// The caller's events for (section, layer), if that point is set.
bool timing_events(const dflash_handle* h, int section, int layer, hipEvent_t* a, hipEvent_t* b) {
  for (int i = 0; i < h->n_timing; ++i) {
    const dflash_timing_point& p = h->timing[i];
    if (p.section == section && (p.layer == layer || layer < 0)) {
      *a = static_cast<hipEvent_t>(p.ev_start);
      *b = static_cast<hipEvent_t>(p.ev_stop);
      return true;
    }
  }
  return false;
}

// RoPE inverse frequencies theta^(-2i/d) in double.
RopeFreq rope_freq(const dflash_config& c) {
  RopeFreq f{};
  for (int i = 0; i < c.head_dim / 2 && i < 64; ++i)
    f.inv[i] = pow(static_cast<double>(c.rope_theta),
                   -2.0 * static_cast<double>(i) / static_cast<double>(c.head_dim));
  return f;
}

template <typename P> P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// ------------------------------------------------------------- GEMM launcher
// One launch over rows [A.m0, A.m0 + A.mc): ksplit workgroups per tile group
// (grid.y), nw waves per workgroup, tiles_per_wg steps of pt pair tiles each.
// pt = 2 is taken only for one 16-row group (mc <= 16); skinny_pt() says
// which pt a launch runs with, for epilogues that count workgroups.
inline int skinny_pt(int pt, int mc) { return pt == 2 && mc <= 16 ? 2 : 1; }
inline int skinny_wgs(int n_tiles, int tiles_per_wg, int pt) {
  return ((n_tiles + pt - 1) / pt + tiles_per_wg - 1) / tiles_per_wg;
}
template <typename T, int NW, class Epi>
hipError_t launch_skinny_nw(const AOperand<T>& A, int K, int n_tiles, int tiles_per_wg,
                            int ksplit, const Epi& epi, hipStream_t st, int pt = 1,
                            hipEvent_t ev0 = nullptr, hipEvent_t ev1 = nullptr) {
  const int kper = K / (NW * ksplit);
  // the kernel's slab pick: 32-column steps never straddle slabs, and its
  // 40-bit reciprocal of slab_k is exact for columns below K
  if (A.slab_k % 32 != 0 || static_cast<int64_t>(K) * A.slab_k >= (int64_t{1} << 40))
    return hipErrorInvalidValue;
  const int mc = A.mc;
  const bool slabs = A.slab_k < K;   // the fusion input: several feature slabs along K
  pt = skinny_pt(pt, mc);
  dim3 grid(skinny_wgs(n_tiles, tiles_per_wg, pt), ksplit);
  // with timing events, the dispatch records them itself (the span is the
  // kernel's execution, without the packets an event record adds)
  AOperand<T> a_arg = A;
  int k_arg = K, nt_arg = n_tiles, tpw_arg = tiles_per_wg;
  Epi e_arg = epi;
  void* argv[] = {&a_arg, &k_arg, &nt_arg, &tpw_arg, &e_arg};
  hipError_t ext = hipSuccess;
#define DF_SK2(MT, U, PT, SL)                                                                   \
  do {                                                                                          \
    if (ev0)                                                                                    \
      ext = hipExtLaunchKernel(                                                                 \
          reinterpret_cast<const void*>(&skinny_gemm_kernel<T, MT, U, NW, PT, Epi, SL>), grid,   \
          dim3(NW * 64), argv, 0, st, ev0, ev1, 0);                                             \
    else                                                                                        \
      skinny_gemm_kernel<T, MT, U, NW, PT, Epi, SL><<<grid, NW * 64, 0, st>>>(A, K, n_tiles,     \
                                                                              tiles_per_wg, epi); \
  } while (0)
#define DF_SK(MT, U, PT)                  \
  do {                                    \
    if (slabs) DF_SK2(MT, U, PT, true);   \
    else DF_SK2(MT, U, PT, false);        \
  } while (0)
  if (mc <= 16) {
    if (pt == 2) {
      if (kper % 64 == 0) DF_SK(1, 2, 2);
      else DF_SK(1, 1, 2);
    } else {
      if (kper % 64 == 0) DF_SK(1, 2, 1);
      else DF_SK(1, 1, 1);
    }
  } else if (mc <= 32) {
    if (kper % 64 == 0) DF_SK(2, 2, 1);
    else DF_SK(2, 1, 1);
  } else if (mc <= 64) {
    DF_SK(4, 1, 1);
  } else if (mc <= 128) {
    DF_SK(8, 1, 1);
  } else {
    return hipErrorInvalidValue;
  }
#undef DF_SK
#undef DF_SK2
  if (ext != hipSuccess) return ext;
  return hipGetLastError();
}

// Rows [0, M) in launches of at most 128 rows; `per_launch` adjusts
// per-launch epilogue state.  4 waves per workgroup, 2 k-steps per stage: the
// best streaming configuration measured on MI355X for these shapes.
template <typename T, class Epi, class PerLaunch>
hipError_t run_rows(AOperand<T> A, int K, int n_tiles, int tiles_per_wg, int ksplit, Epi epi,
                    hipStream_t st, PerLaunch per_launch, int nw = 4, int pt = 1) {
  if (nw == 8 && K % (8 * ksplit * 32) != 0) nw = 4;
  for (int m0 = 0, li = 0; m0 < A.M; m0 += kMaxRowsPerLaunch, ++li) {
    A.m0 = m0;
    A.mc = A.M - m0 < kMaxRowsPerLaunch ? A.M - m0 : kMaxRowsPerLaunch;
    per_launch(epi, li);
    hipError_t e = nw == 8
                       ? launch_skinny_nw<T, 8, Epi>(A, K, n_tiles, tiles_per_wg, ksplit, epi, st, pt)
                       : launch_skinny_nw<T, 4, Epi>(A, K, n_tiles, tiles_per_wg, ksplit, epi, st, pt);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
// wfrag: the epilogue's W pointers are packed (fragment-major) weights.
template <int BM, int BN, int WM, int WN, class Epi>
hipError_t launch_tiled_cfg(const AOperand<uint16_t>& A, int N, int K, int parts, int ksplit,
                            const Epi& epi, hipStream_t st, bool wfrag) {
  if (A.frag && A.slab_k != K) return hipErrorInvalidValue;   // fragment-major: one slab
  auto kern = &tiled_gemm_kernel<BM, BN, WM, WN, Epi>;
  constexpr size_t lds = tiled_lds_bytes(BM, BN);
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_dynamic_lds_once(lds_set, reinterpret_cast<const void*>(kern),
                                            static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const int tm = (A.M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  kern<<<dim3(tm * tn, parts, ksplit), WM * WN * 64, lds, st>>>(A, N, K, tm, tn, wfrag ? 1 : 0,
                                                                 epi);
  return hipGetLastError();
}

// Prefill fusion / injection: 256 x 256 tiles.
template <class Epi>
hipError_t launch_tiled(const AOperand<uint16_t>& A, int N, int K, int parts, int ksplit,
                        const Epi& epi, hipStream_t st, bool wfrag) {
  return launch_tiled_cfg<kPreBM, kPreBN, 2, 4>(A, N, K, parts, ksplit, epi, st, wfrag);
}

// LM head of a batch of blocks on the tiled GEMM.  One workgroup per compute
// unit fits (LDS), so 256-column tiles run in rounds of kCUs tiles; when the
// last round would be short, the vocabulary rows past the whole rounds go to
// a second launch that fits in one round: above 128 rows on 128 x 256 tiles
// (the two row tiles of a W panel share it through L2; batch 16: 594 tiles =
// 2.3 rounds become 512 tiles + 164 of 128 x 256, 372 against 383 us with
// 163 of 256 x 128, whose 128 x 32 wave tiles read the most LDS per MFMA),
// else on 128-column tiles.  `make(n_base, part_base)` builds the epilogue of
// one launch.
constexpr int kCUs = 256;   // compute units of the MI355X
struct LmSplit {
  int whole;     // 256-column tiles of the first launch (all of them when not split)
  int n_tail;    // vocabulary rows of the second launch (0: not split)
  int n_parts;   // per-row partials of both launches
  int tail_bn;   // column tile of the second launch: 256 (on 128-row tiles) or 128
};
inline LmSplit lm_split(int M, int V) {
  const int bm = M <= 64 ? 64 : M <= 128 ? 128 : 256;
  const int tm = (M + bm - 1) / bm;
  const int ct = (V + 255) / 256;
  const int whole = (tm * ct / kCUs) * kCUs / tm;   // 256-column tiles in whole rounds
  const int n_tail = V - whole * 256;
  if (whole < 1 || n_tail <= 0) return LmSplit{ct, 0, ct, 256};
  if (M > 128) {
    const int tm2 = (M + 127) / 128, ct2 = (n_tail + 255) / 256;
    if (tm2 * ct2 <= kCUs) return LmSplit{whole, n_tail, whole + ct2, 256};
  }
  const int ct_tail = (n_tail + 127) / 128;
  if (tm * ct_tail > kCUs) return LmSplit{ct, 0, ct, 256};
  return LmSplit{whole, n_tail, whole + ct_tail, 128};
}

// A batch of blocks (M = 64 .. 256 rows): the row tile covers M.
template <int BN, class Epi>
hipError_t launch_mid(const AOperand<uint16_t>& A, int N, int K, int ksplit, const Epi& epi,
                      hipStream_t st, bool wfrag) {
  if (A.M <= 64) return launch_tiled_cfg<64, BN, 1, 4>(A, N, K, 1, ksplit, epi, st, wfrag);
  if (A.M <= 128) return launch_tiled_cfg<128, BN, 2, 4>(A, N, K, 1, ksplit, epi, st, wfrag);
  return launch_tiled_cfg<256, BN, 2, 4>(A, N, K, 1, ksplit, epi, st, wfrag);
}

// The O projection of a batch of blocks: above 128 rows, 128-row tiles (two
// or more row tiles share each W column tile through L2 -- tiles go to XCDs
// in groups of row tiles -- and the grid grows with them).  Measured at 256
// block rows: 20.5 against 26.8 us per layer on 256-row tiles; at 1024 rows
// 51 against 71 us.  The gate/up and down projections measured slower that
// way (81 -> 100 and 51 -> 63 us at 256 rows) and keep the row tile = M.
template <class Epi>
hipError_t launch_mid_o(const AOperand<uint16_t>& A, int N, int K, int ksplit, const Epi& epi,
                        hipStream_t st, bool wfrag) {
  if (A.M <= 128) return launch_mid<128>(A, N, K, ksplit, epi, st, wfrag);
  return launch_tiled_cfg<128, 128, 2, 4>(A, N, K, 1, ksplit, epi, st, wfrag);
}

// LM head over rows A (M = A.M) on the tiled GEMM, split as lm_split says.
template <class MakeEpi>
hipError_t launch_lm_tiled(const AOperand<uint16_t>& A, int V, int K, MakeEpi make,
                           hipStream_t st, bool wfrag) {
  const LmSplit sp = lm_split(A.M, V);
  if (sp.n_tail == 0) return launch_mid<256>(A, V, K, 1, make(0, 0), st, wfrag);
  hipError_t e = launch_mid<256>(A, sp.whole * 256, K, 1, make(0, 0), st, wfrag);
  if (e != hipSuccess) return e;
  if (sp.tail_bn == 256)
    return launch_tiled_cfg<128, 256, 2, 4>(A, sp.n_tail, K, 1, 1, make(sp.whole * 256, sp.whole),
                                            st, wfrag);
  return launch_mid<128>(A, sp.n_tail, K, 1, make(sp.whole * 256, sp.whole), st, wfrag);
}

struct NoPerLaunch {
  template <class E> void operator()(E&, int) const {}
};

template <typename T>
AOperand<T> a_single(const void* p, int64_t lda, int K, int M) {
  AOperand<T> A{};
  for (int i = 0; i < 6; ++i) A.slab[i] = static_cast<const T*>(p);
  A.lda = lda;
  A.slab_k = K;
  A.M = M;
  return A;
}
// u / h as the drafter's own kernels store them for a weight-streaming GEMM
template <typename T>
AOperand<T> a_frag(const void* p, int K, int M) {
  AOperand<T> A = a_single<T>(p, K, K, M);
  A.frag = 1;
  return A;
}

// ------------------------------------------------------------- checks
bool bad_cfg(const dflash_config& c) {
  if (c.n_layers < 1 || c.n_layers > DFLASH_MAX_LAYERS) return true;
  if (c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.ffn <= 0 || c.vocab < 2) return true;
  if (c.n_feat_layers < 1 || c.n_feat_layers > DFLASH_MAX_FEAT) return true;
  if (c.mask_token_id < 0 || c.mask_token_id >= c.vocab) return true;
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 1.f)) return true;
  if (c.dtype != DFLASH_F32 && c.dtype != DFLASH_BF16) return true;
  return false;
}
bool unsupported_cfg(const dflash_config& c) {
  if (c.head_dim != 64 && c.head_dim != 128) return true;
  if (c.n_q_heads % c.n_kv_heads != 0) return true;
  if (c.hidden % 128 || c.ffn % 128 || (c.n_q_heads * c.head_dim) % 128) return true;
  if (c.hidden > 8192) return true;
  return false;
}

dflash_status check_kv(const dflash_handle* h, const dflash_kv* kv) {
  if (!kv || !kv->k || !kv->v || !kv->seq_off || !kv->seq_cap || !kv->seq_len)
    return DFLASH_ERR_INVALID_ARG;
  if (kv->batch < 1 || kv->batch > DFLASH_MAX_BATCH || kv->cap_total <= 0) return DFLASH_ERR_INVALID_ARG;
  // one kv head's slab (cap_total rows of head_dim values) must be addressable
  // by the 32-bit byte offsets of the attention kernel's buffer loads
  if (kv->cap_total * h->cfg.head_dim >= (int64_t{1} << 30)) return DFLASH_ERR_UNSUPPORTED;
  for (int l = 0; l < h->cfg.n_layers; ++l)
    if (!kv->k[l] || !kv->v[l] || !aligned16(kv->k[l]) || !aligned16(kv->v[l]))
      return DFLASH_ERR_INVALID_ARG;
  for (int b = 0; b < kv->batch; ++b) {
    const int64_t off = kv->seq_off[b];
    const int32_t cap = kv->seq_cap[b], len = kv->seq_len[b];
    if (off < 0 || cap < 0 || (off % 32) || (cap % 32) || off + cap > kv->cap_total)
      return DFLASH_ERR_INVALID_ARG;
    if (len < 0 || len > cap) return DFLASH_ERR_INVALID_ARG;
  }
  // sequence ranges must not overlap
  for (int a = 0; a < kv->batch; ++a)
    for (int b = a + 1; b < kv->batch; ++b) {
      const int64_t a0 = kv->seq_off[a], a1 = a0 + kv->seq_cap[a];
      const int64_t b0 = kv->seq_off[b], b1 = b0 + kv->seq_cap[b];
      if (a0 < b1 && b0 < a1 && kv->seq_cap[a] > 0 && kv->seq_cap[b] > 0)
        return DFLASH_ERR_INVALID_ARG;
    }
  return DFLASH_OK;
}

// ------------------------------------------------------------- the calls
template <typename T>
dflash_status fuse_impl(dflash_handle* h, const void* const* feats, int64_t n_tokens,
                        void* ctx_out, void* ws, hipStream_t st) {
  const Dims D = dims(h->cfg);
  const int T_ = static_cast<int>(n_tokens);
  const Layout L = layout(h, 1, 1, n_tokens);
  const GemmPlan g = gemm_plan(D);
  AOperand<T> A{};
  for (int i = 0; i < 6; ++i) A.slab[i] = static_cast<const T*>(feats[i < D.nf ? i : 0]);
  A.lda = D.H;
  A.slab_k = D.H;
  A.M = T_;
  const int K = D.nf * D.H;
  const int ks = fuse_ksplit(h, n_tokens);
  float* Y = at<float>(ws, L.part_off);
  DF_MARK(DFLASH_SEC_FUSE_GEMM, -1, false);
  if (sizeof(T) == 2 && T_ >= kTiledMinRows) {
    AOperand<uint16_t> At{};
    for (int i = 0; i < 6; ++i) At.slab[i] = reinterpret_cast<const uint16_t*>(A.slab[i]);
    At.lda = A.lda; At.slab_k = A.slab_k; At.M = A.M; At.m0 = 0; At.mc = A.M;
    TEpiStoreF32 te{static_cast<const uint16_t*>(h->packed ? h->pk_fc : h->w.fc), K, Y, D.H, T_};
    DF_HIP(launch_tiled(At, D.H, K, 1, ks, te, st, h->packed));
  } else {
    EpiPartialF32<T> epi{static_cast<const T*>(h->w.fc), K, Y, D.H, T_};
    DF_HIP(run_rows<T>(A, K, g.tiles_fc, 1, ks, epi, st, NoPerLaunch{}));
  }
  DF_MARK(DFLASH_SEC_FUSE_GEMM, -1, true);
  DF_MARK(DFLASH_SEC_FUSE_NORM, -1, false);
  DF_HIP(launch_resid_rmsnorm(h->cfg.dtype == DFLASH_BF16, nullptr, Y, ks,
                              static_cast<int64_t>(T_) * D.H, h->w.fc_norm, ctx_out, T_, D.H,
                              h->cfg.rms_eps, st));
  DF_MARK(DFLASH_SEC_FUSE_NORM, -1, true);
  return DFLASH_OK;
}

template <typename T>
dflash_status inject_impl(dflash_handle* h, const void* ctx, const SeqTable& seq, int total,
                          dflash_kv* kv, void* ws, hipStream_t st) {
  const Dims D = dims(h->cfg);
  const GemmPlan g = gemm_plan(D);
  DF_MARK(DFLASH_SEC_INJECT, -1, false);
  EpiInject<T> epi{};
  for (int l = 0; l < D.L; ++l) {
    epi.wk[l] = static_cast<const T*>(h->layers[l].wk);
    epi.wv[l] = static_cast<const T*>(h->layers[l].wv);
    epi.kc[l] = static_cast<T*>(kv->k[l]);
    epi.vc[l] = static_cast<T*>(kv->v[l]);
  }
  epi.K = D.H;
  epi.d = D.d;
  epi.Hkv = D.Hkv;
  epi.cap = kv->cap_total;
  epi.freq = rope_freq(h->cfg);
  epi.seq = seq;
  if (sizeof(T) == 2 && total >= kTiledMinRows) {
    TEpiInject te{};
    for (int l = 0; l < D.L; ++l) {
      te.wk[l] = static_cast<const uint16_t*>(h->packed ? h->pk_layers[l].wk : h->layers[l].wk);
      te.wv[l] = static_cast<const uint16_t*>(h->packed ? h->pk_layers[l].wv : h->layers[l].wv);
      te.kc[l] = reinterpret_cast<uint16_t*>(epi.kc[l]);
      te.vc[l] = reinterpret_cast<uint16_t*>(epi.vc[l]);
    }
    te.K = D.H;
    te.d = D.d;
    te.cap = kv->cap_total;
    te.freq = epi.freq;
    te.seq = seq;
    const AOperand<uint16_t> At = a_single<uint16_t>(ctx, D.H, D.H, total);
    // 256 x 256 tiles when they cover the 256 compute units at least twice.
    // Fewer: the parts (layer, K or V) that fill whole rounds on 256 x 256
    // tiles, the rest in a second launch when it fits in one round -- on
    // 128 x 128 tiles if those fit (2048 rows, 320 tiles = 8 parts in one
    // round + 2 parts as 256 quarter tiles: every compute unit busy; measured
    // 207-215 against 235-241 us with the 2 parts as 128 half tiles of
    // 256 x 128, which leave half the GPU idle), else on 256 x 128 tiles;
    // else everything on 256 x 128 tiles.
    const int parts = 2 * D.L;
    const int64_t per_part = static_cast<int64_t>((total + kPreBM - 1) / kPreBM) *
                             ((D.kvd + kPreBN - 1) / kPreBN);
    const int64_t big_tiles = per_part * parts;
    const int pa = static_cast<int>(big_tiles / kCUs * kCUs / per_part);
    const bool pk = h->packed;
    if (big_tiles >= 2 * kCUs) {
      DF_HIP(launch_tiled(At, D.kvd, D.H, parts, 1, te, st, pk));
    } else if (pa >= 1 && pa < parts && (parts - pa) * per_part * 2 <= kCUs) {
      DF_HIP(launch_tiled(At, D.kvd, D.H, pa, 1, te, st, pk));
      te.part_base = pa;
      const int64_t quarter = static_cast<int64_t>(parts - pa) * ((total + 127) / 128) *
                              ((D.kvd + 127) / 128);
      if (quarter <= kCUs)
        DF_HIP((launch_tiled_cfg<128, 128, 2, 4>(At, D.kvd, D.H, parts - pa, 1, te, st, pk)));
      else
        DF_HIP((launch_tiled_cfg<kPreBM, 128, 2, 4>(At, D.kvd, D.H, parts - pa, 1, te, st, pk)));
    } else {
      DF_HIP((launch_tiled_cfg<kPreBM, 128, 2, 4>(At, D.kvd, D.H, parts, 1, te, st, pk)));
    }
  } else {
    DF_HIP(run_rows<T>(a_single<T>(ctx, D.H, D.H, total), D.H, g.tiles_inj, 1, 1, epi, st,
                       NoPerLaunch{}));
  }
  DF_MARK(DFLASH_SEC_INJECT, -1, true);
  return DFLASH_OK;
}

// A training-layout request: entry b of the batch is a block at anchor
// position len[b] of the sequence whose cache slab starts at off[b]; the LM
// head then scores slots 1..B-1 against labels (device [n][B-1]).
struct TrainSpec {
  int n;
  const int32_t* len;      // host [n]
  const int64_t* off;      // host [n]
  const int32_t* labels;   // device [n][B-1]
  float gamma;
  float* slot_loss;        // device [n][B-1]
  float* loss;             // device [1]
};

// Committed lengths in device memory (device-resident step), at most max.
struct DevLen {
  const int32_t* len;
  int max;
};

template <typename T>
dflash_status draft_impl(dflash_handle* h, dflash_kv* kv, int B, const int32_t* anchors,
                         int32_t* draft, float* dbg_h, float* dbg_z, void* ws, hipStream_t st,
                         const TrainSpec* tr = nullptr, const DevLen* dl = nullptr) {
  const Dims D = dims(h->cfg);
  const int nb = tr ? tr->n : kv->batch, M = nb * B;
  const bool bf = h->cfg.dtype == DFLASH_BF16;
  const Layout L = layout(h, nb, B, 1);
  const GemmPlan g = gemm_plan(D);
  const float eps = h->cfg.rms_eps;

  SeqTable seq{};
  seq.n = nb;
  int max_keys = 0;   // keys in the cache per entry (training: the context part only)
  // (device lengths: the launch plan covers every length up to dl->max)
  for (int b = 0; b < nb; ++b) {
    seq.len[b] = tr ? tr->len[b] : (dl ? dl->max : kv->seq_len[b]);
    seq.off[b] = tr ? tr->off[b] : kv->seq_off[b];
    const int nk = seq.len[b] + (tr ? 0 : B);
    max_keys = nk > max_keys ? nk : max_keys;
  }
  if (dl) {
    seq.dlen = dl->len;
    seq.len_max = dl->max;
  }
  // training layout: the blocks' own K/V in the workspace, kTrainSlab rows each
  const int64_t capb = static_cast<int64_t>(nb) * kTrainSlab;
  T* bk = tr ? at<T>(ws, L.bkv_off) : nullptr;
  T* bv = tr ? bk + static_cast<int64_t>(D.Hkv) * capb * D.d : nullptr;
  const RopeFreq freq = rope_freq(h->cfg);
  float* x = at<float>(ws, L.x_off);
  T* u = at<T>(ws, L.u_off);
  T* qb = at<T>(ws, L.q_off);
  T* ob = at<T>(ws, L.o_off);
  T* hb = at<T>(ws, L.h_off);
  float* part = at<float>(ws, L.part_off);
  const int64_t pstride = static_cast<int64_t>(M) * D.H;   // one K-split slab
  // batches of blocks: the layer GEMMs and the LM head on the LDS-tiled GEMM
  const bool mid = bf && M >= kMidMinRows;
  // u, h and the attention output are stored fragment-major for either GEMM
  // (one contiguous 1 KB block per 16 rows x 32 columns an operand load reads)
  const bool frag = true;
  // the LDS-tiled GEMMs read the packed weights when the caller made them
  const bool pk = h->packed;
  const MidPlan mp = mid_plan(D, M);
  const int ks_o = mid ? mp.ks_o : g.ks_o, ks_d = mid ? mp.ks_d : g.ks_d;
  float* qkvp = at<float>(ws, L.qkvp_off);
  auto a16 = [&](const void* p, int K) { return a_frag<uint16_t>(p, K, M); };
  auto w16 = [&](const void* raw, const void* packed) {
    return static_cast<const uint16_t*>(pk ? packed : raw);
  };

  // block embedding fused with layer 0's attention RMSNorm
  DF_MARK(DFLASH_SEC_EMBED, -1, false);
  DF_HIP(launch_embed(bf, h->w.embed, D.H, D.V, anchors, h->cfg.mask_token_id, nb, B, x,
                      h->layers[0].attn_norm, u, eps, st, frag));
  DF_MARK(DFLASH_SEC_EMBED, -1, true);

  // attention split (see attn_chunk)
  int32_t keys[DFLASH_MAX_BATCH];
  for (int b = 0; b < nb; ++b) keys[b] = seq.len[b] + B;
  const int max_c = static_cast<int>(
      std::max<int64_t>(1, std::min<int64_t>(kMaxAttnChunks, attn_slots(nb, D.Hkv) / (nb * D.Hkv))));
  // (training: one chunk of every entry holds its block's keys)
  int chunk = attn_chunk(keys, nb, D.Hkv, max_keys, tr ? max_c - 1 : max_c);
  AttnArgs aa{};
  // ragged batches with host-held lengths: longest-first order (training
  // layout: entries' context keys, plus one chunk of their B block keys)
  if (tr) {
    int32_t ctx_keys[DFLASH_MAX_BATCH];
    for (int b = 0; b < nb; ++b) ctx_keys[b] = seq.len[b];
    attn_plan_order(ctx_keys, nb, D.Hkv, std::max(max_keys, 1), max_c - 1, B, &chunk, &aa);
  } else if (!dl) {
    attn_plan_order(keys, nb, D.Hkv, max_keys, max_c, 0, &chunk, &aa);
  }
  aa.q = qb;
  aa.ldq = D.qd;
  aa.cap = kv->cap_total;
  aa.o = ob;
  aa.ofrag = frag ? 1 : 0;
  aa.part_o = at<float>(ws, L.ao_off);
  aa.part_ml = at<float2>(ws, L.aml_off);
  aa.B = B;
  aa.G = D.G;
  aa.n_kv = D.Hkv;
  aa.head_dim = D.d;
  aa.chunk = chunk;
  aa.max_chunks = (max_keys + chunk - 1) / chunk + (tr ? 1 : 0);
  aa.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(D.d)));
  aa.seq = seq;
  aa.kb = bk;
  aa.vb = bv;
  aa.capb = capb;
  // where the QKV finish puts the block's K/V: the cache, or the block buffer
  auto kdst = [&](int l) -> void* { return tr ? static_cast<void*>(bk) : kv->k[l]; };
  auto vdst = [&](int l) -> void* { return tr ? static_cast<void*>(bv) : kv->v[l]; };
  const int64_t dcap = tr ? capb : kv->cap_total;

  int pending = 0;   // K-split slabs of the last projection, not yet added to x
  for (int l = 0; l < D.L; ++l) {
    const dflash_layer_weights& w = h->layers[l];
    const dflash_layer_weights& wp = h->pk_layers[l];
    // attention half: x += (down partials of the previous layer); u = RMSNorm(x)
    if (l > 0) {
      DF_MARK(DFLASH_SEC_ATTN_NORM, l, false);
      DF_HIP(launch_resid_rmsnorm(bf, x, part, pending, pstride, w.attn_norm, u, M, D.H, eps, st,
                                  frag));
      DF_MARK(DFLASH_SEC_ATTN_NORM, l, true);
    }
    DF_MARK(DFLASH_SEC_QKV, l, false);
    if (mid) {
      const int nq = D.qd + 2 * D.kvd;
      TEpiQKVParts e{w16(w.wq, wp.wq), w16(w.wk, wp.wk), w16(w.wv, wp.wv), D.H, D.qd, D.kvd,
                     qkvp, nq, M};
      DF_HIP(launch_mid<128>(a16(u, D.H), nq, D.H, mp.ks_qkv, e, st, pk));
      DF_HIP(launch_qkv_finish(true, qkvp, mp.ks_qkv, static_cast<int64_t>(M) * nq, M, D.qd,
                               D.kvd, D.d, B, qb, D.qd, kdst(l), vdst(l), dcap, freq, seq, st,
                               tr != nullptr));
    } else if (tr) {
      // training layout: split K over workgroups, then sum the slabs, rotate
      // and send the block K/V to the block buffer in the finishing kernel
      const int nq = D.qd + 2 * D.kvd;
      EpiQKVPartF32<T> e{static_cast<const T*>(w.wq), static_cast<const T*>(w.wk),
                         static_cast<const T*>(w.wv), D.H, D.qd, D.kvd, qkvp, nq, M};
      DF_HIP(run_rows<T>(a_frag<T>(u, D.H, M), D.H, g.tiles_qkv, 1, g.ks_qkv, e, st,
                         NoPerLaunch{}));
      DF_HIP(launch_qkv_finish(bf, qkvp, g.ks_qkv, static_cast<int64_t>(M) * nq, M, D.qd,
                               D.kvd, D.d, B, qb, D.qd, kdst(l), vdst(l), dcap, freq, seq, st,
                               tr != nullptr));
    } else {
      EpiQKV<T> e{};
      e.wq = static_cast<const T*>(w.wq);
      e.wk = static_cast<const T*>(w.wk);
      e.wv = static_cast<const T*>(w.wv);
      e.K = D.H; e.d = D.d; e.Hq = D.Hq; e.Hkv = D.Hkv; e.B = B;
      e.q = qb; e.ldq = D.qd;
      e.kc = static_cast<T*>(kv->k[l]);
      e.vc = static_cast<T*>(kv->v[l]);
      e.cap = kv->cap_total;
      e.freq = freq;
      e.seq = seq;
      // no K split (the epilogue rotates whole sums and writes q and the
      // cache rows itself): 4 waves per pair tile.  On the 8B shape (192
      // tiles, 3/4 of the CUs) this measured 16.0 us, against 16.9 us with 8
      // waves and 19.5 us for four K-split slabs plus the finishing kernel.
      DF_HIP(run_rows<T>(a_frag<T>(u, D.H, M), D.H, g.tiles_qkv, 1, 1, e, st,
                         NoPerLaunch{}, 4));
    }
    DF_MARK(DFLASH_SEC_QKV, l, true);
    aa.kc = kv->k[l];
    aa.vc = kv->v[l];
    DF_MARK(DFLASH_SEC_ATTENTION, l, false);
    DF_HIP(launch_block_attention(bf, D.d, aa, nb, st));
    DF_MARK(DFLASH_SEC_ATTENTION, l, true);
    DF_MARK(DFLASH_SEC_O_PROJ, l, false);
    if (mid) {
      TEpiStoreF32 e{w16(w.wo, wp.wo), D.qd, part, D.H, M};
      DF_HIP(launch_mid_o(a16(ob, D.qd), D.H, D.qd, ks_o, e, st, pk));
    } else {
      EpiPartialF32<T> e{static_cast<const T*>(w.wo), D.qd, part, D.H, M};
      // two pair tiles per step share each A fragment (measured faster here,
      // slower on the QKV, down and LM-head shapes); 8 waves split each K
      // slab (8B shape: 9.5 us against 10.2 us with 4 waves; 8 waves on the
      // QKV, gate/up and down shapes measured no gain)
      DF_HIP(run_rows<T>(a_frag<T>(ob, D.qd, M), D.qd, g.tiles_o, 1, g.ks_o, e, st,
                         NoPerLaunch{}, 8, 2));
    }
    DF_MARK(DFLASH_SEC_O_PROJ, l, true);
    // feed-forward half: x += O partials; u = RMSNorm(x)
    DF_MARK(DFLASH_SEC_FFN_NORM, l, false);
    DF_HIP(launch_resid_rmsnorm(bf, x, part, ks_o, pstride, w.ffn_norm, u, M, D.H, eps, st, frag));
    DF_MARK(DFLASH_SEC_FFN_NORM, l, true);
    DF_MARK(DFLASH_SEC_GATE_UP, l, false);
    if (mid) {
      TEpiSwiGLUPair e{w16(w.wg, wp.wg), w16(w.wu, wp.wu), D.H, D.F, 128,
                       reinterpret_cast<uint16_t*>(hb), D.F, 1};
      DF_HIP(launch_mid<128>(a16(u, D.H), 2 * D.F, D.H, 1, e, st, pk));
    } else {
      EpiSwiGLU<T> e{static_cast<const T*>(w.wg), static_cast<const T*>(w.wu), D.H, hb, D.F, 1};
      DF_HIP(run_rows<T>(a_frag<T>(u, D.H, M), D.H, g.tiles_gu, 1, 1, e, st, NoPerLaunch{}));
    }
    DF_MARK(DFLASH_SEC_GATE_UP, l, true);
    DF_MARK(DFLASH_SEC_DOWN, l, false);
    if (mid) {
      TEpiStoreF32 e{w16(w.wd, wp.wd), D.F, part, D.H, M};
      DF_HIP(launch_mid<128>(a16(hb, D.F), D.H, D.F, ks_d, e, st, pk));
    } else {
      EpiPartialF32<T> e{static_cast<const T*>(w.wd), D.F, part, D.H, M};
      DF_HIP(run_rows<T>(a_frag<T>(hb, D.F, M), D.F, g.tiles_d, 1, g.ks_d, e, st,
                         NoPerLaunch{}));
    }
    DF_MARK(DFLASH_SEC_DOWN, l, true);
    pending = ks_d;
  }
  // x += down partials of the last layer; u = RMSNorm(x)
  DF_MARK(DFLASH_SEC_FINAL_NORM, -1, false);
  DF_HIP(launch_resid_rmsnorm(bf, x, part, pending, pstride, h->w.final_norm, u, M, D.H, eps, st,
                              frag));
  DF_MARK(DFLASH_SEC_FINAL_NORM, -1, true);
  if (dbg_h)
    DF_HIP(hipMemcpyAsync(dbg_h, x, static_cast<size_t>(M) * D.H * 4, hipMemcpyDeviceToDevice, st));
  DF_MARK(DFLASH_SEC_LM_HEAD, -1, false);
  if (tr) {
    // training layout: cross-entropy partials (tiled GEMM for many block
    // rows, else the weight-streaming one), then the per-slot losses and
    // their weighted mean
    float4* lpart = at<float4>(ws, L.lm_off);
    const T* W = static_cast<const T*>(h->w.lm_head);
    EpiLMLoss<T, 1> l1{W, D.H, D.V, g.wg_lm, lpart, tr->labels, B, dbg_z};
    EpiLMLoss<T, 2> l2{W, D.H, D.V, g.wg_lm, lpart, tr->labels, B, dbg_z};
    EpiLMLoss<T, 4> l4{W, D.H, D.V, g.wg_lm, lpart, tr->labels, B, dbg_z};
    EpiLMLoss<T, 8> l8{W, D.H, D.V, g.wg_lm, lpart, tr->labels, B, dbg_z};
    const AOperand<T> A = a_frag<T>(u, D.H, M);
    int n_parts = g.wg_lm;
    DF_MARK(DFLASH_SEC_LM_GEMM, -1, false);
    if (mid) {
      // many block rows: the LDS-tiled GEMM, 256 vocabulary rows per tile
      n_parts = lm_split(M, D.V).n_parts;
      const int np = n_parts;
      auto make = [&](int n_base, int part_base) {
        return TEpiLoss{w16(h->w.lm_head, h->pk_lm), D.H, D.V, np, B, lpart, tr->labels, dbg_z,
                        n_base, part_base};
      };
      DF_HIP(launch_lm_tiled(a16(u, D.H), D.V, D.H, make, st, pk));
    }
    for (int m0 = 0; !mid && m0 < M; m0 += kMaxRowsPerLaunch) {
      AOperand<T> Ai = A;
      Ai.m0 = m0;
      Ai.mc = M - m0 < kMaxRowsPerLaunch ? M - m0 : kMaxRowsPerLaunch;
      const int mt = (Ai.mc + 15) / 16;
      hipError_t e;
      if (mt <= 1) e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, l1, st);
      else if (mt <= 2) e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, l2, st);
      else if (mt <= 4) e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, l4, st);
      else e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, l8, st);
      DF_HIP(e);
    }
    DF_MARK(DFLASH_SEC_LM_GEMM, -1, true);
    DF_HIP(launch_lm_loss(lpart, n_parts, M, B, tr->gamma, tr->slot_loss, tr->loss, st));
    DF_MARK(DFLASH_SEC_LM_HEAD, -1, true);
    return DFLASH_OK;
  }
  {
    float2* lm_part = at<float2>(ws, L.lm_off);
    const int n_wg = g.wg_lm;
    EpiLMHead<T, 1> e1{static_cast<const T*>(h->w.lm_head), D.H, D.V, n_wg, lm_part, dbg_z};
    EpiLMHead<T, 2> e2{static_cast<const T*>(h->w.lm_head), D.H, D.V, g.wg_lm, lm_part, dbg_z};
    EpiLMHead<T, 4> e4{static_cast<const T*>(h->w.lm_head), D.H, D.V, g.wg_lm, lm_part, dbg_z};
    EpiLMHead<T, 8> e8{static_cast<const T*>(h->w.lm_head), D.H, D.V, g.wg_lm, lm_part, dbg_z};
    const AOperand<T> A = a_frag<T>(u, D.H, M);
    if (mid) {
      const int n_parts = lm_split(M, D.V).n_parts;
      auto make = [&](int n_base, int part_base) {
        return TEpiArgmax{w16(h->w.lm_head, h->pk_lm), D.H, D.V, n_parts, lm_part, dbg_z, n_base,
                          part_base};
      };
      DF_MARK(DFLASH_SEC_LM_GEMM, -1, false);
      DF_HIP(launch_lm_tiled(a16(u, D.H), D.V, D.H, make, st, pk));
      DF_MARK(DFLASH_SEC_LM_GEMM, -1, true);
      DF_HIP(launch_lm_argmax_finalize(lm_part, n_parts, M, B, anchors, D.V, draft, st));
    }
    // one launch covers M: the LM-GEMM timing point (if set) is recorded by
    // that dispatch; otherwise around the launches
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    const bool one = M <= kMaxRowsPerLaunch && timing_events(h, DFLASH_SEC_LM_GEMM, -1, &ev0, &ev1);
    if (!mid && !one) DF_MARK(DFLASH_SEC_LM_GEMM, -1, false);
    for (int m0 = 0; !mid && m0 < M; m0 += kMaxRowsPerLaunch) {
      AOperand<T> Ai = A;
      Ai.m0 = m0;
      Ai.mc = M - m0 < kMaxRowsPerLaunch ? M - m0 : kMaxRowsPerLaunch;
      const int mt = (Ai.mc + 15) / 16;
      hipError_t e;
      const hipEvent_t a = one ? ev0 : nullptr, b = one ? ev1 : nullptr;
      if (mt <= 1) e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, e1, st, 1, a, b);
      else if (mt <= 2) e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, e2, st, 1, a, b);
      else if (mt <= 4) e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, e4, st, 1, a, b);
      else e = launch_skinny_nw<T, 4>(Ai, D.H, g.tiles_lm, kLmTilesPerWg, 1, e8, st, 1, a, b);
      DF_HIP(e);
    }
    if (!mid) {
      if (!one) DF_MARK(DFLASH_SEC_LM_GEMM, -1, true);
      DF_HIP(launch_lm_argmax_finalize(lm_part, n_wg, M, B, anchors, D.V, draft, st));
    }
  }
  DF_MARK(DFLASH_SEC_LM_HEAD, -1, true);
  return DFLASH_OK;
}

// The device-resident step's fused context rows sit past everything the
// fusion of those rows uses in the workspace.
size_t step_ctx_off(const dflash_handle* h, int64_t rows) {
  return align_up(layout(h, 1, 1, rows).total);
}

// verify -> append the accepted rows -> advance the lengths -> next draft,
// every count and length read on the device (see dflash_step_resident).
template <typename T>
dflash_status step_impl(dflash_handle* h, dflash_kv* kv, int B, int32_t* dev_len, int len_max,
                        const void* logits, bool logits_bf16, const void* const* feats,
                        int32_t* draft, int32_t* anchor, int32_t* accept, int32_t* status,
                        void* ws, hipStream_t st) {
  const Dims D = dims(h->cfg);
  const int nb = kv->batch, M = nb * B;
  const Layout L = layout(h, nb, B, 1);
  DF_HIP(launch_verify(logits, logits_bf16, draft, nb, B, D.V, accept, anchor,
                       at<void>(ws, L.ver_off), st));
  void* ctx = at<void>(ws, step_ctx_off(h, M));
  dflash_status s = fuse_impl<T>(h, feats, M, ctx, ws, st);
  if (s != DFLASH_OK) return s;
  SeqTable seq{};
  seq.n = nb;
  for (int b = 0; b < nb; ++b) {
    seq.len[b] = len_max;
    seq.off[b] = kv->seq_off[b];
  }
  seq.dlen = dev_len;
  seq.dcnt = accept;
  seq.len_max = len_max;
  seq.stride = B;
  s = inject_impl<T>(h, ctx, seq, M, kv, ws, st);
  if (s != DFLASH_OK) return s;
  DF_HIP(launch_advance_lengths(dev_len, accept, nb, B, len_max, status, st));
  const DevLen dl{dev_len, len_max};
  return draft_impl<T>(h, kv, B, anchor, draft, nullptr, nullptr, ws, st, nullptr, &dl);
}

// ------------------------------------------------------------- packed weights
// Every bf16 GEMM weight, fragment-major with its rows padded to a multiple
// of 16, at 256-byte aligned offsets: per layer wq, wk, wv, wo, wg, wu, wd,
// then fc, then lm_head.
constexpr int kPackPerLayer = 7;
struct PackMat {
  const void* src;
  int N, K;
  size_t off;
};
struct PackPlan {
  PackMat m[kPackPerLayer * DFLASH_MAX_LAYERS + 2];
  int n;
  size_t total;
};
PackPlan pack_plan(const dflash_handle* h) {
  const Dims D = dims(h->cfg);
  PackPlan p{};
  size_t off = 0;
  auto add = [&](const void* src, int N, int K) {
    p.m[p.n++] = PackMat{src, N, K, off};
    off += align_up(static_cast<size_t>((N + 15) / 16) * 16 * K * 2);
  };
  for (int l = 0; l < D.L; ++l) {
    const dflash_layer_weights& w = h->layers[l];
    add(w.wq, D.qd, D.H);
    add(w.wk, D.kvd, D.H);
    add(w.wv, D.kvd, D.H);
    add(w.wo, D.H, D.qd);
    add(w.wg, D.F, D.H);
    add(w.wu, D.F, D.H);
    add(w.wd, D.H, D.F);
  }
  add(h->w.fc, D.H, D.nf * D.H);
  add(h->w.lm_head, D.V, D.H);
  p.total = off;
  return p;
}

}  // namespace

// ------------------------------------------------------------- static scratch
// The workspace of dflash_draft_block_noalloc, for callers that cannot
// allocate: one array per device (each device that runs the call holds its
// own copy until the process ends).  In host code the array's name is only a
// stand-in for the device symbol; every use goes through the device address
// hipGetSymbolAddress returns, looked up once per device with that device
// current.  Nothing in a draft's workspace needs clearing (every slot read is
// written earlier in the same call), so the array keeps whatever the last
// call left; calls that overlap on one device race on it.
static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

dflash_status scratch_address(void** out) {
  int dev = -1;
  DF_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    DF_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return DFLASH_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DFLASH_OK;
}
}  // namespace

// ================================================================ C ABI

extern "C" {

int32_t dflash_target_layer_ids(int32_t n_target_layers, int32_t n_select, int32_t* out) {
  if (!out || n_select < 2 || n_select > DFLASH_MAX_FEAT || n_target_layers < n_select + 3)
    return -1;
  // grid point k sits at 2 + k (L - 4) / (n - 1); round half up in integers
  const int64_t den = n_select - 1;
  for (int32_t k = 0; k < n_select; ++k) {
    const int64_t num = 2 * den + static_cast<int64_t>(k) * (n_target_layers - 4);
    out[k] = static_cast<int32_t>((2 * num + den) / (2 * den));
  }
  return n_select;
}

const char* dflash_status_string(dflash_status s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_INVALID_ARG: return "invalid argument";
    case DFLASH_ERR_CAPACITY: return "cache capacity exceeded";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported shape";
    case DFLASH_ERR_HIP: return "HIP runtime error";
    case DFLASH_ERR_SCRATCH: return "needs more scratch than the static buffer holds";
  }
  return "unknown status";
}

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w, dflash_handle** out) {
  if (!cfg || !w || !out) return DFLASH_ERR_INVALID_ARG;
  *out = nullptr;
  if (bad_cfg(*cfg)) return DFLASH_ERR_INVALID_ARG;
  if (unsupported_cfg(*cfg)) return DFLASH_ERR_UNSUPPORTED;
  if ((cfg->n_q_heads / cfg->n_kv_heads) * 2 > 80) return DFLASH_ERR_UNSUPPORTED;
  const void* top[6] = {w->fc, w->fc_norm, w->final_norm, w->embed, w->lm_head, w->layers};
  for (const void* p : top)
    if (!p) return DFLASH_ERR_INVALID_ARG;
  for (int i = 0; i < 5; ++i)
    if (!aligned16(top[i])) return DFLASH_ERR_INVALID_ARG;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    const void* ps[9] = {lw.attn_norm, lw.wq, lw.wk, lw.wv, lw.wo, lw.ffn_norm, lw.wg, lw.wu, lw.wd};
    for (const void* p : ps)
      if (!p || !aligned16(p)) return DFLASH_ERR_INVALID_ARG;
  }
  dflash_handle* h = new (std::nothrow) dflash_handle;
  if (!h) return DFLASH_ERR_INVALID_ARG;
  h->cfg = *cfg;
  h->w = *w;
  for (int l = 0; l < cfg->n_layers; ++l) h->layers[l] = w->layers[l];
  h->w.layers = h->layers;
  h->n_timing = 0;
  h->packed = false;
  for (int l = 0; l < DFLASH_MAX_LAYERS; ++l) h->pk_layers[l] = dflash_layer_weights{};
  h->pk_fc = h->pk_lm = nullptr;
  *out = h;
  return DFLASH_OK;
}

dflash_status dflash_packed_weights_size(const dflash_handle* h, size_t* bytes) {
  if (!h || !bytes) return DFLASH_ERR_INVALID_ARG;
  if (h->cfg.dtype != DFLASH_BF16) return DFLASH_ERR_UNSUPPORTED;
  *bytes = pack_plan(h).total;
  return DFLASH_OK;
}

dflash_status dflash_pack_weights(dflash_handle* h, void* dst, size_t bytes, void* stream) {
  if (!h) return DFLASH_ERR_INVALID_ARG;
  if (!dst) {
    if (bytes) return DFLASH_ERR_INVALID_ARG;
    h->packed = false;   // back to the caller's row-major weights
    return DFLASH_OK;
  }
  if (h->cfg.dtype != DFLASH_BF16) return DFLASH_ERR_UNSUPPORTED;
  if (!aligned16(dst)) return DFLASH_ERR_INVALID_ARG;
  const PackPlan p = pack_plan(h);
  if (bytes < p.total) return DFLASH_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // unbound until every copy is launched: a failed call leaves the handle on
  // the row-major weights
  h->packed = false;
  char* base = static_cast<char*>(dst);
  for (int i = 0; i < p.n; ++i)
    DF_HIP(launch_pack_frag(static_cast<const uint16_t*>(p.m[i].src), p.m[i].N, p.m[i].K,
                            reinterpret_cast<uint16_t*>(base + p.m[i].off), st));
  for (int l = 0; l < h->cfg.n_layers; ++l) {
    const PackMat* m = p.m + kPackPerLayer * l;
    dflash_layer_weights& w = h->pk_layers[l];
    w.wq = base + m[0].off;
    w.wk = base + m[1].off;
    w.wv = base + m[2].off;
    w.wo = base + m[3].off;
    w.wg = base + m[4].off;
    w.wu = base + m[5].off;
    w.wd = base + m[6].off;
  }
  h->pk_fc = base + p.m[p.n - 2].off;
  h->pk_lm = base + p.m[p.n - 1].off;
  h->packed = true;
  return DFLASH_OK;
}

dflash_status dflash_destroy(dflash_handle* h) {
  if (!h) return DFLASH_ERR_INVALID_ARG;
  delete h;
  return DFLASH_OK;
}

dflash_status dflash_workspace_size(const dflash_handle* h, int32_t max_batch, int32_t max_block,
                                    int64_t max_tokens, size_t* bytes) {
  if (!h || !bytes || max_batch < 1 || max_batch > DFLASH_MAX_BATCH || max_block < 2 ||
      max_block > DFLASH_MAX_BLOCK || max_tokens < 0)
    return DFLASH_ERR_INVALID_ARG;
  const size_t es = h->cfg.dtype == DFLASH_BF16 ? 2 : 4;
  const int64_t rows = static_cast<int64_t>(max_batch) * max_block;
  // the device-resident step: its fusion's scratch, then its context rows
  const size_t step = step_ctx_off(h, rows) + align_up(static_cast<size_t>(rows) * h->cfg.hidden * es);
  *bytes = std::max(layout(h, max_batch, max_block, max_tokens).total, step);
  return DFLASH_OK;
}

dflash_status dflash_fuse_context(dflash_handle* h, const void* const* feats, int64_t n_tokens,
                                  void* ctx_out, void* ws, void* stream) {
  if (!h || !feats || !ctx_out || !ws || n_tokens < 0 || n_tokens > (1 << 24))
    return DFLASH_ERR_INVALID_ARG;
  if (!aligned16(ctx_out) || !aligned16(ws)) return DFLASH_ERR_INVALID_ARG;
  for (int i = 0; i < h->cfg.n_feat_layers; ++i)
    if (!feats[i] || !aligned16(feats[i])) return DFLASH_ERR_INVALID_ARG;
  if (n_tokens == 0) return DFLASH_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return h->cfg.dtype == DFLASH_BF16 ? fuse_impl<uint16_t>(h, feats, n_tokens, ctx_out, ws, st)
                                     : fuse_impl<float>(h, feats, n_tokens, ctx_out, ws, st);
}

dflash_status dflash_inject_kv(dflash_handle* h, const void* ctx, const int32_t* pos_start,
                               const int32_t* n_new, dflash_kv* kv, void* ws, void* stream) {
  if (!h || !n_new || !ws) return DFLASH_ERR_INVALID_ARG;
  dflash_status s = check_kv(h, kv);
  if (s != DFLASH_OK) return s;
  SeqTable seq{};
  seq.n = kv->batch;
  int64_t total = 0;
  for (int b = 0; b < kv->batch; ++b) {
    const int32_t p0 = pos_start ? pos_start[b] : kv->seq_len[b];
    if (n_new[b] < 0 || p0 < 0 || p0 > kv->seq_len[b]) return DFLASH_ERR_INVALID_ARG;
    if (static_cast<int64_t>(p0) + n_new[b] > kv->seq_cap[b]) return DFLASH_ERR_CAPACITY;
    seq.row0[b] = static_cast<int32_t>(total);
    seq.pos0[b] = p0;
    seq.off[b] = kv->seq_off[b];
    seq.len[b] = kv->seq_len[b];
    total += n_new[b];
  }
  if (total > (1 << 24)) return DFLASH_ERR_INVALID_ARG;
  if (total > 0 && (!ctx || !aligned16(ctx))) return DFLASH_ERR_INVALID_ARG;
  if (!aligned16(ws)) return DFLASH_ERR_INVALID_ARG;
  if (total > 0) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    s = h->cfg.dtype == DFLASH_BF16
            ? inject_impl<uint16_t>(h, ctx, seq, static_cast<int>(total), kv, ws, st)
            : inject_impl<float>(h, ctx, seq, static_cast<int>(total), kv, ws, st);
    if (s != DFLASH_OK) return s;
  }
  for (int b = 0; b < kv->batch; ++b)
    kv->seq_len[b] = (pos_start ? pos_start[b] : kv->seq_len[b]) + n_new[b];
  return DFLASH_OK;
}

dflash_status dflash_draft_block(dflash_handle* h, dflash_kv* kv, int32_t block_size,
                                 const int32_t* anchor_ids, int32_t* draft_ids,
                                 float* dbg_final_hidden, float* dbg_logits, void* ws,
                                 void* stream) {
  if (!h || !anchor_ids || !draft_ids || !ws) return DFLASH_ERR_INVALID_ARG;
  if (block_size < 2 || block_size > DFLASH_MAX_BLOCK) return DFLASH_ERR_INVALID_ARG;
  dflash_status s = check_kv(h, kv);
  if (s != DFLASH_OK) return s;
  const Dims D = dims(h->cfg);
  if (D.G * block_size > 80) return DFLASH_ERR_UNSUPPORTED;
  if (!aligned16(ws)) return DFLASH_ERR_INVALID_ARG;
  int max_keys = 0;
  for (int b = 0; b < kv->batch; ++b) {
    if (static_cast<int64_t>(kv->seq_len[b]) + block_size > kv->seq_cap[b]) return DFLASH_ERR_CAPACITY;
    max_keys = kv->seq_len[b] + block_size > max_keys ? kv->seq_len[b] + block_size : max_keys;
  }
  if ((max_keys + 255) / 256 > kMaxAttnChunks * 64) return DFLASH_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return h->cfg.dtype == DFLASH_BF16
             ? draft_impl<uint16_t>(h, kv, block_size, anchor_ids, draft_ids, dbg_final_hidden,
                                    dbg_logits, ws, st)
             : draft_impl<float>(h, kv, block_size, anchor_ids, draft_ids, dbg_final_hidden,
                                 dbg_logits, ws, st);
}

dflash_status dflash_draft_block_noalloc(dflash_handle* h, dflash_kv* kv, int32_t block_size,
                                         const int32_t* anchor_ids, int32_t* draft_ids,
                                         float* dbg_final_hidden, float* dbg_logits,
                                         void* stream) {
  if (!h || !anchor_ids || !draft_ids) return DFLASH_ERR_INVALID_ARG;
  if (block_size < 2 || block_size > DFLASH_MAX_BLOCK) return DFLASH_ERR_INVALID_ARG;
  dflash_status s = check_kv(h, kv);
  if (s != DFLASH_OK) return s;
  if (layout(h, kv->batch, block_size, 1).total > DFLASH_NOALLOC_SCRATCH_BYTES)
    return DFLASH_ERR_SCRATCH;
  void* ws = nullptr;
  s = scratch_address(&ws);
  if (s != DFLASH_OK) return s;
  return dflash_draft_block(h, kv, block_size, anchor_ids, draft_ids, dbg_final_hidden,
                            dbg_logits, ws, stream);
}

dflash_status dflash_train_forward(dflash_handle* h, const dflash_kv* kv, int32_t n_blocks,
                                   int32_t block_size, const int32_t* block_seq,
                                   const int32_t* anchor_pos, const int32_t* anchor_ids,
                                   const int32_t* labels, float gamma, float* slot_loss,
                                   float* loss, float* dbg_logits, void* ws, void* stream) {
  if (!h || !block_seq || !anchor_pos || !anchor_ids || !labels || !slot_loss || !loss || !ws)
    return DFLASH_ERR_INVALID_ARG;
  if (block_size < 2 || block_size > DFLASH_MAX_BLOCK) return DFLASH_ERR_INVALID_ARG;
  if (n_blocks < 1 || n_blocks > DFLASH_MAX_BATCH) return DFLASH_ERR_INVALID_ARG;
  if (!(gamma > 0.f) || !(gamma < INFINITY)) return DFLASH_ERR_INVALID_ARG;
  dflash_status s = check_kv(h, kv);
  if (s != DFLASH_OK) return s;
  const Dims D = dims(h->cfg);
  if (D.G * block_size > 80) return DFLASH_ERR_UNSUPPORTED;
  if (!aligned16(ws)) return DFLASH_ERR_INVALID_ARG;
  // one chunk per (block, kv head) must stay free for the block's own keys
  if (std::min<int64_t>(kMaxAttnChunks, attn_slots(n_blocks, D.Hkv) / (n_blocks * D.Hkv)) < 2)
    return DFLASH_ERR_UNSUPPORTED;
  int32_t len[DFLASH_MAX_BATCH];
  int64_t off[DFLASH_MAX_BATCH];
  int max_len = 0;
  for (int i = 0; i < n_blocks; ++i) {
    const int sq = block_seq[i];
    if (sq < 0 || sq >= kv->batch) return DFLASH_ERR_INVALID_ARG;
    if (anchor_pos[i] < 0 || anchor_pos[i] > kv->seq_len[sq]) return DFLASH_ERR_INVALID_ARG;
    len[i] = anchor_pos[i];
    off[i] = kv->seq_off[sq];
    max_len = len[i] > max_len ? len[i] : max_len;
  }
  if ((max_len + 255) / 256 > kMaxAttnChunks * 64) return DFLASH_ERR_UNSUPPORTED;
  const TrainSpec tr{n_blocks, len, off, labels, gamma, slot_loss, loss};
  hipStream_t st = static_cast<hipStream_t>(stream);
  dflash_kv* kvm = const_cast<dflash_kv*>(kv);   // read only: the caches and the slab table
  return h->cfg.dtype == DFLASH_BF16
             ? draft_impl<uint16_t>(h, kvm, block_size, anchor_ids, nullptr, nullptr, dbg_logits,
                                    ws, st, &tr)
             : draft_impl<float>(h, kvm, block_size, anchor_ids, nullptr, nullptr, dbg_logits, ws,
                                 st, &tr);
}

dflash_status dflash_step_resident(dflash_handle* h, dflash_kv* kv, int32_t block_size,
                                   int32_t* dev_len, int32_t len_max, const void* target_logits,
                                   dflash_dtype logits_dtype, const void* const* block_feats,
                                   int32_t* draft_ids, int32_t* anchor_ids, int32_t* accept,
                                   int32_t* status, void* ws, void* stream) {
  if (!h || !dev_len || !target_logits || !block_feats || !draft_ids || !anchor_ids || !accept ||
      !status || !ws)
    return DFLASH_ERR_INVALID_ARG;
  if (logits_dtype != DFLASH_F32 && logits_dtype != DFLASH_BF16) return DFLASH_ERR_INVALID_ARG;
  if (block_size < 2 || block_size > DFLASH_MAX_BLOCK) return DFLASH_ERR_INVALID_ARG;
  dflash_status s = check_kv(h, kv);
  if (s != DFLASH_OK) return s;
  const Dims D = dims(h->cfg);
  if (D.G * block_size > 80) return DFLASH_ERR_UNSUPPORTED;
  if (!aligned16(ws) || !aligned16(target_logits)) return DFLASH_ERR_INVALID_ARG;
  for (int i = 0; i < h->cfg.n_feat_layers; ++i)
    if (!block_feats[i] || !aligned16(block_feats[i])) return DFLASH_ERR_INVALID_ARG;
  if (len_max < 0) return DFLASH_ERR_INVALID_ARG;
  // every position the step can write, len_max + block_size - 1 at most,
  // stays inside each sequence's slab
  for (int b = 0; b < kv->batch; ++b)
    if (static_cast<int64_t>(len_max) + block_size > kv->seq_cap[b]) return DFLASH_ERR_CAPACITY;
  if ((len_max + block_size + 255) / 256 > kMaxAttnChunks * 64) return DFLASH_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool lbf = logits_dtype == DFLASH_BF16;
  return h->cfg.dtype == DFLASH_BF16
             ? step_impl<uint16_t>(h, kv, block_size, dev_len, len_max, target_logits, lbf,
                                   block_feats, draft_ids, anchor_ids, accept, status, ws, st)
             : step_impl<float>(h, kv, block_size, dev_len, len_max, target_logits, lbf,
                                block_feats, draft_ids, anchor_ids, accept, status, ws, st);
}

size_t dflash_stochastic_workspace_size(int32_t batch, int32_t block_size, int32_t vocab) {
  if (batch < 1 || block_size < 2 || vocab < 1) return 0;
  return stochastic_ws_bytes(batch, block_size, vocab);
}

dflash_status dflash_sample_drafts(const float* draft_logits, int32_t batch, int32_t block_size,
                                   int32_t vocab, float temperature, const float* uniforms,
                                   int32_t* draft_ids, void* ws, void* stream) {
  if (!draft_logits || !uniforms || !draft_ids || !ws) return DFLASH_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || block_size < 2 || block_size > DFLASH_MAX_BLOCK || vocab < 1)
    return DFLASH_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return DFLASH_ERR_INVALID_ARG;
  if (!aligned16(draft_logits) || !aligned16(uniforms)) return DFLASH_ERR_INVALID_ARG;
  return hip_status(launch_sample_drafts(draft_logits, batch, block_size, vocab, temperature,
                                         uniforms, draft_ids, ws, static_cast<hipStream_t>(stream)));
}

dflash_status dflash_verify_stochastic(const void* target_logits, dflash_dtype dtype,
                                       const float* draft_logits, const int32_t* draft_ids,
                                       int32_t batch, int32_t block_size, int32_t vocab,
                                       float temperature, const float* r_accept,
                                       const float* u_sample, int32_t* accept,
                                       int32_t* next_token, void* ws, void* stream) {
  if (!target_logits || !draft_logits || !draft_ids || !r_accept || !u_sample || !accept ||
      !next_token || !ws)
    return DFLASH_ERR_INVALID_ARG;
  if (dtype != DFLASH_F32 && dtype != DFLASH_BF16) return DFLASH_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || block_size < 2 || block_size > DFLASH_MAX_BLOCK || vocab < 1)
    return DFLASH_ERR_INVALID_ARG;
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return DFLASH_ERR_INVALID_ARG;
  if (!aligned16(ws) || !aligned16(target_logits) || !aligned16(draft_logits))
    return DFLASH_ERR_INVALID_ARG;
  return hip_status(launch_verify_stochastic(target_logits, dtype == DFLASH_BF16, draft_logits,
                                             draft_ids, batch, block_size, vocab, temperature,
                                             r_accept, u_sample, accept, next_token, ws,
                                             static_cast<hipStream_t>(stream)));
}

dflash_status dflash_set_timing(dflash_handle* h, const dflash_timing_point* points, int32_t n) {
  if (!h || n < 0 || n > 32 || (n > 0 && !points)) return DFLASH_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (points[i].section < DFLASH_SEC_FUSE_GEMM || points[i].section > DFLASH_SEC_LM_GEMM ||
        !points[i].ev_start || !points[i].ev_stop)
      return DFLASH_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) h->timing[i] = points[i];
  h->n_timing = n;
  return DFLASH_OK;
}

size_t dflash_verify_workspace_size(int32_t batch, int32_t block_size, int32_t vocab) {
  if (batch < 1 || block_size < 2 || vocab < 1) return 0;
  return verify_ws_bytes(batch, block_size, vocab);
}

dflash_status dflash_verify_greedy(const void* target_logits, dflash_dtype dtype,
                                   const int32_t* draft_ids, int32_t batch, int32_t block_size,
                                   int32_t vocab, int32_t* accept, int32_t* bonus, void* ws,
                                   void* stream) {
  if (!target_logits || !draft_ids || !accept || !bonus || !ws) return DFLASH_ERR_INVALID_ARG;
  if (dtype != DFLASH_F32 && dtype != DFLASH_BF16) return DFLASH_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || block_size < 2 || block_size > DFLASH_MAX_BLOCK || vocab < 1)
    return DFLASH_ERR_INVALID_ARG;
  if (!aligned16(target_logits)) return DFLASH_ERR_INVALID_ARG;
  return hip_status(launch_verify(target_logits, dtype == DFLASH_BF16, draft_ids, batch,
                                  block_size, vocab, accept, bonus, ws,
                                  static_cast<hipStream_t>(stream)));
}

dflash_status dflash_debug_bf16_round(const float* in, uint16_t* out, int64_t n, int32_t packed,
                                      void* stream) {
  if (!in || !out || n < 0 || (packed != 0 && packed != 1)) return DFLASH_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out) || (packed && n % 2)) return DFLASH_ERR_INVALID_ARG;
  return hip_status(launch_bf16_round(in, out, n, packed, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
