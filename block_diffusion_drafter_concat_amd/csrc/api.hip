// C ABI front end of libdflash: argument checks, workspace layout and the
// launch sequence of every call.  All checks run before the first launch, so a
// rejected call has no side effects.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <new>

#include "../../include/dflash.h"
#include "gemm_epilogues.h"
#include "gemm_skinny.h"
#include "kernels.h"
#include "kernels_attn.h"

using namespace dflash;

struct dflash_handle {
  dflash_config cfg;
  dflash_weights w;
  dflash_layer_weights layers[DFLASH_MAX_LAYERS];
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

// Largest attention chunk count per (sequence, kv head).
constexpr int kMaxAttnChunks = 32;
// Rows per launch of the weight-streaming GEMM.
constexpr int kMaxRowsPerLaunch = 128;

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

// Split of K over workgroups for a weight-streaming GEMM: enough workgroups to
// keep bytes in flight on 256 CUs, each wave still streaming >= 256 k.
int pick_ksplit(int n_tiles, int K) {
  int ks = 1;
  while (ks < 8 && n_tiles * ks * 2 <= 1024 && (K / (4 * ks * 2)) >= 256 &&
         (K % (4 * ks * 2 * 32)) == 0)
    ks *= 2;
  return ks;
}

// ------------------------------------------------------------- workspace
struct Layout {
  size_t zero_off, zero_bytes;        // argmax keys + counters, cleared per call
  size_t keys_off, cnt_off;
  size_t rope_off, x_off, u_off, q_off, o_off, h_off, part_off, ao_off, aml_off, y_off, ver_off;
  size_t total;
  int n_counters;
};

struct GemmPlan {
  int tiles_qkv, tiles_o, tiles_gu, tiles_d, tiles_lm, tiles_fc, tiles_inj;
};
GemmPlan gemm_plan(const Dims& D) {
  GemmPlan g;
  g.tiles_qkv = (D.qd + 2 * D.kvd) / 32;
  g.tiles_o = D.H / 32;
  g.tiles_gu = D.F / 16;
  g.tiles_d = D.H / 32;
  g.tiles_lm = (D.V + 31) / 32;
  g.tiles_fc = D.H / 32;
  g.tiles_inj = D.L * 2 * D.kvd / 32;
  return g;
}

Layout layout(const dflash_handle* h, int max_batch, int max_block, int64_t max_tokens) {
  const Dims D = dims(h->cfg);
  const size_t es = h->cfg.dtype == DFLASH_BF16 ? 2 : 4;
  const size_t M = static_cast<size_t>(max_batch) * max_block;
  const size_t T = static_cast<size_t>(max_tokens > 0 ? max_tokens : 1);
  const GemmPlan g = gemm_plan(D);
  const int row_launches = static_cast<int>((M + kMaxRowsPerLaunch - 1) / kMaxRowsPerLaunch);
  const int t_launches = static_cast<int>((T + kMaxRowsPerLaunch - 1) / kMaxRowsPerLaunch);
  Layout L{};
  // counters: per layer QKV, O, GU, D tiles and attention (batch x kv heads),
  // per row-launch; LM head one per row-launch; fuse / inject tiles per launch
  const size_t per_layer = static_cast<size_t>(g.tiles_qkv + g.tiles_o + g.tiles_gu + g.tiles_d) *
                               row_launches + static_cast<size_t>(max_batch) * D.Hkv;
  const size_t n_cnt = per_layer * D.L + row_launches +
                       static_cast<size_t>(g.tiles_fc + g.tiles_inj) * t_launches;
  L.n_counters = static_cast<int>(n_cnt);
  size_t off = 0;
  L.zero_off = off;
  L.keys_off = off;
  off += align_up(M * 8);
  L.cnt_off = off;
  off += align_up(n_cnt * 4);
  L.zero_bytes = off - L.zero_off;
  const size_t rope_rows = M > T ? M : T;
  L.rope_off = off; off += align_up(rope_rows * (D.d / 2) * 8);
  L.x_off = off;    off += align_up(M * D.H * 4);
  L.u_off = off;    off += align_up(M * D.H * es);
  L.q_off = off;    off += align_up(M * D.qd * es);
  L.o_off = off;    off += align_up(M * D.qd * es);
  L.h_off = off;    off += align_up(M * D.F * es);
  // split-K partials: per (tile, split) 128 rows x 16 columns x (v0, v1) floats
  constexpr size_t kPartPerTile = static_cast<size_t>(kMaxRowsPerLaunch) * 16 * 2 * 4;
  size_t part = 0;
  const int gemms[6][2] = {{g.tiles_qkv, D.H}, {g.tiles_o, D.qd}, {g.tiles_gu, D.H},
                           {g.tiles_d, D.F},   {g.tiles_fc, D.nf * D.H}, {g.tiles_inj, D.H}};
  for (const auto& gk : gemms) {
    const size_t p = static_cast<size_t>(gk[0]) * pick_ksplit(gk[0], gk[1]) * kPartPerTile;
    part = p > part ? p : part;
  }
  L.part_off = off; off += align_up(part);
  const size_t qr = static_cast<size_t>((D.G * max_block + 15) / 16 * 16);
  const size_t slots = static_cast<size_t>(max_batch) * D.Hkv * kMaxAttnChunks;
  L.ao_off = off;  off += align_up(slots * qr * D.d * 4);
  L.aml_off = off; off += align_up(slots * qr * 8);
  L.y_off = off;   off += align_up(T * D.H * 4);
  L.ver_off = off; off += align_up(verify_ws_bytes(max_batch, max_block, D.V));
  L.total = off;
  return L;
}

template <typename P> P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// ------------------------------------------------------------- GEMM launcher
template <typename T, class Epi>
hipError_t run_skinny(AOperand<T> A, int K, int n_tiles, const Epi& epi, int ksplit, float* part,
                      int* counters, hipStream_t st) {
  const int kper = K / (4 * ksplit);
  dim3 grid(n_tiles, ksplit);
  const int mc = A.mc;
  if (mc <= 16) {
    if (kper % 128 == 0) skinny_gemm_kernel<T, 1, 4, Epi><<<grid, 256, 0, st>>>(A, K, ksplit, part, counters, epi);
    else skinny_gemm_kernel<T, 1, 1, Epi><<<grid, 256, 0, st>>>(A, K, ksplit, part, counters, epi);
  } else if (mc <= 32) {
    if (kper % 128 == 0) skinny_gemm_kernel<T, 2, 4, Epi><<<grid, 256, 0, st>>>(A, K, ksplit, part, counters, epi);
    else skinny_gemm_kernel<T, 2, 1, Epi><<<grid, 256, 0, st>>>(A, K, ksplit, part, counters, epi);
  } else if (mc <= 64) {
    if (kper % 64 == 0) skinny_gemm_kernel<T, 4, 2, Epi><<<grid, 256, 0, st>>>(A, K, ksplit, part, counters, epi);
    else skinny_gemm_kernel<T, 4, 1, Epi><<<grid, 256, 0, st>>>(A, K, ksplit, part, counters, epi);
  } else if (mc <= 128) {
    skinny_gemm_kernel<T, 8, 1, Epi><<<grid, 256, 0, st>>>(A, K, ksplit, part, counters, epi);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Rows [0, M) in launches of at most 128 rows.  `counters` advances by
// n_tiles per launch; `per_launch` adjusts per-launch epilogue state.
template <typename T, class Epi, class PerLaunch>
hipError_t run_rows(AOperand<T> A, int K, int n_tiles, Epi epi, int ksplit, float* part,
                    int* counters, hipStream_t st, PerLaunch per_launch) {
  for (int m0 = 0, li = 0; m0 < A.M; m0 += kMaxRowsPerLaunch, ++li) {
    A.m0 = m0;
    A.mc = A.M - m0 < kMaxRowsPerLaunch ? A.M - m0 : kMaxRowsPerLaunch;
    per_launch(epi, li);
    hipError_t e = run_skinny<T, Epi>(A, K, n_tiles, epi, ksplit, part,
                                      counters + static_cast<size_t>(li) * n_tiles, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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
  return false;
}

dflash_status check_kv(const dflash_handle* h, const dflash_kv* kv) {
  if (!kv || !kv->k || !kv->v || !kv->seq_off || !kv->seq_cap || !kv->seq_len)
    return DFLASH_ERR_INVALID_ARG;
  if (kv->batch < 1 || kv->batch > DFLASH_MAX_BATCH || kv->cap_total <= 0) return DFLASH_ERR_INVALID_ARG;
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
  const int ks = pick_ksplit(g.tiles_fc, K);
  float* Y = at<float>(ws, L.y_off);
  int* cnt = at<int>(ws, L.cnt_off);
  if (ks > 1) {
    const int t_launches = (T_ + kMaxRowsPerLaunch - 1) / kMaxRowsPerLaunch;
    DF_HIP(launch_zero(cnt, static_cast<int64_t>(g.tiles_fc) * t_launches, st));
  }
  EpiStoreF32<T> epi{static_cast<const T*>(h->w.fc), K, Y, D.H};
  DF_HIP(run_rows<T>(A, K, g.tiles_fc, epi, ks, at<float>(ws, L.part_off), cnt, st, NoPerLaunch{}));
  DF_HIP(launch_rmsnorm(h->cfg.dtype == DFLASH_BF16, Y, D.H, h->w.fc_norm, ctx_out, D.H, T_, D.H,
                        h->cfg.rms_eps, st));
  return DFLASH_OK;
}

template <typename T>
dflash_status inject_impl(dflash_handle* h, const void* ctx, const SeqTable& seq, int total,
                          dflash_kv* kv, void* ws, hipStream_t st) {
  const Dims D = dims(h->cfg);
  const Layout L = layout(h, 1, 1, total);
  const GemmPlan g = gemm_plan(D);
  float2* rope = at<float2>(ws, L.rope_off);
  DF_HIP(launch_rope_rows(rope, total, D.d, static_cast<double>(h->cfg.rope_theta), seq, st));
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
  epi.rope = rope;
  epi.seq = seq;
  const int ks = pick_ksplit(g.tiles_inj, D.H);
  int* cnt = at<int>(ws, L.cnt_off);
  if (ks > 1) {
    const int t_launches = (total + kMaxRowsPerLaunch - 1) / kMaxRowsPerLaunch;
    DF_HIP(launch_zero(cnt, static_cast<int64_t>(g.tiles_inj) * t_launches, st));
  }
  DF_HIP(run_rows<T>(a_single<T>(ctx, D.H, D.H, total), D.H, g.tiles_inj, epi, ks,
                     at<float>(ws, L.part_off), cnt, st, NoPerLaunch{}));
  return DFLASH_OK;
}

template <typename T>
dflash_status draft_impl(dflash_handle* h, dflash_kv* kv, int B, const int32_t* anchors,
                         int32_t* draft, float* dbg_h, float* dbg_z, void* ws, hipStream_t st) {
  const Dims D = dims(h->cfg);
  const int nb = kv->batch, M = nb * B;
  const bool bf = h->cfg.dtype == DFLASH_BF16;
  const Layout L = layout(h, nb, B, 1);
  const GemmPlan g = gemm_plan(D);
  const int row_launches = (M + kMaxRowsPerLaunch - 1) / kMaxRowsPerLaunch;

  SeqTable seq{};
  seq.n = nb;
  int max_keys = 0;
  for (int b = 0; b < nb; ++b) {
    seq.len[b] = kv->seq_len[b];
    seq.off[b] = kv->seq_off[b];
    max_keys = (kv->seq_len[b] + B > max_keys) ? kv->seq_len[b] + B : max_keys;
  }
  unsigned long long* keys = at<unsigned long long>(ws, L.keys_off);
  int* cnt = at<int>(ws, L.cnt_off);
  float2* rope = at<float2>(ws, L.rope_off);
  float* x = at<float>(ws, L.x_off);
  T* u = at<T>(ws, L.u_off);
  T* qb = at<T>(ws, L.q_off);
  T* ob = at<T>(ws, L.o_off);
  T* hb = at<T>(ws, L.h_off);
  float* part = at<float>(ws, L.part_off);

  DF_HIP(launch_embed(bf, h->w.embed, D.H, D.V, anchors, h->cfg.mask_token_id, nb, B, x, rope, D.d,
                      static_cast<double>(h->cfg.rope_theta), seq, at<uint32_t>(ws, L.zero_off),
                      static_cast<int64_t>(L.zero_bytes / 4), st));

  // attention split: chunks of >= 256 keys, at most kMaxAttnChunks per sequence
  int chunk = 256;
  while ((max_keys + chunk - 1) / chunk > kMaxAttnChunks) chunk += 128;
  AttnArgs aa{};
  aa.q = qb;
  aa.ldq = D.qd;
  aa.cap = kv->cap_total;
  aa.o = ob;
  aa.part_o = at<float>(ws, L.ao_off);
  aa.part_ml = at<float2>(ws, L.aml_off);
  aa.B = B;
  aa.G = D.G;
  aa.n_kv = D.Hkv;
  aa.chunk = chunk;
  aa.max_chunks = (max_keys + chunk - 1) / chunk;
  aa.scale_log2 = static_cast<float>(1.4426950408889634 / sqrt(static_cast<double>(D.d)));
  aa.seq = seq;

  int* c = cnt;
  for (int l = 0; l < D.L; ++l) {
    const dflash_layer_weights& w = h->layers[l];
    // attention half
    DF_HIP(launch_rmsnorm(bf, x, D.H, w.attn_norm, u, D.H, M, D.H, h->cfg.rms_eps, st));
    {
      EpiQKV<T> e{};
      e.wq = static_cast<const T*>(w.wq);
      e.wk = static_cast<const T*>(w.wk);
      e.wv = static_cast<const T*>(w.wv);
      e.K = D.H; e.d = D.d; e.Hq = D.Hq; e.Hkv = D.Hkv; e.B = B;
      e.q = qb; e.ldq = D.qd;
      e.kc = static_cast<T*>(kv->k[l]);
      e.vc = static_cast<T*>(kv->v[l]);
      e.cap = kv->cap_total;
      e.rope = rope;
      e.seq = seq;
      const int ks = pick_ksplit(g.tiles_qkv, D.H);
      DF_HIP(run_rows<T>(a_single<T>(u, D.H, D.H, M), D.H, g.tiles_qkv, e, ks, part, c, st,
                         NoPerLaunch{}));
      c += g.tiles_qkv * row_launches;
    }
    aa.kc = kv->k[l];
    aa.vc = kv->v[l];
    aa.counters = c;
    c += nb * D.Hkv;
    DF_HIP(launch_block_attention(bf, D.d, aa, nb, st));
    {
      EpiResidual<T> e{static_cast<const T*>(w.wo), D.qd, x, D.H};
      const int ks = pick_ksplit(g.tiles_o, D.qd);
      DF_HIP(run_rows<T>(a_single<T>(ob, D.qd, D.qd, M), D.qd, g.tiles_o, e, ks, part, c, st,
                         NoPerLaunch{}));
      c += g.tiles_o * row_launches;
    }
    // feed-forward half
    DF_HIP(launch_rmsnorm(bf, x, D.H, w.ffn_norm, u, D.H, M, D.H, h->cfg.rms_eps, st));
    {
      EpiSwiGLU<T> e{static_cast<const T*>(w.wg), static_cast<const T*>(w.wu), D.H, hb, D.F};
      const int ks = pick_ksplit(g.tiles_gu, D.H);
      DF_HIP(run_rows<T>(a_single<T>(u, D.H, D.H, M), D.H, g.tiles_gu, e, ks, part, c, st,
                         NoPerLaunch{}));
      c += g.tiles_gu * row_launches;
    }
    {
      EpiResidual<T> e{static_cast<const T*>(w.wd), D.F, x, D.H};
      const int ks = pick_ksplit(g.tiles_d, D.F);
      DF_HIP(run_rows<T>(a_single<T>(hb, D.F, D.F, M), D.F, g.tiles_d, e, ks, part, c, st,
                         NoPerLaunch{}));
      c += g.tiles_d * row_launches;
    }
  }
  if (dbg_h)
    DF_HIP(hipMemcpyAsync(dbg_h, x, static_cast<size_t>(M) * D.H * 4, hipMemcpyDeviceToDevice, st));
  DF_HIP(launch_rmsnorm(bf, x, D.H, h->w.final_norm, u, D.H, M, D.H, h->cfg.rms_eps, st));
  {
    EpiLMHead<T> e{};
    e.W = static_cast<const T*>(h->w.lm_head);
    e.K = D.H; e.V = D.V; e.B = B; e.n_tiles = g.tiles_lm;
    e.keys = keys;
    e.counter = c;
    e.draft = draft;
    e.dbg = dbg_z;
    int* lm_cnt = c;
    DF_HIP(run_rows<T>(a_single<T>(u, D.H, D.H, M), D.H, g.tiles_lm, e, 1, part, c, st,
                       [lm_cnt](EpiLMHead<T>& ep, int li) { ep.counter = lm_cnt + li; }));
  }
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
  *out = h;
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
  *bytes = layout(h, max_batch, max_block, max_tokens).total;
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

}  // extern "C"
