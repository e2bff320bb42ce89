/*
 * dflash.h -- C ABI of the MI355X (gfx950) drafter hot path for block-diffusion
 * speculative decoding (DFlash).
 *
 * The drafter turns target hidden states into a draft block in one forward
 * pass and the target's logits into an accepted length.  Four calls carry the
 * work, in the order a speculative cycle uses them:
 *
 *   dflash_fuse_context   hidden states of the sampled target layers -> compact
 *                         context feature (zhichai.net, "DFlash 的架构密码",
 *                         第一层 Feature Fusion; 技术细节补充 / 投影层).
 *   dflash_inject_kv      context feature -> K and V of every drafter layer's
 *                         cache (same page, 第二层 KV Injection).
 *   dflash_draft_block    one forward pass over a block [anchor, mask, ...]
 *                         -> B-1 draft tokens per sequence (same page, 第三层
 *                         Block Diffusion; 训练策略 1 and 3; 技术细节补充 /
 *                         稀疏注意力训练).
 *   dflash_verify_greedy  target logits of the block -> accepted draft count
 *                         and bonus token (same page, 训练策略 1; ai-stack.site,
 *                         "DFlash：基于块扩散的闪存推测解码方法", 实践 2).
 *
 * For sampling at a temperature, dflash_sample_drafts and
 * dflash_verify_stochastic replace the argmax and the greedy verify (same
 * page, FAQ 4: the output keeps the target's distribution).
 * And, for the training layout, dflash_train_forward: several blocks per
 * sequence at sampled anchors, each seeing only the context before its
 * anchor, scored with the position-decayed cross-entropy (same page, 训练策略
 * 1 and 2).  dflash_step_resident chains verify, append and the next draft
 * on the device, with no host sync between cycles.
 *
 * Conventions shared by every call
 *   - Pointers marked (device) are HIP device memory; (host) is host memory.
 *     All buffers belong to the caller.  The library never allocates device
 *     memory: scratch comes from the caller's workspace `ws`, sized by
 *     dflash_workspace_size, 256-byte aligned.  One workspace serves one stream.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and never synchronises it, so a call may be captured
 *     into a HIP graph.
 *   - Arguments are checked on the host before anything is enqueued; a failing
 *     call returns a status and has changed nothing.  A failed launch returns
 *     DFLASH_ERR_HIP.  No C++ exception crosses this interface.
 *   - Storage type: every weight, feature, cache and activation tensor of a
 *     handle has the handle's dtype (float32 or bf16 bit patterns); residual
 *     stream, statistics, softmax and logits are float32 in every case.
 *   - Matrices are row-major, `nn.Linear` layout [out_features, in_features].
 *   - Device pointers must be 16-byte aligned.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_MAX_BATCH 64      /* sequences per call */
#define DFLASH_MAX_BLOCK 16      /* block slots B, anchor included */
#define DFLASH_MAX_LAYERS 16     /* drafter layers */
#define DFLASH_MAX_FEAT 6        /* fused target layers */
#define DFLASH_NOALLOC_SCRATCH_BYTES (64u << 20)   /* static scratch per device */

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_INVALID_ARG = 1,  /* null pointer, bad size, misaligned pointer */
  DFLASH_ERR_CAPACITY = 2,     /* a cache write would pass a sequence's capacity */
  DFLASH_ERR_UNSUPPORTED = 3,  /* shape the kernels do not cover (see dflash_config) */
  DFLASH_ERR_HIP = 4,          /* a HIP runtime call or launch failed */
  DFLASH_ERR_SCRATCH = 5       /* dflash_draft_block_noalloc: the call needs more scratch
                                  than DFLASH_NOALLOC_SCRATCH_BYTES */
} dflash_status;

typedef enum { DFLASH_F32 = 0, DFLASH_BF16 = 1 } dflash_dtype;

/* Drafter shape.  Supported: head_dim 64 or 128; hidden, ffn, n_q_heads*head_dim
 * multiples of 128; n_q_heads a multiple of n_kv_heads with
 * (n_q_heads/n_kv_heads) * block_size <= 80; n_feat_layers 1..6;
 * 1 <= n_layers <= 16; mask_token_id in [0, vocab). */
typedef struct {
  int32_t n_layers;
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;
  int32_t n_feat_layers;
  int32_t mask_token_id;
  float rms_eps;       /* RMSNorm epsilon, e.g. 1e-6 */
  float rope_theta;    /* RoPE base, e.g. 1e6 */
  dflash_dtype dtype;
} dflash_config;

/* One decoder layer (device pointers, handle dtype).  Shapes with H = hidden,
 * Q = n_q_heads*head_dim, KV = n_kv_heads*head_dim, F = ffn:
 * attn_norm, ffn_norm [H]; wq [Q,H]; wk, wv [KV,H]; wo [H,Q]; wg, wu [F,H];
 * wd [H,F]. */
typedef struct {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *wg, *wu, *wd;
} dflash_layer_weights;

/* All weights.  fc [H, n_feat*H] (column block i multiplies the hidden state
 * of the i-th fused layer, ascending layer id), fc_norm [H], final_norm [H],
 * embed [V,H] and lm_head [V,H] (the target's own; they may alias).
 * `layers` is a host array of n_layers entries.  The handle copies the
 * pointers; the memory they point to must outlive the handle. */
typedef struct {
  const void *fc, *fc_norm;
  const dflash_layer_weights *layers;
  const void *final_norm, *embed, *lm_head;
} dflash_weights;

/* The drafter's KV cache for a batch of sequences (caller-owned).
 *   k[l] (device) [n_kv_heads][cap_total][head_dim]  keys of layer l, RoPE applied
 *   v[l] (device) [n_kv_heads][head_dim][cap_total]  values of layer l, transposed
 * Sequence b owns rows [seq_off[b], seq_off[b] + seq_cap[b]) of the position
 * axis; its committed context is the first seq_len[b] of them.  seq_off and
 * seq_cap must be multiples of 32 and the ranges must not overlap.
 * dflash_draft_block uses rows [seq_len[b], seq_len[b] + B) of each sequence as
 * scratch for the block's own K/V, so seq_cap[b] >= seq_len[b] + B is needed
 * there; those rows hold nothing committed.  dflash_inject_kv updates the host
 * array seq_len.  cap_total * head_dim must stay below 2^30 (the attention
 * kernel addresses one kv head's slab with 32-bit byte offsets); larger
 * caches give DFLASH_ERR_UNSUPPORTED. */
typedef struct {
  void *const *k;            /* (host) array [n_layers] of device pointers */
  void *const *v;            /* (host) array [n_layers] of device pointers */
  int32_t batch;
  int64_t cap_total;         /* position rows in each head slab */
  const int64_t *seq_off;    /* (host) [batch] */
  const int32_t *seq_cap;    /* (host) [batch] */
  int32_t *seq_len;          /* (host) [batch] */
} dflash_kv;

typedef struct dflash_handle dflash_handle;

/* 1-based ids of the n_select target layers whose hidden states are fused:
 * spread uniformly from layer 2 to the third-from-last layer, a grid point
 * half-way between two layers rounding up (zhichai.net, "DFlash 的架构密码",
 * 技术细节补充 / 提取层数).  Writes n_select ids to out (host) and returns
 * n_select, or -1 if n_select < 2, n_select > DFLASH_MAX_FEAT,
 * n_target_layers < n_select + 3 or out is NULL. */
int32_t dflash_target_layer_ids(int32_t n_target_layers, int32_t n_select, int32_t *out);

/* Validate a config and weights and make a handle (host memory only). */
dflash_status dflash_create(const dflash_config *cfg, const dflash_weights *w,
                            dflash_handle **out);
dflash_status dflash_destroy(dflash_handle *h);

/* Packed weights: a copy of every bf16 GEMM weight (per layer wq, wk, wv, wo,
 * wg, wu, wd; then fc and lm_head) in fragment-major order -- rows in groups
 * of 16, each group stored as consecutive 1 KB blocks of 16 rows x 32
 * columns, rows past a matrix's end zero -- so that the LDS-tiled GEMMs
 * (fuse/inject of 129 or more rows, blocks of 64 or more rows) read each
 * operand block as one contiguous run instead of 16 strided row pieces.
 * A storage layout only: every result is bit-identical with and without it.
 * The weight-streaming GEMMs (fewer rows) keep reading the row-major weights,
 * which stay required.
 *
 * dflash_packed_weights_size: bytes of the packed copy (bf16 handles; float32
 * handles get DFLASH_ERR_UNSUPPORTED).
 * dflash_pack_weights: writes the copy into dst (device, caller-owned, 16-byte
 * aligned, at least that many bytes) on `stream` and makes the handle's
 * tiled GEMMs read it from then on.  The caller keeps dst alive and unchanged
 * while the handle uses it, orders later calls on other streams after this
 * one, and calls it again after changing the row-major weights.  dst = NULL
 * with bytes = 0 switches back to the row-major weights (then dst may be
 * freed once the calls that used it have finished).  DFLASH_ERR_INVALID_ARG
 * for a short or misaligned dst; on DFLASH_ERR_HIP the handle stays on the
 * row-major weights. */
dflash_status dflash_packed_weights_size(const dflash_handle *h, size_t *bytes);
dflash_status dflash_pack_weights(dflash_handle *h, void *dst, size_t bytes, void *stream);

/* Bytes of workspace that every call below needs for batches up to max_batch,
 * blocks up to max_block slots and fuse/inject calls of up to max_tokens rows. */
dflash_status dflash_workspace_size(const dflash_handle *h, int32_t max_batch,
                                    int32_t max_block, int64_t max_tokens, size_t *bytes);

/* Compact context feature c = RMSNorm(concat(feats) . fc^T) * fc_norm.
 *   feats    (host) array [n_feat_layers] of device pointers, each [n_tokens, H]
 *   ctx_out  (device) [n_tokens, H], handle dtype (bf16: rounded to nearest even)
 * Feature fusion: zhichai.net, "DFlash 的架构密码", 第一层 Feature Fusion and
 * 技术细节补充 / 投影层 (light FC then RMSNorm, no bias). */
dflash_status dflash_fuse_context(dflash_handle *h, const void *const *feats, int64_t n_tokens,
                                  void *ctx_out, void *ws, void *stream);

/* Write the K and V that context features contribute to every drafter layer.
 * For each sequence b, rows [pos_start[b], pos_start[b] + n_new[b]) of its
 * cache receive K = RoPE(c . wk^T) at those positions and V = c . wv^T, for
 * every layer, from the next n_new[b] rows of ctx (rows of sequence 0 first).
 * Then seq_len[b] = pos_start[b] + n_new[b]: rows past it are dropped, which is
 * how a caller rewinds.  pos_start == NULL appends (pos_start[b] = seq_len[b]).
 *   ctx       (device) [sum n_new, H]
 *   pos_start (host) [batch] or NULL, each 0 <= pos_start[b] <= seq_len[b]
 *   n_new     (host) [batch], each >= 0
 * DFLASH_ERR_CAPACITY if pos_start[b] + n_new[b] > seq_cap[b].
 * KV injection: zhichai.net, "DFlash 的架构密码", 第二层 KV Injection (the
 * feature enters every layer's K and V projection, not the input embedding). */
dflash_status dflash_inject_kv(dflash_handle *h, const void *ctx, const int32_t *pos_start,
                               const int32_t *n_new, dflash_kv *kv, void *ws, void *stream);

/* One forward pass of the drafter over one block per sequence.  Slot 0 holds
 * the anchor (the bonus token of the previous cycle), slots 1..B-1 the mask
 * token; slot j sits at position seq_len[b] + j.  Inside a block every slot
 * attends to every slot; a block also sees its own sequence's committed
 * context and nothing else.  Draft j is the lowest-index argmax of slot j's
 * logits through the shared LM head.
 *   anchor_ids        (device) int32 [batch]; a block whose anchor is outside
 *                     [0, vocab) gets draft ids -1 (its rows are computed
 *                     from a clamped embedding row, so nothing is read out
 *                     of bounds, and its drafts are refused)
 *   draft_ids         (device) int32 [batch, B-1]
 *   dbg_final_hidden  (device) float [batch*B, H] or NULL: residual stream after
 *                     the last layer
 *   dbg_logits        (device) float [batch*B, V] or NULL
 * DFLASH_ERR_CAPACITY if seq_len[b] + B > seq_cap[b] for some b.
 * zhichai.net, "DFlash 的架构密码": 第三层 Block Diffusion (one step, one
 * forward pass per block), 训练策略 1 (blocks start at the verified bonus
 * token), 训练策略 3 (shared embedding and LM head), 技术细节补充 / 稀疏注意力
 * 训练 (bidirectional inside a block, no flow between blocks). */
dflash_status dflash_draft_block(dflash_handle *h, dflash_kv *kv, int32_t block_size,
                                 const int32_t *anchor_ids, int32_t *draft_ids,
                                 float *dbg_final_hidden, float *dbg_logits, void *ws,
                                 void *stream);

/* dflash_draft_block without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments, kernels and results as
 * dflash_draft_block; the scratch is a library-owned static device array of
 * DFLASH_NOALLOC_SCRATCH_BYTES (64 MiB) per device -- the current device's
 * copy is used, so `stream` must belong to the current device.  A call whose
 * workspace exceeds it (one sequence of 16 slots needs 37 MiB at the
 * Qwen3-8B shape and 46 MiB at the 27B shape; the chunk partials of block
 * attention grow with the batch, so larger batches at those shapes do not
 * fit) returns DFLASH_ERR_SCRATCH before anything is enqueued.  Nothing is allocated:
 * no hipMalloc, no hipFree.  Every call on a device shares that device's
 * array, so calls that overlap on one device (two streams, two threads) race
 * on it; serialise them.  The first call on a device looks up the array's
 * device address (DFLASH_ERR_HIP if that fails). */
dflash_status dflash_draft_block_noalloc(dflash_handle *h, dflash_kv *kv, int32_t block_size,
                                         const int32_t *anchor_ids, int32_t *draft_ids,
                                         float *dbg_final_hidden, float *dbg_logits,
                                         void *stream);
/* Greedy verification of one block per sequence.  t_j = lowest-index argmax of
 * target row j; accept[b] = the largest a <= B-1 with t_j == draft[b][j] for
 * all j < a; bonus[b] = t_a.  a + 1 tokens are committed (anchor and a drafts)
 * and the bonus token anchors the next block.
 *   target_logits (device) [batch, B, vocab] in `dtype`
 *   draft_ids     (device) int32 [batch, B-1]
 *   accept, bonus (device) int32 [batch]
 *   ws            (device) at least dflash_verify_workspace_size bytes
 * Inputs must be finite.  zhichai.net, "DFlash 的架构密码", 训练策略 1;
 * ai-stack.site, "DFlash：基于块扩散的闪存推测解码方法", 实践 2 (keep up to the
 * last correct token) and 实践 5 (verification stays in a GPU kernel). */
dflash_status dflash_verify_greedy(const void *target_logits, dflash_dtype dtype,
                                   const int32_t *draft_ids, int32_t batch, int32_t block_size,
                                   int32_t vocab, int32_t *accept, int32_t *bonus, void *ws,
                                   void *stream);
size_t dflash_verify_workspace_size(int32_t batch, int32_t block_size, int32_t vocab);

/* Stochastic drafting and lossless verification (speculative sampling).
 * Both distributions are softmax(logits / T) at one temperature T > 0 (finite);
 * every random number is a caller input, so a call is deterministic.
 * ai-stack.site, "DFlash：基于块扩散的闪存推测解码方法", FAQ 4 and the
 * workflow answer (candidates are accepted or rejected by the target's
 * distribution and a rejection is resampled, so the output keeps the target's
 * distribution); the rule is the textbook speculative-sampling one that page
 * points to.
 *
 * dflash_sample_drafts: draft_ids[n][j-1] = argmax_v (z[n][j][v] / T -
 *   log(-log u[n][j-1][v])) for slots j = 1..B-1 (a draw from softmax(z / T);
 *   ties to the lowest index).  draft_logits: device fp32 [batch][B][vocab]
 *   (e.g. dflash_draft_block's dbg_logits); uniforms: device fp32
 *   [batch][B-1][vocab] in (0, 1); draft_ids: device int32 [batch][B-1].
 * dflash_verify_stochastic: draft k (slot k+1, token x = draft_ids[n][k]) is
 *   kept while r[n][k] * p_{k+1}(x) < q_k(x), with q_j = softmax of target row j
 *   (the target's distribution of the token after slot j) and p_j = softmax of
 *   drafter row j; accept[n] = drafts kept (a); next_token[n] = the smallest
 *   column whose cumulative weight exceeds u[n] * total, the weights being
 *   (q_a - p_{a+1})_+ after a rejection and q_{B-1} after B-1 acceptances.
 *   A draft id outside [0, vocab) is never accepted.
 *   target_logits: device [batch][B][vocab] in `dtype`, 16-byte aligned;
 *   draft_logits: device fp32 [batch][B][vocab]; r_accept: device fp32
 *   [batch][B-1] in [0, 1); u_sample: device fp32 [batch] in [0, 1);
 *   accept, next_token: device int32 [batch].
 * Both take ws of dflash_stochastic_workspace_size(batch, B, vocab) bytes
 * (device, 16-byte aligned) and enqueue on `stream`; every logits and uniform
 * buffer must be 16-byte aligned.  Argument errors return before anything is
 * enqueued. */
size_t dflash_stochastic_workspace_size(int32_t batch, int32_t block_size, int32_t vocab);
dflash_status dflash_sample_drafts(const float *draft_logits, int32_t batch, int32_t block_size,
                                   int32_t vocab, float temperature, const float *uniforms,
                                   int32_t *draft_ids, void *ws, void *stream);
dflash_status dflash_verify_stochastic(const void *target_logits, dflash_dtype dtype,
                                       const float *draft_logits, const int32_t *draft_ids,
                                       int32_t batch, int32_t block_size, int32_t vocab,
                                       float temperature, const float *r_accept,
                                       const float *u_sample, int32_t *accept,
                                       int32_t *next_token, void *ws, void *stream);

/* Training-layout forward and its position-weighted loss.  Block i belongs to
 * sequence block_seq[i] of kv and starts at anchor position a = anchor_pos[i]
 * (0 <= a <= seq_len): slot 0 holds anchor_ids[i] (the token at a), slots
 * 1..B-1 the mask token, slot j sits at position a + j.  The block sees the
 * first a context rows of its sequence's cache and its own B slots, nothing
 * else -- several blocks share one sequence's cache, and the cache is only
 * read (the blocks' own K/V live in the workspace).  Slot j >= 1 is scored
 * by cross-entropy against labels[i][j-1] (the token at a + j):
 * slot_loss[i][j-1] = log(sum_v exp(z_v)) - z_label, and
 * loss[0] = sum w_j slot_loss / sum w_j with w_j = exp(-(j-1)/gamma).
 * zhichai.net, "DFlash 的架构密码", 训练策略 1 (blocks start at randomly
 * sampled anchor tokens), 训练策略 2 (exponentially decaying weights over the
 * block), 技术细节补充 / 稀疏注意力训练 (bidirectional inside a block, no flow
 * between blocks).
 *   block_seq, anchor_pos: host int32 [n_blocks]; anchor_ids: device int32
 *   [n_blocks]; labels: device int32 [n_blocks][B-1], each in [0, vocab);
 *   slot_loss: device float32 [n_blocks][B-1]; loss: device float32 [1];
 *   dbg_logits: optional device float32 [n_blocks * B][vocab].
 * n_blocks 1..DFLASH_MAX_BATCH, B 2..DFLASH_MAX_BLOCK, gamma > 0 and finite;
 * ws from dflash_workspace_size(h, >= n_blocks, >= B, ...).  The caller owns
 * every buffer; nothing is allocated.  Argument errors return before anything
 * is enqueued; labels out of range give an undefined loss (not checked on the
 * device). */
dflash_status dflash_train_forward(dflash_handle *h, const dflash_kv *kv, int32_t n_blocks,
                                   int32_t block_size, const int32_t *block_seq,
                                   const int32_t *anchor_pos, const int32_t *anchor_ids,
                                   const int32_t *labels, float gamma, float *slot_loss,
                                   float *loss, float *dbg_logits, void *ws, void *stream);

/* Device-resident step of the speculative loop: verify the current block,
 * append the accepted rows to the context, draft the next block -- with no
 * host read in between, so a caller can run step after step (or capture one
 * step into a HIP graph and replay it) without a device-to-host sync per
 * cycle.  The accepted count never leaves the GPU: the appended rows, the
 * lengths and the next anchor are all taken from device memory
 * (ai-stack.site, "DFlash：基于块扩散的闪存推测解码方法", 实践 5: memory
 * pooled before decoding starts, verification kept on the GPU so no data
 * crosses to the CPU; zhichai.net, "DFlash 的架构密码", 训练策略 1: the
 * block after a verify starts at its bonus token).
 *
 * In stream order, for every sequence b (batch = kv->batch, B = block_size):
 *   1. greedy verify: target_logits (device) [batch][B][vocab] of logits_dtype
 *      against draft_ids (device) [batch][B-1] -> accept[b] (device) and the
 *      bonus token, written to anchor_ids[b] (device), exactly as
 *      dflash_verify_greedy;
 *   2. fusion of block_feats (device) [n_feat_layers] pointers to
 *      [batch * B][hidden] arrays in the handle's dtype: the target's hidden
 *      states at the block's B positions (row b * B + j = slot j of b);
 *   3. injection of slots 0 .. accept[b] of sequence b (the anchor and the
 *      accepted drafts) at positions dev_len[b] + j;
 *   4. dev_len[b] += accept[b] + 1;
 *   5. draft of the next block after dev_len[b] with anchor_ids[b] as its
 *      anchor -> draft_ids, exactly as dflash_draft_block.
 *   dev_len (device) [batch]: committed context lengths; the caller sets them
 *     (e.g. from kv->seq_len) before the first step.  kv->seq_len (host) is
 *     neither read nor updated here; copy dev_len back to it when the loop
 *     ends.
 *   len_max: a host bound on every dev_len[b] during the loop; the launch
 *     plan covers contexts up to it.  Each step adds at most B rows, so
 *     (start length) + steps * B is always enough.  A step whose lengths
 *     would pass len_max leaves them unchanged and sets status[0] = 1
 *     (device int32, never cleared by the library); dev_len values outside
 *     [0, len_max] are clamped.  Nothing is then written outside the slabs.
 *   ws: from dflash_workspace_size(h, >= batch, >= B, any max_tokens).
 * Returns DFLASH_ERR_CAPACITY if len_max + B > seq_cap[b] for some b,
 * DFLASH_ERR_UNSUPPORTED past the attention limits of dflash_draft_block. */
dflash_status dflash_step_resident(dflash_handle *h, dflash_kv *kv, int32_t block_size,
                                   int32_t *dev_len, int32_t len_max, const void *target_logits,
                                   dflash_dtype logits_dtype, const void *const *block_feats,
                                   int32_t *draft_ids, int32_t *anchor_ids, int32_t *accept,
                                   int32_t *status, void *ws, void *stream);

/* Timing hook for profiling.  Sections of the launch sequence: */
typedef enum {
  DFLASH_SEC_FUSE_GEMM = 1,   /* dflash_fuse_context: the fusion GEMM launches */
  DFLASH_SEC_FUSE_NORM = 2,   /* dflash_fuse_context: the RMSNorm launch */
  DFLASH_SEC_INJECT = 3,      /* dflash_inject_kv: the injection GEMM (RoPE in its epilogue) */
  DFLASH_SEC_EMBED = 4,       /* dflash_draft_block: block embedding */
  DFLASH_SEC_ATTN_NORM = 5,   /* per layer: attention RMSNorm */
  DFLASH_SEC_QKV = 6,         /* per layer: QKV projection (+RoPE, cache write) */
  DFLASH_SEC_ATTENTION = 7,   /* per layer: block attention */
  DFLASH_SEC_O_PROJ = 8,      /* per layer: O projection + residual */
  DFLASH_SEC_FFN_NORM = 9,    /* per layer: FFN RMSNorm */
  DFLASH_SEC_GATE_UP = 10,    /* per layer: gate/up projection + SwiGLU */
  DFLASH_SEC_DOWN = 11,       /* per layer: down projection + residual */
  DFLASH_SEC_FINAL_NORM = 12, /* final RMSNorm */
  DFLASH_SEC_LM_HEAD = 13,    /* LM head with fused argmax (GEMM and the argmax fold) */
  DFLASH_SEC_LM_GEMM = 14     /* the LM-head GEMM launch alone (argmax partials in its epilogue);
                                 when one dispatch covers the rows, that dispatch records the
                                 two events itself, so the span is its execution time */
} dflash_section;

typedef struct {
  int32_t section;   /* a dflash_section */
  int32_t layer;     /* drafter layer for per-layer sections, else ignored */
  void *ev_start;    /* hipEvent_t, caller-owned */
  void *ev_stop;     /* hipEvent_t, caller-owned */
} dflash_timing_point;

/* While set, each call that launches a listed section records ev_start on its
 * stream just before the section's first launch and ev_stop just after its
 * last.  The handle copies up to 32 points; n = 0 clears the hook.  For
 * profiling tools (the recorded events add stream markers, no other work). */
dflash_status dflash_set_timing(dflash_handle *h, const dflash_timing_point *points, int32_t n);

/* The float32 -> bf16 rounding (to nearest, ties to even; NaN stays NaN) that
 * every kernel of the library applies where it stores bf16, exposed so that
 * its rounding can be tested on every input.  out[i] = bf16 bits of in[i],
 * i < n; packed = 0 uses the scalar conversion, packed = 1 the pair
 * conversion (n even).  in, out: device, 16-byte aligned; enqueued on
 * `stream`.  DFLASH_ERR_INVALID_ARG for null or misaligned pointers, n < 0,
 * an odd n with packed = 1 or packed outside {0, 1}. */
dflash_status dflash_debug_bf16_round(const float *in, uint16_t *out, int64_t n, int32_t packed,
                                      void *stream);

const char *dflash_status_string(dflash_status s);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
