// Host-side launchers of the gfx950 kernels (internal to libdflash.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace dflash {

// ---------------------------------------------------------------- small kernels
// Block inputs: x[m] = embed[token(m)] (fp32) and u[m] = RMSNorm(x[m]) * gain
// (layer 0's attention norm), one workgroup per block slot.
hipError_t launch_embed(bool bf16, const void* embed, int H, int V, const int32_t* anchors,
                        int mask_id, int batch, int B, float* x, const void* gain, void* u,
                        float eps, hipStream_t st, bool frag = false);

// Row m: v = x[m] + sum_s part[s * split_stride + m*H ...] (x and part may be
// null); x[m] = v when x; out[m] = RMSNorm(v) * gain when out (handle type).
hipError_t launch_resid_rmsnorm(bool bf16, float* x, const float* part, int n_split,
                                int64_t split_stride, const void* gain, void* out, int rows,
                                int H, float eps, hipStream_t st, bool frag = false);

// QKV of a batch of blocks from ks fp32 partial slabs [ks][rows][qd + 2 kvd]
// (slab = rows * (qd + 2 kvd)): sum, RoPE on q and k at the block positions,
// q -> q[rows][ldq], k -> K cache rows, v -> transposed V cache (block_rows:
// rows b * kTrainSlab + j of a training layout's block K/V buffer instead,
// kc / vc / cap then naming that buffer).
hipError_t launch_qkv_finish(bool bf16, const float* part, int ks, int64_t slab, int rows, int qd,
                             int kvd, int d, int B, void* q, int64_t ldq, void* kc, void* vc,
                             int64_t cap, const RopeFreq& freq, const SeqTable& seq,
                             hipStream_t st, bool block_rows = false);

// Training layout: per-slot cross-entropy from the LM head's (max, sum,
// label logit) partials [rows][n_wg], then the weighted mean over all slots
// (rows = n_blocks * B; slot 0 of a block is not scored).
hipError_t launch_lm_loss(const float4* part, int n_wg, int rows, int B, float gamma,
                          float* slot_loss, float* loss, hipStream_t st);

// Stochastic drafting and verification (k_sample.hip): Gumbel-max draws of
// slots 1..B-1 from fp32 drafter logits [N][B][V] with uniforms [N][B-1][V];
// speculative-sampling verification of drafts [N][B-1] against target logits
// [N][B][V] (bf16 or fp32) with accept uniforms r [N][B-1] and sampling
// uniforms u [N].  Workspace: stochastic_ws_bytes(N, B, V).
size_t stochastic_ws_bytes(int batch, int B, int V);
hipError_t launch_sample_drafts(const float* logits, int batch, int B, int V, float temperature,
                                const float* uniforms, int32_t* ids, void* ws, hipStream_t st);
hipError_t launch_verify_stochastic(const void* target_logits, bool bf16, const float* draft_logits,
                                    const int32_t* drafts, int batch, int B, int V,
                                    float temperature, const float* r, const float* u,
                                    int32_t* accept, int32_t* next_tok, void* ws, hipStream_t st);

// Draft ids from the LM head's per-workgroup (value, index) partials [rows][n_wg];
// the drafts of a block whose anchor (anchors[row / B]) is outside [0, V) are -1.
hipError_t launch_lm_argmax_finalize(const float2* part, int n_wg, int rows, int B,
                                     const int32_t* anchors, int V, int32_t* draft,
                                     hipStream_t st);

// Greedy verify: per-chunk row argmax, then per-sequence prefix scan.
size_t verify_ws_bytes(int batch, int B, int V);
hipError_t launch_advance_lengths(int32_t* len, const int32_t* accept, int n, int B, int len_max,
                                  int32_t* status, hipStream_t st);
hipError_t launch_verify(const void* logits, bool bf16, const int32_t* drafts, int batch, int B,
                         int V, int32_t* accept, int32_t* bonus, void* ws, hipStream_t st);

// float32 -> bf16 with the library's own rounding (scalar or pair conversion).
hipError_t launch_bf16_round(const float* in, uint16_t* out, int64_t n, int packed,
                             hipStream_t st);

// Row-major [N, K] bf16 (K a multiple of 32) -> fragment-major, rows padded
// with zeros to a multiple of 16 (dst holds ceil(N/16)*16 x K elements).
hipError_t launch_pack_frag(const uint16_t* src, int N, int K, uint16_t* dst, hipStream_t st);

}  // namespace dflash
