// Launcher of the block-attention kernel (internal to libdflash.so).
#pragma once

#include "device_common.h"

namespace dflash {

// Longest-first order: at most this many (sequence, chunk) entries.
constexpr int kAttnOrderMax = 256;

struct AttnArgs {
  const void* q;        // [batch*B, n_q*D] block queries after RoPE
  int64_t ldq;          // row stride of q and o, elements
  const void* kc;       // layer K cache [n_kv][cap][D]
  const void* vc;       // layer V cache [n_kv][D][cap]
  int64_t cap;
  void* o;              // [batch*B, n_q*D] attention output (row stride ldq)
  int ofrag;            // 1: o stored fragment-major (frag_major(), row length ldq)
  float* part_o;        // [batch][n_kv][max_chunks][NQ][D/16][64 lanes][4] (C layout)
  float2* part_ml;      // [batch][n_kv][max_chunks][ceil16(G*B)]  (max, sum), base 2
  int B, G, n_kv;
  int head_dim;
  int chunk;            // keys per workgroup, multiple of 128
  int max_chunks;       // grid.x
  float scale_log2;     // log2(e) / sqrt(D)
  SeqTable seq;         // len[b], off[b]
  // Training layout (kb set): entry b is a block whose keys are the first
  // len[b] rows of its sequence's cache slab (off[b]) plus its own B keys,
  // which sit in rows [b * kTrainSlab, + B) of these buffers (same layouts as
  // kc / vc, capacity capb); null for inference, where the block's keys
  // follow the context inside the cache slab.
  const void* kb;
  const void* vb;
  int64_t capb;
  // Longest-first order (n_order > 0): a 1-D grid of n_order * n_kv
  // workgroups; workgroup w takes entry order[w / n_kv] = b * 128 + c (chunk c
  // of sequence b) and kv head w % n_kv.  Otherwise grid (chunk, kv head, b).
  int n_order;
  uint16_t order[kAttnOrderMax];
};

// The (chunk, kv head, sequence) of this workgroup.
__device__ __forceinline__ void attn_wg_coords(const AttnArgs& p, int& c, int& g, int& b) {
  if (p.n_order > 0) {
    const int w = blockIdx.x;
    const int it = w / p.n_kv;
    g = w - it * p.n_kv;
    const int e = p.order[it];
    b = e >> 7;
    c = e & 127;
  } else {
    c = blockIdx.x;
    g = blockIdx.y;
    b = blockIdx.z;
  }
}

// The keys workgroup c of entry b reads: a range of one source's rows.
// Inference: keys [0, len + B) of the cache slab, in chunks.  Training
// layout: keys [0, len) of the cache slab in chunks, then one more chunk
// with the block's own B keys from the block buffer.
struct KeySpan {
  int kbeg, kend;      // key range within the source
  int n_src;           // keys the source holds for this entry (row clamp bound)
  int n_chunks;        // chunks of the entry
  int64_t base, cap;   // first row of the entry in the source, source capacity
  const void* k;
  const void* v;
};
__device__ __forceinline__ int attn_n_chunks(const AttnArgs& p, int b) {
  const bool train = p.kb != nullptr;
  const int n_ctx = seq_len_of(p.seq, b) + (train ? 0 : p.B);
  return (n_ctx + p.chunk - 1) / p.chunk + (train ? 1 : 0);
}
__device__ __forceinline__ bool attn_key_span(const AttnArgs& p, int b, int c, KeySpan& s) {
  const bool train = p.kb != nullptr;
  const int n_ctx = seq_len_of(p.seq, b) + (train ? 0 : p.B);
  const int nck = (n_ctx + p.chunk - 1) / p.chunk;
  s.n_chunks = nck + (train ? 1 : 0);
  if (c >= s.n_chunks) return false;
  if (train && c == nck) {
    s.kbeg = 0;
    s.kend = p.B;
    s.n_src = p.B;
    s.base = static_cast<int64_t>(b) * kTrainSlab;
    s.cap = p.capb;
    s.k = p.kb;
    s.v = p.vb;
  } else {
    s.kbeg = c * p.chunk;
    s.kend = min(s.kbeg + p.chunk, n_ctx);
    s.n_src = n_ctx;
    s.base = p.seq.off[b];
    s.cap = p.cap;
    s.k = p.kc;
    s.v = p.vc;
  }
  return true;
}

hipError_t launch_block_attention(bool bf16, int head_dim, const AttnArgs& a, int batch,
                                  hipStream_t st);

}  // namespace dflash
