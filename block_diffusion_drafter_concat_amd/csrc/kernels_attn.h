// Launcher of the block-attention kernel (internal to libdflash.so).
#pragma once

#include "device_common.h"

namespace dflash {

struct AttnArgs {
  const void* q;        // [batch*B, n_q*D] block queries after RoPE
  int64_t ldq;          // row stride of q and o, elements
  const void* kc;       // layer K cache [n_kv][cap][D]
  const void* vc;       // layer V cache [n_kv][D][cap]
  int64_t cap;
  void* o;              // [batch*B, n_q*D] attention output
  float* part_o;        // [batch][n_kv][max_chunks][NQ][D/16][64 lanes][4] (C layout)
  float2* part_ml;      // [batch][n_kv][max_chunks][ceil16(G*B)]  (max, sum), base 2
  int B, G, n_kv;
  int head_dim;
  int chunk;            // keys per workgroup, multiple of 128
  int max_chunks;       // grid.x
  float scale_log2;     // log2(e) / sqrt(D)
  SeqTable seq;         // len[b], off[b]
};

hipError_t launch_block_attention(bool bf16, int head_dim, const AttnArgs& a, int batch,
                                  hipStream_t st);

}  // namespace dflash
