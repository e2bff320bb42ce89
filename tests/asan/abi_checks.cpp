// Host-side checks of the C ABI under AddressSanitizer and UBSan (CPU only).
//
// Every call below is rejected by the library's host checks before anything
// is enqueued, or -- with --no-device on a machine without a GPU -- reaches
// its first launch and fails there with DFLASH_ERR_HIP.  The device
// addresses are fake and never dereferenced by host code; a sanitizer report
// or a wrong status fails the run (exit code != 0).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "dflash.h"

static int failures = 0;
#define EXPECT(call, want)                                                        \
  do {                                                                            \
    const int got_ = static_cast<int>(call);                                      \
    if (got_ != static_cast<int>(want)) {                                         \
      std::fprintf(stderr, "%s:%d: %s -> %d, want %d\n", __FILE__, __LINE__, #call, \
                   got_, static_cast<int>(want));                                 \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

static void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t{1} << 40) + i * 4096); }

struct Model {
  dflash_config cfg{};
  std::vector<dflash_layer_weights> layers;
  dflash_weights w{};
};

static Model make_model(int layers, int hidden, int hq, int hkv, int d, int ffn, int vocab,
                        dflash_dtype dt) {
  Model m;
  m.cfg = dflash_config{layers, hidden, hq, hkv, d, ffn, vocab, 5, vocab - 1, 1e-6f, 1e6f, dt};
  uintptr_t k = 0;
  for (int l = 0; l < layers; ++l)
    m.layers.push_back(dflash_layer_weights{fake(k++), fake(k++), fake(k++), fake(k++), fake(k++),
                                            fake(k++), fake(k++), fake(k++), fake(k++)});
  m.w = dflash_weights{fake(k++), fake(k++), m.layers.data(), fake(k++), fake(k++), fake(k++)};
  return m;
}

struct Cache {
  std::vector<void*> k, v;
  std::vector<int64_t> off;
  std::vector<int32_t> cap, len;
  dflash_kv kv{};
};

static Cache make_cache(int layers, std::vector<int32_t> lens, std::vector<int32_t> caps,
                        int64_t cap_total = 0) {
  Cache c;
  for (int l = 0; l < layers; ++l) {
    c.k.push_back(fake(1000 + l));
    c.v.push_back(fake(2000 + l));
  }
  int64_t o = 0;
  for (size_t b = 0; b < caps.size(); ++b) {
    c.off.push_back(o);
    o += caps[b];
  }
  c.cap = caps;
  c.len = lens;
  c.kv = dflash_kv{c.k.data(), c.v.data(), static_cast<int32_t>(caps.size()),
                   cap_total ? cap_total : o, c.off.data(), c.cap.data(), c.len.data()};
  return c;
}

int main(int argc, char** argv) {
  const bool no_device = argc > 1 && std::strcmp(argv[1], "--no-device") == 0;
  int32_t ids[8];
  EXPECT(dflash_target_layer_ids(36, 5, ids), 5);
  EXPECT(ids[0] * 10000 + ids[4], 2 * 10000 + 34);
  EXPECT(dflash_target_layer_ids(7, 5, ids), -1);
  EXPECT(dflash_target_layer_ids(40, 5, nullptr), -1);

  Model m = make_model(5, 4096, 32, 8, 128, 12288, 151936, DFLASH_BF16);
  dflash_handle* h = nullptr;
  EXPECT(dflash_create(nullptr, &m.w, &h), DFLASH_ERR_INVALID_ARG);
  dflash_config bad = m.cfg;
  bad.head_dim = 96;
  EXPECT(dflash_create(&bad, &m.w, &h), DFLASH_ERR_UNSUPPORTED);
  bad = m.cfg;
  bad.mask_token_id = bad.vocab;
  EXPECT(dflash_create(&bad, &m.w, &h), DFLASH_ERR_INVALID_ARG);
  EXPECT(dflash_create(&m.cfg, &m.w, &h), DFLASH_OK);

  size_t bytes = 0;
  EXPECT(dflash_workspace_size(h, 16, 16, 2048, &bytes), DFLASH_OK);
  EXPECT(bytes > 0, 1);
  EXPECT(dflash_workspace_size(h, 65, 16, 1, &bytes), DFLASH_ERR_INVALID_ARG);

  void* p = fake(7);
  int32_t* ip = static_cast<int32_t*>(fake(8));
  // draft: capacity, block size, overlap, slab bound, scratch limit
  Cache full = make_cache(5, {60}, {64});
  EXPECT(dflash_draft_block(h, &full.kv, 16, ip, ip, nullptr, nullptr, p, nullptr),
         DFLASH_ERR_CAPACITY);
  Cache c1 = make_cache(5, {10}, {64});
  EXPECT(dflash_draft_block(h, &c1.kv, 17, ip, ip, nullptr, nullptr, p, nullptr),
         DFLASH_ERR_INVALID_ARG);
  Cache ov = make_cache(5, {1, 1}, {64, 64});
  ov.off[1] = 32;
  EXPECT(dflash_draft_block(h, &ov.kv, 8, ip, ip, nullptr, nullptr, p, nullptr),
         DFLASH_ERR_INVALID_ARG);
  Cache huge = make_cache(5, {10}, {1 << 23});
  EXPECT(dflash_draft_block(h, &huge.kv, 8, ip, ip, nullptr, nullptr, p, nullptr),
         DFLASH_ERR_UNSUPPORTED);
  Cache four = make_cache(5, {10, 10, 10, 10}, {64, 64, 64, 64});
  EXPECT(dflash_draft_block_noalloc(h, &four.kv, 16, ip, ip, nullptr, nullptr, nullptr),
         DFLASH_ERR_SCRATCH);
  // inject: past capacity, start past the committed length (lengths untouched)
  int32_t n_new[1] = {60}, pos[1] = {11};
  EXPECT(dflash_inject_kv(h, p, nullptr, n_new, &c1.kv, p, nullptr), DFLASH_ERR_CAPACITY);
  n_new[0] = 1;
  EXPECT(dflash_inject_kv(h, p, pos, n_new, &c1.kv, p, nullptr), DFLASH_ERR_INVALID_ARG);
  EXPECT(c1.len[0], 10);
  // fusion, verify, training layout, stochastic, resident step, timing, rounding
  const void* feats[6] = {p, p, p, p, p, p};
  EXPECT(dflash_fuse_context(h, feats, -1, p, p, nullptr), DFLASH_ERR_INVALID_ARG);
  EXPECT(dflash_fuse_context(h, feats, 0, p, p, nullptr), DFLASH_OK);
  EXPECT(dflash_verify_greedy(p, DFLASH_BF16, ip, 1, 1, 10, ip, ip, p, nullptr),
         DFLASH_ERR_INVALID_ARG);
  int32_t bseq[2] = {0, 5}, apos[2] = {3, 0};
  EXPECT(dflash_train_forward(h, &c1.kv, 2, 8, bseq, apos, ip, ip, 4.f, static_cast<float*>(p),
                              static_cast<float*>(p), nullptr, p, nullptr),
         DFLASH_ERR_INVALID_ARG);
  EXPECT(dflash_sample_drafts(static_cast<float*>(p), 1, 8, 1024, 0.f, static_cast<float*>(p), ip,
                              p, nullptr),
         DFLASH_ERR_INVALID_ARG);
  EXPECT(dflash_step_resident(h, &c1.kv, 8, ip, 60, p, DFLASH_BF16, feats, ip, ip, ip, ip, p,
                              nullptr),
         DFLASH_ERR_CAPACITY);
  dflash_timing_point tp{99, 0, p, p};
  EXPECT(dflash_set_timing(h, &tp, 1), DFLASH_ERR_INVALID_ARG);
  EXPECT(dflash_debug_bf16_round(static_cast<float*>(p), static_cast<uint16_t*>(p), 7, 1, nullptr),
         DFLASH_ERR_INVALID_ARG);
  EXPECT(std::strlen(dflash_status_string(DFLASH_ERR_SCRATCH)) > 0, 1);
  // weight packing: size query, short / misaligned buffers, unbinding
  size_t packed = 0;
  EXPECT(dflash_packed_weights_size(h, &packed), DFLASH_OK);
  EXPECT(packed > 0, 1);
  EXPECT(dflash_pack_weights(h, p, packed - 1, nullptr), DFLASH_ERR_INVALID_ARG);
  EXPECT(dflash_pack_weights(h, static_cast<char*>(p) + 8, packed, nullptr),
         DFLASH_ERR_INVALID_ARG);
  EXPECT(dflash_pack_weights(h, nullptr, 0, nullptr), DFLASH_OK);

  if (no_device) {
    // arguments that pass every host check: the first launch fails
    EXPECT(dflash_verify_greedy(p, DFLASH_BF16, ip, 2, 8, 1024, ip, ip, p, nullptr), DFLASH_ERR_HIP);
    EXPECT(dflash_draft_block(h, &c1.kv, 8, ip, ip, nullptr, nullptr, p, nullptr), DFLASH_ERR_HIP);
    n_new[0] = 3;
    EXPECT(dflash_inject_kv(h, p, nullptr, n_new, &c1.kv, p, nullptr), DFLASH_ERR_HIP);
    EXPECT(c1.len[0], 10);
    EXPECT(dflash_fuse_context(h, feats, 4, p, p, nullptr), DFLASH_ERR_HIP);
    EXPECT(dflash_draft_block_noalloc(h, &c1.kv, 8, ip, ip, nullptr, nullptr, nullptr),
           DFLASH_ERR_HIP);
    EXPECT(dflash_pack_weights(h, p, packed, nullptr), DFLASH_ERR_HIP);
  }
  EXPECT(dflash_destroy(h), DFLASH_OK);
  EXPECT(dflash_destroy(nullptr), DFLASH_ERR_INVALID_ARG);
  if (failures) std::fprintf(stderr, "%d check(s) failed\n", failures);
  else std::printf("abi checks ok%s\n", no_device ? " (incl. launches without a device)" : "");
  return failures ? 1 : 0;
}
