// Host-side paths of libsdv under AddressSanitizer and UndefinedBehaviorSanitizer: the
// launch plans, workspace sizes and every argument check that returns before anything
// is enqueued.  No GPU is needed (no call here reaches a launch).  Exit status 0 when
// every expectation holds; the sanitizers abort the process on a finding.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "../../include/sdv.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                           \
    }                                                                       \
  } while (0)

static void* fake(size_t i) { return (void*)(uintptr_t)(4096 * (i + 1)); }   // never dereferenced

struct Model {
  std::vector<sdv_layer> layers;
  sdv_model m;
  Model(int L, int d, int H, int Hkv, int dh, int F, int V, int dtype, int S = 0, int Vc = 0) {
    layers.resize(L);
    for (int l = 0; l < L; ++l)
      layers[l] = sdv_layer{(const float*)fake(1), fake(2), fake(3), (const float*)fake(4), fake(5), fake(6)};
    memset(&m, 0, sizeof m);
    m.n_layers = L; m.d = d; m.n_heads = H; m.n_kv_heads = Hkv; m.head_dim = dh; m.ffn = F; m.vocab = V;
    m.dtype = dtype; m.eps = 1e-6f; m.rope_theta = 10000.f;
    m.embed = fake(7); m.final_norm = (const float*)fake(8); m.lm_head = fake(9); m.layers = layers.data();
    if (S) { m.n_codebooks = S; m.codebook_size = Vc; m.codebook_base = V - S * Vc; m.codebook = fake(10);
             m.stream_emb = (const float*)fake(11); }
  }
};

int main() {
  // plans of every workload shape: sizes are positive and grow with the pass
  Model m17(24, 2048, 32, 32, 64, 8192, 49152, SDV_BF16), m8(36, 4096, 32, 8, 128, 12288, 151936, SDV_BF16);
  Model mcb(36, 4096, 32, 8, 128, 12288, 151936, SDV_BF16, 8, 1024), toy(2, 256, 4, 4, 64, 1024, 4096, SDV_F32);
  const size_t w17 = sdv_verify_workspace_size(&m17.m, 1, 41, 17, 4096);
  const size_t w8 = sdv_verify_workspace_size(&m8.m, 1, 65, 41, 8192);
  const size_t wcb = sdv_verify_workspace_size(&mcb.m, 64, 41, 17, 16384);
  EXPECT(w17 > 0 && w8 > w17 && wcb > w8 && sdv_verify_workspace_size(&toy.m, 1, 20, 9, 512) > 0);
  for (int T = 1; T <= SDV_MAX_T; T += 7)
    for (int ctx : {0, 1, 17, 4095, 16384, 100000}) EXPECT(sdv_verify_workspace_size(&m8.m, 3, T, 1 + T / 2, ctx) > 0);
  EXPECT(sdv_verify_workspace_size(&m8.m, 1, SDV_MAX_T + 1, 1, 10) == 0);
  EXPECT(sdv_verify_workspace_size(&m8.m, 1, 10, 11, 10) == 0);
  EXPECT(sdv_verify_workspace_size(nullptr, 1, 10, 1, 10) == 0);

  // verify: argument errors come back before any launch
  sdv_kv kv{fake(20), fake(21), (const int32_t*)fake(22), (int32_t*)fake(23), 1000, 600, 1};
  int32_t rows[4] = {0, 1, 2, 3};
  sdv_verify_in in{1, 8, 4, 4, 100, (const int32_t*)fake(24), nullptr, rows, SDV_HEAD_LM, nullptr, 1.f};
  sdv_verify_out out;
  memset(&out, 0, sizeof out);
  out.argmax = (int32_t*)fake(25); out.margin = (float*)fake(26); out.lse = (float*)fake(27); out.err = (int32_t*)fake(28);
  EXPECT(sdv_verify_forward(&m17.m, &kv, &in, &out, nullptr, 0, nullptr) == SDV_ERR_WORKSPACE);
  EXPECT(strlen(sdv_last_error()) > 0);
  sdv_verify_in bad = in;
  bad.T = 0;
  EXPECT(sdv_verify_forward(&m17.m, &kv, &bad, &out, fake(30), 1 << 30, nullptr) == SDV_ERR_SHAPE);
  bad = in;
  bad.max_ctx = 600 * 16;   // beyond the capacity
  EXPECT(sdv_verify_forward(&m17.m, &kv, &bad, &out, fake(30), 1 << 30, nullptr) == SDV_ERR_SHAPE);
  bad = in;
  bad.head = SDV_HEAD_CODEBOOK;
  EXPECT(sdv_verify_forward(&m17.m, &kv, &bad, &out, fake(30), 1 << 30, nullptr) == SDV_ERR_UNSUPPORTED);
  Model odd(2, 256, 4, 4, 96, 1024, 4096, SDV_BF16);
  EXPECT(sdv_verify_forward(&odd.m, &kv, &in, &out, fake(30), 1 << 30, nullptr) == SDV_ERR_UNSUPPORTED);
  // the no-alloc variant rejects a pass beyond its static scratch before touching the device
  sdv_kv kvcb{fake(20), fake(21), (const int32_t*)fake(22), (int32_t*)fake(23), 64 * 1100, 1100, 64};
  sdv_verify_in incb{64, 41, 25, 17, 16384, (const int32_t*)fake(24), nullptr, rows, SDV_HEAD_CODEBOOK, nullptr, 2.f};
  EXPECT(sdv_verify_forward_noalloc(&mcb.m, &kvcb, &incb, &out, nullptr) == SDV_ERR_WORKSPACE);

  // greedy acceptance, rollback, sampling, packing
  EXPECT(sdv_accept_greedy(1, 4096, 1, (const int32_t*)fake(1), nullptr, 1, (const int32_t*)fake(2),
                           (const int32_t*)fake(3), nullptr, (int32_t*)fake(4), (int32_t*)fake(5), nullptr, nullptr,
                           nullptr, nullptr, nullptr, nullptr) == SDV_ERR_SHAPE);
  EXPECT(sdv_kv_rollback(&m17.m, &kv, nullptr, nullptr, nullptr, 0, nullptr, nullptr) == SDV_ERR_NULL);
  EXPECT(sdv_sample_workspace_size(64, 7, 151936) > 0 && sdv_sample_workspace_size(64, SDV_SAMPLE_MAX_K + 1, 10) == 0);
  EXPECT(sdv_accept_sample(4, 3, 100, (const float*)fake(1), (const float*)fake(2), (const int32_t*)fake(3), 0.f, 1,
                           nullptr, (int32_t*)fake(4), (int32_t*)fake(5), nullptr, fake(6), 1 << 20, nullptr,
                           nullptr) == SDV_ERR_SHAPE);
  EXPECT(sdv_packed_bytes(SDV_BF16, 6144, 2048) == (size_t)6144 * 2048 * 2 && sdv_packed_bytes(SDV_BF16, 0, 64) == 0);
  EXPECT(sdv_pack_weights(SDV_PACK_QKV, SDV_BF16, 2048, 96, fake(1), 96, fake(2), 96, fake(3), 96, fake(4),
                          1 << 30, nullptr) == SDV_ERR_UNSUPPORTED);

  // drafting plans
  int32_t lens[4] = {32, 8, 8, 8};
  EXPECT(sdv_draft_workspace_size(&m8.m, 1, 25, 2, lens, 8192) > 0);
  EXPECT(sdv_draft_workspace_size(&m8.m, 1, 25, 4, lens, 8192) > 0);
  int32_t too_wide[17];
  for (int i = 0; i < 17; ++i) too_wide[i] = 9;
  EXPECT(sdv_draft_workspace_size(&m8.m, 1, 25, 17, too_wide, 8192) == 0);      // more than 16 branches
  EXPECT(sdv_draft_workspace_size(&m8.m, 1, 25, 16, too_wide, 8192) == 0);      // 1 + 8 * 16 rows > 128
  sdv_draft_in din{1, 25, 2, 8192, (const int32_t*)fake(1), lens};
  EXPECT(sdv_draft_tree(&m8.m, &kv, &din, (int32_t*)fake(2), (int32_t*)fake(3), nullptr, 0, nullptr) != SDV_OK);

  // hypothesis pool and stream bookkeeping
  sdv_pool pool{(int32_t*)fake(1), (int32_t*)fake(2), (uint64_t*)fake(3), (int32_t*)fake(4), (int32_t*)fake(5), 100, 1000, 4};
  EXPECT(sdv_pool_clear(&pool, nullptr) == SDV_ERR_SHAPE);
  pool.n_slots = 1024;
  EXPECT(sdv_pool_insert(&pool, nullptr, 3, nullptr, nullptr) == SDV_ERR_NULL);
  sdv_stream_cfg sc{8, 1024, 143744, 143000, 1023, 1022, 0, 64, nullptr};
  sdv_stream_cfg bad_sc = sc;
  bad_sc.eoa_code = 1024;
  EXPECT(sdv_phase_mask(&bad_sc, 1, 1, (const float*)fake(1), 10, 0, 10, (const int32_t*)fake(2), nullptr,
                        (int32_t*)fake(3), nullptr, nullptr) == SDV_ERR_SHAPE);
  EXPECT(sdv_stream_commit(&sc, 1, 200, 1, 1, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr) == SDV_ERR_NULL);
  EXPECT(sdv_abi_version() == SDV_ABI_VERSION);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
