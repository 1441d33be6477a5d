// Drives the host half of libwave (planner, tail balancing, C ABI shim) over
// a grid of plans and through every entry point, for a build under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Device pointers are fake
// (aligned, never dereferenced: the kernel launchers are host stubs).
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "wave.h"

namespace stub {
extern long launches;
}

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed: %s (line %d): %s\n", #cond, __LINE__, \
                   wave_last_error());                                           \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

static void* fake(uintptr_t v) { return reinterpret_cast<void*>(v); }

static long exercise(const wave_plan_params& prm) {
  wave_plan_t* plan = nullptr;
  CHECK(wave_plan(&prm, &plan) == WAVE_OK && plan);
  wave_plan_view v;
  CHECK(wave_plan_view_get(plan, &v) == WAVE_OK);
  long sum = 0;  // touch every view array
  for (int t = 0; t <= v.num_rounds; ++t) sum += v.round_node_begin[t] + v.round_write_begin[t] + v.round_work_begin[t];
  for (int t = 0; t < v.num_rounds; ++t) sum += v.round_q_rows[t] + v.round_src_rows[t];
  for (int n = 0; n < v.num_nodes; ++n) {
    const wave_node& nd = v.nodes[n];
    for (int c = 0; c < nd.ctx_count; ++c) sum += v.ctx[nd.ctx_begin + c].phys_slot;
    for (int w = 0; w < nd.write_count; ++w) sum += v.writes[nd.write_begin + w].len;
  }
  for (int w = 0; w < v.num_work; ++w) sum += v.work[w].keys;
  size_t bytes = 0;
  CHECK(wave_plan_desc_size(plan, &bytes) == WAVE_OK && bytes % 4 == 0);
  std::vector<int32_t> desc(bytes / 4);
  CHECK(wave_plan_desc_pack(plan, desc.data(), bytes) == WAVE_OK);
  CHECK(wave_plan_desc_pack(plan, desc.data(), bytes - 4) == WAVE_ERR_INVALID_ARG);

  const int heads = 3, hd = 128, lpad = (v.max_slot_len + 63) / 64 * 64;
  wave_kv_cache cache{fake(0x100000), fake(0x200000), v.num_phys_slots, heads, hd, lpad};
  const void* d = fake(0x300000);
  void* st = nullptr;
  const int64_t row = heads * hd;
  for (int t = 0; t < v.num_rounds; ++t) {
    CHECK(kv_write(plan, d, t, &cache, fake(0x400000), fake(0x500000), WAVE_DTYPE_BF16, row, st) == WAVE_OK);
    size_t ws = 0;
    int32_t items = -1, splits = -1;
    CHECK(wave_attn_workspace(plan, t, heads, hd, 0, &ws, &items, &splits) == WAVE_OK);
    CHECK(wave_attn(plan, d, t, &cache, fake(0x600000), WAVE_DTYPE_BF16, row, fake(0x700000), nullptr, 0.1f,
                    ws ? fake(0x800000) : nullptr, ws, st) == WAVE_OK);
    CHECK(wave_attn(plan, d, t, &cache, fake(0x600000), WAVE_DTYPE_FP32, row, fake(0x700000),
                    static_cast<float*>(fake(0x900000)), 0.1f, nullptr, 0, st) == WAVE_OK);
    int32_t used = 0;
    CHECK(wave_attn_splitkv_workspace(plan, t, heads, hd, 0, &ws, &used) == WAVE_OK && used >= 1);
    CHECK(wave_attn_splitkv(plan, d, t, &cache, fake(0x600000), WAVE_DTYPE_BF16, row, fake(0x700000), nullptr,
                            0.1f, 0, fake(0x800000), ws, st) == WAVE_OK);
    const int32_t rc = wave_attn_splitkv_noalloc(plan, d, t, &cache, fake(0x600000), WAVE_DTYPE_BF16, row,
                                                 fake(0x700000), nullptr, 0.1f, 2, st);
    CHECK(rc == WAVE_OK || rc == WAVE_ERR_CAPACITY);
    const void* srcs[2] = {fake(0x400000), fake(0x400000)};
    const void* qs[2] = {fake(0x600000), fake(0x600000)};
    void* os[2] = {fake(0x700000), fake(0x700000)};
    wave_kv_cache caches[2] = {cache, cache};
    CHECK(wave_round(plan, d, t, 2, caches, srcs, srcs, WAVE_DTYPE_BF16, row, qs, WAVE_DTYPE_BF16, row, os,
                     nullptr, 0.1f, nullptr, 0, st) == WAVE_OK);
    if (prm.cond_len == 0 && prm.query_len == 0) {
      wave_kv_cache c2{fake(0x100000), fake(0x200000), v.num_phys_slots, 2, 64, lpad};
      size_t pw = 0;
      CHECK(qkv_project_workspace(plan, t, &pw) == WAVE_OK);
      CHECK(qkv_project(plan, d, t, &c2, fake(0xa00000), WAVE_X_ROUND, nullptr, fake(0xb00000), fake(0x600000),
                        fake(0xc00000), pw, st) == WAVE_OK);
      CHECK(wave_attn_chain(plan, d, t, &c2, fake(0x600000), WAVE_DTYPE_BF16, 128, fake(0x700000), nullptr, 0.1f,
                            static_cast<float*>(fake(0xe00000)), nullptr, 0, st) == WAVE_OK);
      CHECK(qkv_project(plan, d, t, &c2, fake(0x700000), WAVE_X_ROUND, static_cast<const float*>(fake(0xe00000)),
                        fake(0xb00000), fake(0x600000), fake(0xc00000), pw, st) == WAVE_OK);
      CHECK(chain_store(plan, d, t, 128, fake(0x700000), fake(0xd00000), st) == WAVE_OK);
    }
    // invalid arguments are refused on the host
    CHECK(wave_attn(plan, d, t, &cache, nullptr, WAVE_DTYPE_BF16, row, fake(0x700000), nullptr, 0.1f, nullptr, 0,
                    st) == WAVE_ERR_INVALID_ARG);
    CHECK(std::strlen(wave_last_error()) > 0);
  }
  CHECK(kv_write(plan, d, v.num_rounds, &cache, fake(0x400000), fake(0x500000), 0, row, st) == WAVE_ERR_INVALID_ARG);
  // the memoised tail-balancing choice, queried from several threads at once
  std::vector<std::thread> th;
  for (int k = 0; k < 4; ++k)
    th.emplace_back([plan, &v, k]() {
      for (int t = 0; t < v.num_rounds; ++t) {
        size_t ws = 0;
        CHECK(wave_attn_workspace(plan, t, 12 + k % 2, 128, 256, &ws, nullptr, nullptr) == WAVE_OK);
      }
    });
  for (auto& x : th) x.join();
  wave_plan_destroy(plan);
  return sum;
}

int main() {
  long plans = 0, sum = 0;
  const int Bs[] = {1, 2, 3, 5, 7, 12}, Ks[] = {1, 2, 3, 4, 6}, Hs[] = {-1, 0, 1, 2, 6};
  for (int B : Bs)
    for (int K : Ks)
      for (int pol = 0; pol < 3; ++pol)
        for (int sch = 0; sch < 2; ++sch)
          for (int H : Hs)
            for (int cond : {0, 17}) {
              const int L = (B * 7 + K * 13) % 300 + 1;
              const int qlen = (B + K) % 3 == 0 ? (L + 1) / 2 : 0;
              wave_plan_params prm{B, K, pol, sch, H, L, cond, 0, qlen};
              sum += exercise(prm);
              ++plans;
            }
  // the largest named shapes: 832x480 7-chunk and long-video rounds
  wave_plan_params big{7, 4, WAVE_PROGRESSIVE, WAVE_SCHED_WAVE, -1, 4680, 0, 0, 0};
  sum += exercise(big);
  wave_plan_params lv{28, 4, WAVE_PROGRESSIVE, WAVE_SCHED_WAVE, 6, 4680, 0, 0, 0};
  sum += exercise(lv);
  // rejected parameters leave no plan behind
  wave_plan_t* none = reinterpret_cast<wave_plan_t*>(1);
  wave_plan_params bad{0, 2, 0, 1, -1, 16, 0, 0, 0};
  CHECK(wave_plan(&bad, &none) == WAVE_ERR_INVALID_ARG && none == nullptr);
  std::printf("plans %ld launches %ld checksum %ld\n", plans + 2, stub::launches, sum);
  return 0;
}
