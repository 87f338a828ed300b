// Host-side exercise of the planner and the page pool, built together with
// plan.cpp and pool.cpp (no HIP kernels) under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitize.py. It runs the C
// ABI over random batches, every mode, re-plans, queue images, error paths
// and a page-pool serving loop, and checks a few invariants on the way: a
// sanitizer report or a failed check exits non-zero.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "pkv_internal.h"

// The planner's three device hooks (decode.hip in the library); the checks
// pass num_cus, so no device is ever asked.
namespace pkv {
pkv_status query_num_cus(int32_t* num_cus) {
  *num_cus = 256;
  return PKV_OK;
}
void wait_upload(pkv_plan*) {}
void release_device_resources(pkv_plan*) {}
}  // namespace pkv

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static void plan_round(std::mt19937& rng, int mode, int merge) {
  std::uniform_int_distribution<int> bdist(0, 12), ldist(0, 40000), cdist(0, 80), sdist(0, 40);
  const int B = bdist(rng);
  const int heads[][2] = {{8, 2}, {32, 8}, {16, 16}, {64, 8}, {8, 4}};
  const auto& hh = heads[rng() % 5];
  std::vector<int32_t> lens(B);
  int32_t max_pages = 1;
  int64_t pages = 0;
  for (int b = 0; b < B; ++b) {
    lens[b] = (rng() % 4 == 0) ? 0 : ldist(rng);
    max_pages = std::max(max_pages, (lens[b] + 15) / 16);
    pages += (lens[b] + 15) / 16;
  }
  pkv_shape s{};
  s.batch = B;
  s.num_q_heads = hh[0];
  s.num_kv_heads = hh[1];
  s.head_dim = (rng() % 2) ? 128 : 64;
  s.page_size = 16;
  s.block_table_stride = max_pages + (int)(rng() % 3);
  s.num_pages = std::max<int64_t>(pages, 1);
  s.dtype = (rng() % 2) ? PKV_BF16 : PKV_F16;
  pkv_opts o{};
  o.mode = mode;
  o.num_splits = sdist(rng);
  o.chunk_pages = cdist(rng);
  o.num_cus = 256;
  o.queue_seed = (rng() % 2) ? 0u : (uint32_t)rng();
  o.merge = merge;
  pkv_plan* p = nullptr;
  const pkv_status st = pkv_plan_create(&s, lens.data(), &o, &p);
  CHECK(st == PKV_OK);
  if (st != PKV_OK) return;
  pkv_plan_stats stats{};
  CHECK(pkv_plan_stats_get(p, &stats) == PKV_OK);
  pkv_workspace_layout lay{};
  CHECK(pkv_plan_layout_get(p, &lay) == PKV_OK);
  CHECK((size_t)lay.total_bytes == pkv_plan_workspace_bytes(p));
  std::vector<char> img((size_t)stats.upload_bytes + 1);
  CHECK(pkv_plan_queue_get(p, img.data(), (size_t)stats.upload_bytes) == PKV_OK);
  // Every item of a work queue names pages inside its row.
  if (stats.mode == PKV_MODE_WORKQUEUE || stats.mode == PKV_MODE_BUCKETED) {
    const auto* it = reinterpret_cast<const pkv::Item*>(img.data() + lay.items_offset);
    for (int i = 0; i < lay.num_items; ++i) {
      const int b = it[i].bg / s.num_kv_heads;
      CHECK(b >= 0 && b < B);
      if (it[i].slot >= 0) {
        CHECK(it[i].page_begin < it[i].page_end);
        CHECK(it[i].page_end <= (lens[b] + 15) / 16);
        CHECK(it[i].slot < stats.num_slots);
      }
    }
  }
  // Re-plan a few times with new lengths (some past the table: refused).
  for (int r = 0; r < 3; ++r) {
    for (int b = 0; b < B; ++b) lens[b] = std::min(lens[b] + (int)(rng() % 40), s.block_table_stride * 16);
    if (B > 0 && r == 2) lens[0] = s.block_table_stride * 16 + 1;
    const pkv_status u = pkv_plan_update(p, lens.data());
    CHECK(u == PKV_OK || (r == 2 && u == PKV_ERR_INVALID));
    int32_t need = -1;
    CHECK(pkv_plan_upload_needed(p, &need) == PKV_OK && need == 1);
  }
  pkv_plan_destroy(p);
}

static void error_paths() {
  pkv_plan* p = nullptr;
  CHECK(pkv_plan_create(nullptr, nullptr, nullptr, &p) == PKV_ERR_INVALID && p == nullptr);
  pkv_shape s{1, 8, 3, 128, 16, 4, 8, PKV_BF16, 0.0f};
  int32_t len = 10;
  CHECK(pkv_plan_create(&s, &len, nullptr, &p) == PKV_ERR_INVALID);  // 8 % 3 != 0
  s.num_kv_heads = 2;
  s.head_dim = 96;
  pkv_opts o{};
  o.num_cus = 256;
  CHECK(pkv_plan_create(&s, &len, &o, &p) == PKV_ERR_UNSUPPORTED);
  s.head_dim = 128;
  len = 4 * 16 + 1;
  CHECK(pkv_plan_create(&s, &len, &o, &p) == PKV_ERR_INVALID);  // past the table row
  CHECK(std::strlen(pkv_last_error()) > 0);
  CHECK(std::strcmp(pkv_status_string(PKV_ERR_POOL), "PKV_ERR_POOL") == 0);
  int32_t need;
  CHECK(pkv_plan_upload_needed(nullptr, &need) == PKV_ERR_INVALID);
  pkv_plan_destroy(nullptr);
}

static void pool_loop(std::mt19937& rng) {
  const int num_pages = 512, B = 6, stride = 64;
  pkv_pool* pool = nullptr;
  CHECK(pkv_pool_create(num_pages, &pool) == PKV_OK);
  pkv_pool* none = reinterpret_cast<pkv_pool*>(&pool);
  CHECK(pkv_pool_create(0, &none) == PKV_ERR_INVALID && none == nullptr);
  std::vector<int32_t> bt(B * stride, -1), lens(B, 0);
  for (int step = 0; step < 4000; ++step) {
    int32_t taken = 0;
    const pkv_status st = pkv_append_prepare(pool, B, stride, 16, lens.data(), bt.data(), &taken);
    CHECK(st == PKV_OK || st == PKV_ERR_POOL || st == PKV_ERR_INVALID);
    if (st == PKV_OK) {
      for (int b = 0; b < B; ++b) ++lens[b];
    }
    // Finish a row now and then (or when it cannot grow): its pages go back.
    const int b = (int)(rng() % B);
    if (st != PKV_OK || rng() % 97 == 0 || lens[b] >= stride * 16) {
      CHECK(pkv_pool_release_row(pool, bt.data() + b * stride, lens[b], 16) == PKV_OK);
      lens[b] = 0;
    }
    int used = 0;
    for (int r = 0; r < B; ++r) used += (lens[r] + 15) / 16;
    CHECK(pkv_pool_free_pages(pool) == num_pages - used);
  }
  // Double frees and foreign pages are refused as a whole.
  int32_t pages[3];
  CHECK(pkv_pool_alloc(pool, 3, pages) == PKV_OK);
  int32_t twice[2] = {pages[0], pages[0]};
  CHECK(pkv_pool_free(pool, twice, 2) == PKV_ERR_INVALID);
  int32_t foreign[1] = {num_pages + 5};
  CHECK(pkv_pool_free(pool, foreign, 1) == PKV_ERR_INVALID);
  CHECK(pkv_pool_free(pool, pages, 3) == PKV_OK);
  pkv_pool_destroy(pool);
}

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 300;
  std::mt19937 rng(20260623u);
  for (int i = 0; i < rounds; ++i)
    for (int mode = PKV_MODE_AUTO; mode <= PKV_MODE_BUCKETED; ++mode)
      plan_round(rng, mode, i % 2 ? PKV_MERGE_FUSED : PKV_MERGE_KERNEL);
  error_paths();
  pool_loop(rng);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host checks passed (%d planning rounds per mode)\n", rounds);
  return 0;
}
