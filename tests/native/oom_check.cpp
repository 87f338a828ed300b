// Allocation failures in the planner and the page pool come back as a
// status, never as an exception across the C ABI: a global operator new
// that throws once, after a chosen number of allocations, is armed before
// each call, and the failure point is walked over every allocation the
// call makes. It also counts allocations over warmed-up re-plans, which
// must make none. Built with plan.cpp and pool.cpp (no HIP kernels) by
// tests/test_host_sanitize.py. Exits non-zero on a failed check; an
// escaping exception would terminate the program instead.
#include <cstdio>
#include <cstdlib>
#include <new>
#include <vector>

#include "pkv_internal.h"

namespace pkv {
pkv_status query_num_cus(int32_t* num_cus) {
  *num_cus = 256;
  return PKV_OK;
}
void wait_upload(pkv_plan*) {}
void release_device_resources(pkv_plan*) {}
}  // namespace pkv

static long g_left = -1;  // allocations before the one that fails; -1: none fails
static long g_failed = 0;
static long g_count = 0;  // allocations made

void* operator new(std::size_t n) {
  if (g_left == 0) {
    g_left = -1;
    ++g_failed;
    throw std::bad_alloc();
  }
  if (g_left > 0) --g_left;
  ++g_count;
  void* p = std::malloc(n ? n : 1);
  if (!p) throw std::bad_alloc();
  return p;
}
void* operator new[](std::size_t n) { return operator new(n); }
void* operator new(std::size_t n, const std::nothrow_t&) noexcept {
  try {
    return operator new(n);
  } catch (...) {
    return nullptr;
  }
}
void* operator new[](std::size_t n, const std::nothrow_t& t) noexcept { return operator new(n, t); }
void operator delete(void* p) noexcept { std::free(p); }
void operator delete[](void* p) noexcept { std::free(p); }
void operator delete(void* p, std::size_t) noexcept { std::free(p); }
void operator delete[](void* p, std::size_t) noexcept { std::free(p); }

static int failures = 0;
#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

int main() {
  // A ragged batch in every mode: several hundred items, buckets and the
  // longest-first ordering all allocate.
  const std::vector<int32_t> lens = {4096, 700, 0, 19000, 33, 8192, 1, 2500};
  pkv_shape s{};
  s.batch = (int32_t)lens.size();
  s.num_q_heads = 32;
  s.num_kv_heads = 8;
  s.head_dim = 128;
  s.page_size = 16;
  s.block_table_stride = (19000 + 4000) / 16 + 1;  // room for the grown lengths below
  s.num_pages = 1 << 20;
  s.dtype = PKV_BF16;
  long handled = 0;
  for (int mode : {PKV_MODE_AUTO, PKV_MODE_SPLIT, PKV_MODE_WORKQUEUE, PKV_MODE_BUCKETED}) {
    pkv_opts o{};
    o.mode = mode;
    o.chunk_pages = 8;
    o.num_cus = 256;
    for (long k = 0;; ++k) {  // plan creation failing at its k-th allocation
      g_left = k;
      const long before = g_failed;
      pkv_plan* p = nullptr;
      const pkv_status st = pkv_plan_create(&s, lens.data(), &o, &p);
      g_left = -1;
      if (g_failed == before) {  // no allocation failed: the call is done
        CHECK(st == PKV_OK && p != nullptr);
        pkv_plan_destroy(p);
        break;
      }
      ++handled;
      if (st == PKV_OK) {  // the failure was absorbed (an error message lost)
        pkv_plan_destroy(p);
        continue;
      }
      CHECK(p == nullptr);
    }
    pkv_plan* p = nullptr;
    CHECK(pkv_plan_create(&s, lens.data(), &o, &p) == PKV_OK);
    std::vector<int32_t> grown(lens);
    for (int32_t& n : grown) n += 4000;  // a re-plan that needs more items
    for (long k = 0;; ++k) {  // re-planning failing at its k-th allocation
      g_left = k;
      const long before = g_failed;
      const pkv_status st = pkv_plan_update(p, (k % 2) ? grown.data() : lens.data());
      g_left = -1;
      if (g_failed == before) {
        CHECK(st == PKV_OK);
        break;
      }
      ++handled;
      // the plan stays usable: the next re-plan, with memory, succeeds
      CHECK(pkv_plan_update(p, lens.data()) == PKV_OK);
    }
    pkv_plan_destroy(p);
  }
  for (long k = 0;; ++k) {  // pool creation
    g_left = k;
    const long before = g_failed;
    pkv_pool* pool = nullptr;
    const pkv_status st = pkv_pool_create(100000, &pool);
    g_left = -1;
    if (g_failed == before) {
      CHECK(st == PKV_OK && pool != nullptr);
      pkv_pool_destroy(pool);
      break;
    }
    ++handled;
    if (st == PKV_OK) {
      pkv_pool_destroy(pool);
      continue;
    }
    CHECK(pool == nullptr);
  }
  // Re-planning allocates nothing once warmed up: lengths that move inside
  // their pages, and rows gaining or losing pages within the sizes already
  // seen, in every mode.
  for (int mode : {PKV_MODE_AUTO, PKV_MODE_SPLIT, PKV_MODE_WORKQUEUE, PKV_MODE_BUCKETED}) {
    pkv_opts o{};
    o.mode = mode;
    o.chunk_pages = 8;
    o.num_cus = 256;
    pkv_plan* p = nullptr;
    CHECK(pkv_plan_create(&s, lens.data(), &o, &p) == PKV_OK);
    std::vector<int32_t> step(lens);
    for (int warm = 0; warm < 2; ++warm)
      for (int i = 0; i < 64; ++i) {
        for (size_t b = 0; b < step.size(); ++b) step[b] = lens[b] + (int32_t)((i * 7 + b) % 40);
        if (i == 0 && warm == 1) g_count = 0;  // second pass: count
        CHECK(pkv_plan_update(p, step.data()) == PKV_OK);
      }
    if (mode != PKV_MODE_BUCKETED)  // the comparator's buckets are rebuilt from maps
      CHECK(g_count == 0);
    pkv_plan_destroy(p);
  }
  CHECK(handled > 20);
  std::printf("allocation failures handled: %ld\n", handled);
  return failures ? 1 : 0;
}
