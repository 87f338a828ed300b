// Host page allocator for the paged KV cache and the host half of the
// append step.
//
// PagedAttention keeps a sequence's K/V in fixed-size pages of one shared
// pool: a sequence takes a page when its tail page is full and a finished
// sequence returns its pages to the pool at once (ZimaSpace post, fixed-size
// blocks; blocks released when a request ends; ai-trend study note, "How it
// works", steps two and four). The allocator is a free stack: pages go out
// lowest index first at creation, and the most recently freed page is reused
// first. A per-page flag catches double frees and frees of pages that were
// never taken. Integer work only; no HIP calls.

#include <cstdint>
#include <new>
#include <vector>

#include "pkv_internal.h"

using pkv::clear_error;
using pkv::set_error;

struct pkv_pool {
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<uint8_t> taken;       // per page
};

namespace {

bool valid_page(const pkv_pool* p, int32_t page) {
  return page >= 0 && page < (int32_t)p->taken.size();
}

// Check that `pages` (n of them) are all taken and distinct.
bool check_taken_distinct(pkv_pool* p, const int32_t* pages, int32_t n) {
  bool ok = true;
  int32_t i = 0;
  for (; i < n && ok; ++i) {
    const int32_t pg = pages[i];
    if (!valid_page(p, pg) || p->taken[pg] != 1) {
      ok = false;
      break;
    }
    p->taken[pg] = 2;  // mark seen in this call
  }
  for (int32_t j = 0; j < i; ++j) p->taken[pages[j]] = 1;  // undo the marks
  return ok;
}

}  // namespace

extern "C" {

pkv_status pkv_pool_create(int32_t num_pages, pkv_pool** out_pool) {
  clear_error();
  if (!out_pool) {
    set_error("out_pool is NULL");
    return PKV_ERR_INVALID;
  }
  *out_pool = nullptr;
  if (num_pages <= 0) {
    set_error("num_pages must be > 0 (got %d)", num_pages);
    return PKV_ERR_INVALID;
  }
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) {
    set_error("out of host memory");
    return PKV_ERR_INVALID;
  }
  try {  // no exception crosses the C ABI
    p->taken.assign((size_t)num_pages, 0);
    p->free_stack.resize((size_t)num_pages);
  } catch (const std::bad_alloc&) {
    delete p;
    set_error("out of host memory");
    return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < num_pages; ++i) p->free_stack[(size_t)i] = num_pages - 1 - i;
  *out_pool = p;
  return PKV_OK;
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int32_t pkv_pool_free_pages(const pkv_pool* pool) {
  return pool ? (int32_t)pool->free_stack.size() : -1;
}

pkv_status pkv_pool_alloc(pkv_pool* pool, int32_t n, int32_t* pages) {
  clear_error();
  if (!pool || n < 0 || (n > 0 && !pages)) {
    set_error("pkv_pool_alloc: null pool/pages or n < 0");
    return PKV_ERR_INVALID;
  }
  if ((size_t)n > pool->free_stack.size()) {
    set_error("pool exhausted: %d pages asked, %zu free", n, pool->free_stack.size());
    return PKV_ERR_POOL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pg = pool->free_stack.back();
    pool->free_stack.pop_back();
    pool->taken[pg] = 1;
    pages[i] = pg;
  }
  return PKV_OK;
}

pkv_status pkv_pool_free(pkv_pool* pool, const int32_t* pages, int32_t n) {
  clear_error();
  if (!pool || n < 0 || (n > 0 && !pages)) {
    set_error("pkv_pool_free: null pool/pages or n < 0");
    return PKV_ERR_INVALID;
  }
  if (!check_taken_distinct(pool, pages, n)) {
    set_error("pkv_pool_free: a page is outside the pool, not taken, or listed twice");
    return PKV_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    pool->taken[pages[i]] = 0;
    pool->free_stack.push_back(pages[i]);
  }
  return PKV_OK;
}

pkv_status pkv_append_prepare(pkv_pool* pool, int32_t batch, int32_t block_table_stride,
                              int32_t page_size, const int32_t* seq_lens_host,
                              int32_t* block_table_host, int32_t* pages_taken) {
  clear_error();
  if (pages_taken) *pages_taken = 0;
  if (!pool || batch < 0 || block_table_stride <= 0 || page_size <= 0 ||
      (batch > 0 && (!seq_lens_host || !block_table_host))) {
    set_error("pkv_append_prepare: null argument or bad size");
    return PKV_ERR_INVALID;
  }
  int32_t need = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = seq_lens_host[b];
    if (n < 0 || (int64_t)n >= (int64_t)block_table_stride * page_size) {
      set_error("row %d: position %d outside the table row (%d pages of %d)", b, n,
                block_table_stride, page_size);
      return PKV_ERR_INVALID;
    }
    need += n % page_size == 0;
  }
  if ((size_t)need > pool->free_stack.size()) {
    set_error("pool exhausted: the step needs %d pages, %zu free", need,
              pool->free_stack.size());
    return PKV_ERR_POOL;
  }
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = seq_lens_host[b];
    if (n % page_size != 0) continue;
    int32_t pg = 0;
    (void)pkv_pool_alloc(pool, 1, &pg);  // cannot fail: counted above
    block_table_host[(int64_t)b * block_table_stride + n / page_size] = pg;
  }
  if (pages_taken) *pages_taken = need;
  return PKV_OK;
}

pkv_status pkv_pool_release_row(pkv_pool* pool, int32_t* block_table_row, int32_t seq_len,
                                int32_t page_size) {
  clear_error();
  if (!pool || seq_len < 0 || page_size <= 0 || (seq_len > 0 && !block_table_row)) {
    set_error("pkv_pool_release_row: null argument or bad size");
    return PKV_ERR_INVALID;
  }
  const int32_t n = (seq_len + page_size - 1) / page_size;
  const pkv_status st = pkv_pool_free(pool, block_table_row, n);
  if (st != PKV_OK) return st;
  for (int32_t i = 0; i < n; ++i) block_table_row[i] = -1;
  return PKV_OK;
}

}  // extern "C"
