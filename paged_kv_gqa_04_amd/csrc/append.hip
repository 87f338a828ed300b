// Paged KV append: the step before decode. Every row b of the batch writes
// its new token's K and V (one d-vector per KV head) at its position
// N_b = seq_lens[b]: page block_table[b][N_b / P], slot N_b % P, the same
// logical-to-physical mapping decode reads through (ZimaSpace post: the
// block table maps a request's logical token order to physical blocks; the
// indirection changes placement, not order).
//
// A pure copy, bound by memory latency at these sizes: one lane per 32-bit
// word of a head vector, several (row, KV head) pairs per workgroup, no
// barriers. Positions and page entries are checked so that a bad table entry
// writes nothing instead of writing outside the pools.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kAppendThreads = 256;

struct AppendParams {
  const uint32_t* __restrict__ k_new;  // [B, Hkv, D/2] words
  const uint32_t* __restrict__ v_new;
  uint32_t* __restrict__ k_pool;       // [num_pages, Hkv, P, D/2] words
  uint32_t* __restrict__ v_pool;
  const int32_t* __restrict__ block_table;
  const int32_t* __restrict__ seq_lens;
  int32_t* __restrict__ new_seq_lens;  // may be null
  int64_t num_pages;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t stride;
};

template <int D>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendParams a) {
  constexpr int W = D / 2;                 // 32-bit words per head vector
  constexpr int PAIRS = kAppendThreads / W;  // (row, KV head) pairs per workgroup
  constexpr int P = kPageTokens;
  const int t = threadIdx.x;
  const int pair = blockIdx.x * PAIRS + t / W;
  const int w = t % W;
  if (pair >= a.batch * a.num_kv_heads) return;
  const int b = pair / a.num_kv_heads;
  const int g = pair - b * a.num_kv_heads;
  const int pos = a.seq_lens[b];
  if (a.new_seq_lens && g == 0 && w == 0) a.new_seq_lens[b] = pos + 1;
  if (pos < 0 || pos / P >= a.stride) return;
  const int page = a.block_table[(int64_t)b * a.stride + pos / P];
  if ((uint64_t)(uint32_t)page >= (uint64_t)a.num_pages) return;
  const int64_t dst = (((int64_t)page * a.num_kv_heads + g) * P + pos % P) * W + w;
  const int64_t src = (int64_t)pair * W + w;
  a.k_pool[dst] = a.k_new[src];
  a.v_pool[dst] = a.v_new[src];
}

bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_append(const pkv_shape* s, const void* k_new, const void* v_new,
                                 void* k_pool, void* v_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t* new_seq_lens,
                                 hipStream_t stream) {
  using namespace pkv;
  clear_error();
  if (!s) {
    set_error("shape is NULL");
    return PKV_ERR_INVALID;
  }
  if (s->batch < 0 || s->num_kv_heads <= 0 || s->block_table_stride <= 0 || s->num_pages <= 0) {
    set_error("bad shape: batch %d, Hkv %d, stride %d, num_pages %lld", s->batch,
              s->num_kv_heads, s->block_table_stride, (long long)s->num_pages);
    return PKV_ERR_INVALID;
  }
  if (s->page_size != kPageTokens || (s->head_dim != 64 && s->head_dim != 128) ||
      (s->dtype != PKV_F16 && s->dtype != PKV_BF16)) {
    set_error("unsupported page size %d, head_dim %d or dtype %d", s->page_size, s->head_dim,
              s->dtype);
    return PKV_ERR_UNSUPPORTED;
  }
  if (s->batch == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_table || !seq_lens) {
    set_error("null device pointer");
    return PKV_ERR_INVALID;
  }
  if (!aligned4(k_new) || !aligned4(v_new) || !aligned4(k_pool) || !aligned4(v_pool) ||
      !aligned4(block_table) || !aligned4(seq_lens) || !aligned4(new_seq_lens)) {
    set_error("pkv_append: every pointer must be 4-byte aligned");
    return PKV_ERR_INVALID;
  }
  if (new_seq_lens && (const void*)new_seq_lens == (const void*)seq_lens) {
    set_error("new_seq_lens must not alias seq_lens");
    return PKV_ERR_INVALID;
  }
  AppendParams p{};
  p.k_new = (const uint32_t*)k_new;
  p.v_new = (const uint32_t*)v_new;
  p.k_pool = (uint32_t*)k_pool;
  p.v_pool = (uint32_t*)v_pool;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.new_seq_lens = new_seq_lens;
  p.num_pages = s->num_pages;
  p.batch = s->batch;
  p.num_kv_heads = s->num_kv_heads;
  p.stride = s->block_table_stride;
  const int64_t pairs = (int64_t)s->batch * s->num_kv_heads;
  if (pairs > INT32_MAX / 2) {
    set_error("batch x Hkv too large");
    return PKV_ERR_INVALID;
  }
  const int per = kAppendThreads / (s->head_dim / 2);
  const dim3 grid((unsigned)((pairs + per - 1) / per));
  if (s->head_dim == 128)
    hipLaunchKernelGGL(append_kernel<128>, grid, dim3(kAppendThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(append_kernel<64>, grid, dim3(kAppendThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("append kernel launch: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}
