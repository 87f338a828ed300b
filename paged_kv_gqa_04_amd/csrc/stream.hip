// Plain streaming read, a measurement aid: reads two device buffers once,
// 16 bytes per lane per load, nontemporal, with no dependent work. Timed on
// the decode's own K/V bytes, it gives the HBM ceiling a one-pass read of
// that many bytes reaches on this device (the decode moves every K/V byte
// once: ai-trend study note, "Why it was needed"), so the decode's time can
// be set against what is reachable rather than against the data-sheet peak.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;  // loads of each buffer in flight per lane per round

__global__ __launch_bounds__(kStreamThreads) void stream_kernel(const u32x4* __restrict__ a,
                                                                const u32x4* __restrict__ b,
                                                                int64_t n16,
                                                                uint32_t* __restrict__ sink) {
  uint32_t x = 0;
  const int64_t lanes = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (kStreamUnroll - 1) * lanes < n16; i += kStreamUnroll * lanes) {
    u32x4 u[kStreamUnroll], v[kStreamUnroll];
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) {
      u[k] = __builtin_nontemporal_load(a + i + k * lanes);
      v[k] = __builtin_nontemporal_load(b + i + k * lanes);
    }
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) x ^= u[k].x ^ u[k].y ^ u[k].z ^ u[k].w ^ v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n16; i += lanes) {
    const u32x4 u = __builtin_nontemporal_load(a + i);
    const u32x4 v = __builtin_nontemporal_load(b + i);
    x ^= u.x ^ u.y ^ u.z ^ u.w ^ v.x ^ v.y ^ v.z ^ v.w;
  }
  // Keeps the loads live; the data never make this true in practice, and
  // the write goes to the caller's 4-byte sink either way.
  if (x == 0x9e3779b9u) *sink = x;
}

// ---------------------------------------------------------------- paged read
//
// A second measurement aid: every K and V tile one decode step reads (pages
// [page_begin, page_end) of each work item, through the block table, as the
// PersistentKV explainer's Methodology 1 gathers them), with the partial
// kernel's work split (same grid and items; wave w of a workgroup takes the
// range's pages w, w + W, ...) and its kind of load path (nontemporal
// 16-byte direct-to-LDS loads into a two-slot ring per wave, table entries
// staged in LDS), read back from LDS and folded into one check word. No q,
// no softmax, no state, no merge: timed beside the decode it shows what the
// paged gather alone costs and what the decode adds to it.

struct PagedReadParams {
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const Item* items;
  int64_t num_pages;
  int32_t mode;
  int32_t num_splits;
  int32_t split_chunk;
  int32_t num_kv_heads;
  int32_t stride;
  uint32_t* sink;
};

constexpr int kReadThreads = kWavesPerGroup * 64;
constexpr int kReadChunk = 512;  // table entries staged in LDS at a time
constexpr uint32_t kReadMark = 0x9e3779b9u;

#define PKV_GPTR(p) ((__attribute__((address_space(1))) void*)(p))
#define PKV_LPTR(p) ((__attribute__((address_space(3))) void*)(p))

// Wait until at most VMS vector-memory loads are outstanding (the slot's own
// loads have landed), read this lane's 16-byte pieces of the slot (1 KiB
// apart), and wait for them, all in one block.
#define PKV_PR_READ8(VMS) \
  asm volatile("s_waitcnt vmcnt(" VMS ")\n" \
               "ds_read_b128 %0, %8\n" \
               "ds_read_b128 %1, %8 offset:1024\n" \
               "ds_read_b128 %2, %8 offset:2048\n" \
               "ds_read_b128 %3, %8 offset:3072\n" \
               "ds_read_b128 %4, %8 offset:4096\n" \
               "ds_read_b128 %5, %8 offset:5120\n" \
               "ds_read_b128 %6, %8 offset:6144\n" \
               "ds_read_b128 %7, %8 offset:7168\n" \
               "s_waitcnt lgkmcnt(0)" \
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), \
                 "=&v"(r[6]), "=&v"(r[7]) \
               : "v"(addr) \
               : "memory")
#define PKV_PR_READ4(VMS) \
  asm volatile("s_waitcnt vmcnt(" VMS ")\n" \
               "ds_read_b128 %0, %4\n" \
               "ds_read_b128 %1, %4 offset:1024\n" \
               "ds_read_b128 %2, %4 offset:2048\n" \
               "ds_read_b128 %3, %4 offset:3072\n" \
               "s_waitcnt lgkmcnt(0)" \
               : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]) \
               : "v"(addr) \
               : "memory")

template <int D>
__global__ __launch_bounds__(kReadThreads, 2) void paged_read_kernel(PagedReadParams a) {
  constexpr int P = kPageTokens;
  constexpr int W = kWavesPerGroup;
  constexpr int TILE = P * D;            // elements of one (page, KV head) tile
  constexpr int NI = TILE * 2 / 1024;    // 1 KiB loads per tile
  constexpr int LPP = 2 * NI;            // loads (and 16-byte pieces per lane) per page
  constexpr int SLOT = LPP * 256;        // words per ring slot
  static_assert(LPP == 4 || LPP == 8, "head_dim 64 or 128");
  __shared__ __attribute__((aligned(16))) uint32_t s_r0[W * SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t s_r1[W * SLOT];
  __shared__ int32_t s_bt[kReadChunk];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads;

  // The work item, found as the partial kernel finds it.
  int b, g, pb, pe;
  if (a.mode == PKV_MODE_WORKQUEUE) {
    const Item it = a.items[blockIdx.x];
    b = it.b;
    g = it.g;
    pb = it.page_begin;
    pe = it.page_end;
  } else if (a.mode == PKV_MODE_SPLIT) {
    b = blockIdx.z;
    g = blockIdx.y;
    const int pages = (a.seq_lens[b] + P - 1) / P;
    const int chunk = a.split_chunk > 0 ? a.split_chunk
                                        : (pages > 0 ? (pages + a.num_splits - 1) / a.num_splits : 1);
    pb = blockIdx.x * chunk;
    pe = pb + chunk;
  } else {
    b = blockIdx.x / Hkv;
    g = blockIdx.x - b * Hkv;
    pb = 0;
    pe = 0x7fffffff;
  }
  const int n = a.seq_lens[b];
  pe = min(pe, min((n + P - 1) / P, a.stride));
  const int32_t* bt_row = a.block_table + (int64_t)b * a.stride;

  uint32_t x = 0;
  for (int cb = pb; cb < pe; cb += kReadChunk) {
    const int span = min(pe - cb, kReadChunk);
    __syncthreads();  // every wave is done with the previous chunk's entries
    for (int i = threadIdx.x; i < span; i += kReadThreads) s_bt[i] = bt_row[cb + i];
    __syncthreads();
    const int cnt = span > wave ? (span - wave + W - 1) / W : 0;
    // Page k of this wave's share into slot sl. An entry outside the pool
    // reads page 0 instead, as the partial kernel does (it then uses no
    // token of it).
    auto issue = [&](int sl, int k) {
      int phys = __builtin_amdgcn_readfirstlane(s_bt[wave + W * k]);
      phys = (uint64_t)(uint32_t)phys < (uint64_t)a.num_pages ? phys : 0;
      const int64_t tile = ((int64_t)phys * Hkv + g) * TILE + lane * 8;
      uint32_t* dst = (sl == 0 ? s_r0 : s_r1) + wave * SLOT;
#pragma unroll
      for (int j = 0; j < NI; ++j)
        __builtin_amdgcn_global_load_lds(PKV_GPTR(a.k_pool + tile + j * 512), PKV_LPTR(dst + j * 256),
                                         16, 0, 2);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        __builtin_amdgcn_global_load_lds(PKV_GPTR(a.v_pool + tile + j * 512),
                                         PKV_LPTR(dst + (NI + j) * 256), 16, 0, 2);
    };
    if (cnt > 0) issue(0, 0);
    if (cnt > 1) issue(1, 1);
    for (int k = 0; k < cnt; ++k) {
      const int sl = k & 1;
      const uint32_t addr =
          (uint32_t)(uintptr_t)PKV_LPTR((sl == 0 ? s_r0 : s_r1) + wave * SLOT) + lane * 16;
      u32x4 r[LPP];
      if constexpr (LPP == 8) {
        if (k + 1 < cnt) PKV_PR_READ8("8");
        else PKV_PR_READ8("0");
      } else {
        if (k + 1 < cnt) PKV_PR_READ4("4");
        else PKV_PR_READ4("0");
      }
#pragma unroll
      for (int j = 0; j < LPP; ++j) x ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
      if (k + 2 < cnt) issue(sl, k + 2);  // the slot just read
    }
  }
  // As in the streaming read: only a lane whose data folds to the mark writes.
  if (x == kReadMark) *a.sink = x;
}

}  // namespace
}  // namespace pkv

extern "C" pkv_status pkv_paged_read(const pkv_plan* plan, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* seq_lens, void* sink,
                                     hipStream_t stream) {
  pkv::clear_error();
  if (!plan || !k_pool || !v_pool || !block_table || !seq_lens || !sink ||
      ((uintptr_t)k_pool | (uintptr_t)v_pool) % 16 != 0 ||
      ((uintptr_t)block_table | (uintptr_t)seq_lens | (uintptr_t)sink) % 4 != 0) {
    pkv::set_error("paged read: null or misaligned pointer");
    return PKV_ERR_INVALID;
  }
  if (plan->mode == PKV_MODE_BUCKETED) {
    pkv::set_error("paged read: the bucketed comparator's launches are not mirrored");
    return PKV_ERR_UNSUPPORTED;
  }
  const int D = plan->shape.head_dim;
  if (D != 64 && D != 128) {
    pkv::set_error("paged read: no kernel for head_dim %d", D);
    return PKV_ERR_UNSUPPORTED;
  }
  if (plan->mode == PKV_MODE_WORKQUEUE && (!plan->uploaded || !plan->workspace)) {
    pkv::set_error("paged read: a work-queue plan must be uploaded (pkv_plan_upload) first");
    return PKV_ERR_STATE;
  }
  if (plan->grid == 0) return PKV_OK;
  pkv::PagedReadParams a{};
  a.k_pool = (const uint16_t*)k_pool;
  a.v_pool = (const uint16_t*)v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.items = plan->mode == PKV_MODE_WORKQUEUE
                ? (const pkv::Item*)((const char*)plan->workspace + plan->layout.items_offset)
                : nullptr;
  a.num_pages = plan->shape.num_pages;
  a.mode = plan->mode;
  a.num_splits = plan->num_splits;
  a.split_chunk = plan->split_chunk;
  a.num_kv_heads = plan->shape.num_kv_heads;
  a.stride = plan->shape.block_table_stride;
  a.sink = (uint32_t*)sink;
  const dim3 grid = plan->mode == PKV_MODE_SPLIT
                        ? dim3(plan->num_splits, plan->shape.num_kv_heads, plan->shape.batch)
                        : dim3(plan->grid);
  if (D == 128)
    hipLaunchKernelGGL(pkv::paged_read_kernel<128>, grid, dim3(pkv::kReadThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(pkv::paged_read_kernel<64>, grid, dim3(pkv::kReadThreads), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    pkv::set_error("paged read launch: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}

extern "C" pkv_status pkv_stream_read(const void* a, const void* b, int64_t bytes_each,
                                      int32_t grid, void* sink, hipStream_t stream) {
  pkv::clear_error();
  if (!a || !b || !sink || bytes_each < 0 || grid <= 0 || bytes_each % 16 != 0 ||
      ((uintptr_t)a | (uintptr_t)b) % 16 != 0 || (uintptr_t)sink % 4 != 0) {
    pkv::set_error("stream read: null or misaligned buffer, size not a multiple of 16, or grid <= 0");
    return PKV_ERR_INVALID;
  }
  hipLaunchKernelGGL(pkv::stream_kernel, dim3(grid), dim3(pkv::kStreamThreads), 0, stream,
                     (const pkv::u32x4*)a, (const pkv::u32x4*)b, (int64_t)(bytes_each / 16),
                     (uint32_t*)sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    pkv::set_error("stream read launch: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  return PKV_OK;
}
