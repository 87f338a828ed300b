// Paged GQA decode kernels for gfx950 (MI355X) and their dispatch.
//
// Partial kernel: one workgroup per (sequence b, KV head g, page range).
// Reads the range's K/V pages straight from the pools through the block
// table (PersistentKV explainer, Technical summary > Methodology 1: the
// engine runs on the paged layout without repacking), computes the G x 16
// logits of each page, keeps an online-softmax state and accumulates P.V in
// fp32. The state of the range is written as a partial (m, l, acc) for the
// merge kernel, or, when the range is the whole row, normalised into out.
//
// Merge: combines a (sequence, KV head) row's partial states for its G
// query heads in split-index order: M = max m_s, weights exp(m_s - M),
// out = sum w_s acc_s / sum w_s l_s (Methodology 1, the merge kernel that
// combines the states exactly). By default the last workgroup of the row to
// finish its range runs it at the end of the partial kernel (one launch per
// step); the separate merge kernel (one workgroup per row) runs the same
// code.
//
// The step is HBM-bound: every K/V byte is read once and each element feeds
// only G multiply-adds (ai-trend study note, "Why it was needed": decode reads
// the whole KV cache per token and is bandwidth bound).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
#define GPTR(p) ((__attribute__((address_space(1))) void*)(p))
#define LPTR(p) ((__attribute__((address_space(3))) void*)(p))
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescaling slack (log2 units): the running reference maximum is only
// raised when a logit exceeds it by more than this, so exponentials stay
// below 2^8 and the accumulator is rescaled rarely.
constexpr float kTau = 8.0f;
// Initial reference maximum: finite, so exp2(x - ref) of a masked logit
// (-inf) is 0 and never NaN; far below any real logit.
constexpr float kNoMax = -1.0e30f;
constexpr int kThreads = kWavesPerGroup * 64;
// K/V ring slots (pages in flight + 1) per wave of the partial kernel.
#ifndef PKV_RING_SLOTS
#define PKV_RING_SLOTS 2
#endif
constexpr int kRingSlots = PKV_RING_SLOTS;
// Block-table entries staged in LDS at a time by the partial kernel.
constexpr int kBtChunk = 512;
static_assert(kBtChunk % kThreads == 0, "table staging: whole rounds of the workgroup");
// s_waitcnt immediate for gfx9: vmcnt(n) (6 bits: [3:0] and [15:14]) with
// expcnt(7) and lgkmcnt(15), i.e. wait on vector-memory loads only.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitVmcnt0 = waitcnt_vm(0);
// Cache-policy operand of the direct-to-LDS load builtin: nontemporal.
constexpr int kLoadNontemporal = 2;

// ---------------------------------------------------------------- helpers

template <int DT>
__device__ __forceinline__ void unpack2(uint32_t u, float& lo, float& hi) {
  if constexpr (DT == PKV_BF16) {
    lo = __uint_as_float(u << 16);
    hi = __uint_as_float(u & 0xffff0000u);
  } else {
    f16x2_t h = __builtin_bit_cast(f16x2_t, u);
    lo = (float)h[0];
    hi = (float)h[1];
  }
}

// fp32 -> storage, round to nearest even.
template <int DT>
__device__ __forceinline__ uint16_t pack1(float f) {
  if constexpr (DT == PKV_BF16) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Partial states cross workgroups, and XCDs with separate L2 caches, when
// the last workgroup of a row merges them inside the partial kernel; they
// move with device-scope (agent) stores and loads, which bypass a stale L2.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 V#: stride 0, 32-bit
// data format); a load past the end returns zeros.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCpolSc1 = 16;  // cache-policy operand: device (agent) scope
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)bytes,
                                           kRawBufferWord3);
}
// 16 bytes of a partial state at byte offset `off`, device-scope store.
__device__ __forceinline__ void st_agent16(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  const u32x4 u = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                   __float_as_uint(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, (int)off, 0, kCpolSc1);
}
// 16 bytes of a partial state at byte offset `off`, device-scope load.
__device__ __forceinline__ float4 ld_agent16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCpolSc1);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                     __uint_as_float(v.w));
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Cross-row exchanges (gfx950): with both operands equal, permlane16_swap
// returns each lane's value and that of the lane 16 away in the paired row;
// permlane32_swap likewise across the two halves of the wave.
__device__ __forceinline__ float swap16_add(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float swap16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum over lane-index bits FROM..5 (the other bits fixed), result in every
// lane: DPP quad permutes for bits 0-1, row rotations by 4 and 8 for bits
// 2-3, row and half-wave swaps for bits 4-5. No LDS round trips.
template <int FROM>
__device__ __forceinline__ float sum_lanes_from(float v) {
  if constexpr (FROM <= 0) v += dpp_mov<0xB1>(v);
  if constexpr (FROM <= 1) v += dpp_mov<0x4E>(v);
  if constexpr (FROM <= 2) v += dpp_mov<0x124>(v);
  if constexpr (FROM <= 3) v += dpp_mov<0x128>(v);
  if constexpr (FROM <= 4) v = swap16_add(v);
  return swap32_add(v);
}

// Maximum over lane-index bits FROM..5, same exchanges as sum_lanes_from.
template <int FROM>
__device__ __forceinline__ float max_lanes_from(float v) {
  if constexpr (FROM <= 0) v = fmaxf(v, dpp_mov<0xB1>(v));
  if constexpr (FROM <= 1) v = fmaxf(v, dpp_mov<0x4E>(v));
  if constexpr (FROM <= 2) v = fmaxf(v, dpp_mov<0x124>(v));
  if constexpr (FROM <= 3) v = fmaxf(v, dpp_mov<0x128>(v));
  if constexpr (FROM <= 4) v = swap16_max(v);
  return swap32_max(v);
}

// 16x16x32 matrix-core product on 8-element bf16 / fp16 operands held as
// raw 16-byte vectors, fp32 accumulate.
template <int DT>
__device__ __forceinline__ floatx4 mfma_16x16x32(u32x4 a, u32x4 b, floatx4 c) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to one register of two storage values (round to nearest
// even; lo in bits 0-15).
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const float2_t f = {lo, hi};
  if constexpr (DT == PKV_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
  }
}

// Workgroup barrier over the LDS data written with ds_write (the staged
// table): waits for this wave's LDS instructions, not for its K/V loads in
// flight. A __syncthreads() would drain those too (the direct-to-LDS loads
// count as LDS writes for a fence), and so would an LDS-only fence. The ring
// slots those loads fill are each wave's own and are read only after an
// explicit vmcnt wait. The memory clobber keeps the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Read one ring slot back from LDS: wait until at most VM vector-memory
// loads are outstanding (the slot's own direct-to-LDS loads have landed),
// then read this lane's K pieces (16 bytes at each of the per-lane LDS byte
// addresses ka[]) and the V^T operand of each 16-column tile T with one
// transposing read from va[T] (ds_read_b64_tr_b16: in each 16-lane group,
// lane i receives 16-bit element i % 4 of the 8 bytes addressed by group
// lanes i / 4 + 4 j, j = 0..3; the mapping was read back on the GPU), and
// wait for them. At most 12 LDS reads are in flight (the counter holds 15).
#define PKV_READ8(VMS) \
  asm volatile("s_waitcnt vmcnt(" VMS ")\n" \
               "ds_read_b128 %0, %[k0]\n" \
               "ds_read_b128 %1, %[k1]\n" \
               "ds_read_b128 %2, %[k2]\n" \
               "ds_read_b128 %3, %[k3]\n" \
               "ds_read_b64_tr_b16 %4, %[v0]\n" \
               "ds_read_b64_tr_b16 %5, %[v1]\n" \
               "ds_read_b64_tr_b16 %6, %[v2]\n" \
               "ds_read_b64_tr_b16 %7, %[v3]\n" \
               "ds_read_b64_tr_b16 %8, %[v4]\n" \
               "ds_read_b64_tr_b16 %9, %[v5]\n" \
               "ds_read_b64_tr_b16 %10, %[v6]\n" \
               "ds_read_b64_tr_b16 %11, %[v7]\n" \
               "s_waitcnt lgkmcnt(0)" \
               : "=&v"(kk[0]), "=&v"(kk[1]), "=&v"(kk[2]), "=&v"(kk[3]), "=&v"(vraw[0]), \
                 "=&v"(vraw[1]), "=&v"(vraw[2]), "=&v"(vraw[3]), "=&v"(vraw[4]), \
                 "=&v"(vraw[5]), "=&v"(vraw[6]), "=&v"(vraw[7]) \
               : [k0] "v"(ka[0]), [k1] "v"(ka[1]), [k2] "v"(ka[2]), [k3] "v"(ka[3]), \
                 [v0] "v"(va[0]), [v1] "v"(va[1]), [v2] "v"(va[2]), [v3] "v"(va[3]), \
                 [v4] "v"(va[4]), [v5] "v"(va[5]), [v6] "v"(va[6]), [v7] "v"(va[7]) \
               : "memory")
#define PKV_READ4(VMS) \
  asm volatile("s_waitcnt vmcnt(" VMS ")\n" \
               "ds_read_b128 %0, %[k0]\n" \
               "ds_read_b128 %1, %[k1]\n" \
               "ds_read_b64_tr_b16 %2, %[v0]\n" \
               "ds_read_b64_tr_b16 %3, %[v1]\n" \
               "ds_read_b64_tr_b16 %4, %[v2]\n" \
               "ds_read_b64_tr_b16 %5, %[v3]\n" \
               "s_waitcnt lgkmcnt(0)" \
               : "=&v"(kk[0]), "=&v"(kk[1]), "=&v"(vraw[0]), "=&v"(vraw[1]), \
                 "=&v"(vraw[2]), "=&v"(vraw[3]) \
               : [k0] "v"(ka[0]), [k1] "v"(ka[1]), [v0] "v"(va[0]), [v1] "v"(va[1]), \
                 [v2] "v"(va[2]), [v3] "v"(va[3]) \
               : "memory")

template <int LPP, int VM, typename KArr, typename VArr>
__device__ __forceinline__ void read_slot(const uint32_t* ka, const uint32_t* va, KArr& k, VArr& vt) {
  u32x4* kk = &k[0];
  constexpr int NT = LPP == 8 ? 8 : 4;
  uint64_t vraw[NT];
  if constexpr (LPP == 8) {
    if constexpr (VM == 0) PKV_READ8("0");
    else if constexpr (VM == 8) PKV_READ8("8");
    else if constexpr (VM == 16) PKV_READ8("16");
    else if constexpr (VM == 24) PKV_READ8("24");
    else static_assert(VM == 8, "ring depth");
  } else {
    static_assert(LPP == 4, "loads per page");
    if constexpr (VM == 0) PKV_READ4("0");
    else if constexpr (VM == 4) PKV_READ4("4");
    else if constexpr (VM == 8) PKV_READ4("8");
    else if constexpr (VM == 12) PKV_READ4("12");
    else static_assert(VM == 4, "ring depth");
  }
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    vt[T][0] = (uint32_t)vraw[T];
    vt[T][1] = (uint32_t)(vraw[T] >> 32);
  }
}


// ------------------------------------------------------------- parameters

struct PartialParams {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k_pool;
  const uint16_t* __restrict__ v_pool;
  const int32_t* __restrict__ block_table;
  const int32_t* __restrict__ seq_lens;
  uint16_t* __restrict__ out;
  const Item* __restrict__ items;
  float* __restrict__ ws_m;
  float* __restrict__ ws_l;
  float* __restrict__ ws_acc;
  int32_t* __restrict__ counters;    // one per (sequence, KV head), PKV_COUNTER_STRIDE bytes apart
  const SeqMeta* __restrict__ meta;  // work queue: (slot_base, S_b) per row
  int64_t num_pages;
  int32_t stride;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t mode;
  int32_t num_splits;
  int32_t split_chunk;  // SPLIT: range size shared by every row (0: per row, from seq_lens)
  int32_t fused;     // last-arriving workgroup of a row merges its states
  float scale_log2;  // sm_scale * log2(e)
  // Folded append (null k_new: none): row b's new token ([B, Hkv, d] each)
  // goes to position seq_lens[b], and the step attends over seq_lens[b] + 1.
  const uint16_t* __restrict__ k_new;
  const uint16_t* __restrict__ v_new;
  int32_t* __restrict__ new_seq_lens;  // seq_lens[b] + 1 (may be null)
};

struct MergeParams {
  const float* __restrict__ ws_m;
  const float* __restrict__ ws_l;
  const float* __restrict__ ws_acc;
  const SeqMeta* __restrict__ meta;
  const int32_t* __restrict__ rows;  // sequences of the launch (null: 0 .. B-1)
  uint16_t* __restrict__ out;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t group;
  int32_t mode;
  int32_t num_splits;
};

// ------------------------------------------------------------ state merge
//
// Merge the `count` partial states of one (sequence, KV head) row, slots
// base .. base+count-1, into the row's G x D outputs, in the two passes of
// the definition (PersistentKV explainer, Methodology 1: the merge kernel
// combines the split states exactly): per head M = max_s m_s, weights
// w_s = 2^(m_s - M) (0 for a neutral state), L = sum_s w_s l_s, then
// out = sum_s w_s acc_s / L (0 when L = 0: an empty row). Run by a whole
// workgroup:
//  * acc: thread t owns float4 column t % NC of the G x D state and the
//    slots t / NC, t / NC + NSUB, ...; its first batch of loads is issued
//    right behind the m / l loads, so that all share one memory latency.
//  * m / l: every wave reads all of them itself (lane = slot * G + head,
//    K lane rounds), reduces each head with fixed DPP / permlane trees and
//    writes its weights to its own LDS area: no cross-wave barrier.
//  * the NSUB column-owner subsets are added in subset order at the end.
// Every reduction order is fixed by the slot indices alone, never by
// timing, so the fused tail and the separate merge kernel (both call this)
// produce the same bits. All state loads are device-scope: the states come
// from workgroups on other XCDs.
constexpr int kMergeBatch = 16;  // acc loads in flight per thread

template <int DT, int G, int D>
__device__ __forceinline__ void merge_row(const float* __restrict__ ws_m,
                                          const float* __restrict__ ws_l,
                                          const float* __restrict__ ws_acc, int base, int count,
                                          uint16_t* __restrict__ out_row) {
  constexpr int NC = G * D / 4;          // float4 columns of one state
  constexpr int NSUB = kThreads / NC;    // slot subsets accumulated side by side
  constexpr int SPW = 64 / G;            // slots per lane round
  constexpr int K = 4;                   // lane rounds per weight round
  constexpr int TPH = K * SPW;           // slots per weight round
  constexpr int PER = kMergeBatch < TPH / NSUB ? kMergeBatch : TPH / NSUB;
  constexpr int SB = PER * NSUB;         // slots per acc batch
  constexpr int W = kWavesPerGroup;
  constexpr int LOG2G = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;
  static_assert(NSUB >= 1 && NSUB * NC == kThreads, "layout");
  static_assert(SB <= TPH && TPH % SB == 0 && (1 << LOG2G) == G, "batches tile a round");
  __shared__ float s_w[W][K * 64];  // per wave: weights of one round, [slot][head]
  __shared__ float4 s_A[NSUB > 1 ? NSUB : 1][NC];
  base = __builtin_amdgcn_readfirstlane(base);  // uniform: one buffer resource
  count = __builtin_amdgcn_readfirstlane(count);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = t % NC, sub = t / NC;
  const int hc = (c * 4) / D;  // head of this thread's acc column
  const int hm = lane % G;     // head of this lane's m / l
  const int sl = lane / G;     // slot (within a lane round) of this lane's m / l

  // The row's acc states as one buffer: slots past `count` read as zeros.
  const __amdgpu_buffer_rsrc_t racc =
      raw_rsrc(ws_acc + (int64_t)base * (G * D), (uint32_t)count * (G * D * 4));
  float4 av[PER];
  auto load_acc = [&](int s0) {
#pragma unroll
    for (int j = 0; j < PER; ++j)
      av[j] = ld_agent16(racc, (uint32_t)((s0 + sub + j * NSUB) * (G * D) + c * 4) * 4u);
  };

  float mk[K], lk[K];
  auto load_m = [&](int r0) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int s = r0 + k * SPW + sl;
      mk[k] = s < count ? ld_agent(ws_m + (int64_t)(base + s) * G + hm) : -INFINITY;
    }
  };
  auto load_l = [&](int r0) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int s = r0 + k * SPW + sl;
      lk[k] = s < count ? ld_agent(ws_l + (int64_t)(base + s) * G + hm) : 0.0f;
    }
  };
  // The first round's m / l go out first and the first acc batch right
  // after: loads return in order, so pass 1 runs while the acc batch is
  // still arriving.
  load_m(0);
  load_l(0);
  load_acc(0);

  // Pass 1: running (max, rescaled sum) per lane, then per head.
  float Mt = -INFINITY, Lt = 0.0f;
  for (int r0 = 0; r0 < count; r0 += TPH) {
    if (r0 > 0) {
      load_m(r0);
      load_l(r0);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const float mn = fmaxf(Mt, mk[k]);
      Lt = (Mt == -INFINITY ? 0.0f : Lt * fast_exp2(Mt - mn)) +
           (mk[k] == -INFINITY ? 0.0f : lk[k] * fast_exp2(mk[k] - mn));
      Mt = mn;
    }
  }
  const float M = max_lanes_from<LOG2G>(Mt);
  const float L = sum_lanes_from<LOG2G>(Mt == -INFINITY ? 0.0f : Lt * fast_exp2(Mt - M));
  const float Lc = __shfl(L, hc);  // lane hc holds head hc

  // Pass 2: weights once per (slot, head), then the weighted acc sums.
  float* sw = s_w[wave];
  float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int r0 = 0; r0 < count; r0 += TPH) {
    if (count > TPH) load_m(r0);  // else pass 1 left this round's m in mk
#pragma unroll
    for (int k = 0; k < K; ++k) sw[k * 64 + lane] = mk[k] == -INFINITY ? 0.0f : fast_exp2(mk[k] - M);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int r1 = min(count, r0 + TPH);
    for (int b0 = r0; b0 < r1; b0 += SB) {
      if (b0 > 0) load_acc(b0);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const float w = sw[(b0 - r0 + sub + j * NSUB) * G + hc];
        A.x = fmaf(w, av[j].x, A.x);
        A.y = fmaf(w, av[j].y, A.y);
        A.z = fmaf(w, av[j].z, A.z);
        A.w = fmaf(w, av[j].w, A.w);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // this round's weights are read
  }
  if constexpr (NSUB > 1) {
    s_A[sub][c] = A;
    __syncthreads();
    if (sub == 0) {
#pragma unroll
      for (int u = 1; u < NSUB; ++u) {
        const float4 o = s_A[u][c];
        A.x += o.x;
        A.y += o.y;
        A.z += o.z;
        A.w += o.w;
      }
    }
  }
  if (sub == 0) {
    const float inv = Lc > 0.0f ? 1.0f / Lc : 0.0f;
    const uint32_t lo = pack1<DT>(A.x * inv) | ((uint32_t)pack1<DT>(A.y * inv) << 16);
    const uint32_t hi = pack1<DT>(A.z * inv) | ((uint32_t)pack1<DT>(A.w * inv) << 16);
    *(uint2*)(out_row + c * 4) = make_uint2(lo, hi);
  }
}

// --------------------------------------------------- fused merge (tail)
//
// Called by every workgroup of (sequence b, KV head g) after it has written
// its partial state. A per-row counter counts arrivals; the workgroup that
// arrives last merges all of the row's states in split-index order (so the
// result does not depend on which one it is) and resets the counter for the
// next step. No workgroup ever waits for another.
//
// Visibility without cache-wide fences: every state store is device-scope
// (written through to the point of coherence shared by all XCDs) and each
// wave waits for its own stores to complete (vmcnt 0) before the barrier
// that precedes the arrival increment; the last arriver reads the states
// with device-scope loads issued after it has seen every other arrival. A
// full agent-scope fence would instead write back and invalidate the whole
// L2 of the XCD, stalling every other workgroup there.
template <int DT, int G, int D>
__device__ void finish_group(const PartialParams& a, int b, int g, SeqMeta row) {
  __shared__ int s_last;
  const int bg = b * a.num_kv_heads + g;
  const int base = row.slot_base, count = row.splits;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's state stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    int32_t* const cnt = a.counters + (int64_t)bg * (PKV_COUNTER_STRIDE / 4);
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == count - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  lds_barrier();  // s_last is published (no memory access of this workgroup is pending)
  if (!s_last) return;
  merge_row<DT, G, D>(a.ws_m, a.ws_l, a.ws_acc, base, count,
                      a.out + ((int64_t)b * a.num_q_heads + g * G) * D);
}

// ---------------------------------------------------------- partial kernel
//
// One workgroup (W waves) per (sequence b, KV head g, page range). Wave w
// takes pages w, w+W, ... of the range. Per 16-token page of one KV head
// (a 16 x D tile, contiguous in the pool):
//  * K and V arrive in the wave's LDS ring by direct-to-LDS loads, each in
//    1 KiB contiguous runs. K rows are stored with their 16-byte chunks
//    rotated by the token index (chunk c of token t at slot position
//    (c + t) mod (2D/16)): every lane still fetches whole row runs, and the
//    MFMA operand reads below touch distinct LDS banks; V rows are rotated
//    by two chunks per 256-byte row step for the same reason.
//  * Logits: S^T = K Q^T on the matrix cores, v_mfma_f32_16x16x32 over d in
//    D/32 steps. A = K (16 rows: the page's tokens), B = Q^T (16 columns:
//    the G heads of the group, padded by repeats). The 16x16 result gives
//    lane l head l % 16 and tokens 4 (l / 16) .. +3.
//  * Softmax: one reference maximum per head, shared by the four lanes of
//    the head, raised only when a logit exceeds it by kTau (then l and acc
//    are rescaled). Masked tokens and padding heads get -inf by select.
//  * P.V on the matrix cores: O^T = V^T P^T, one v_mfma_f32_16x16x32 per
//    16 columns of d. P^T comes out of the logits product already in the
//    B-operand layout; it enters as two 16-bit parts, the rounded weights
//    and their rounding residuals, paired with V twice along k, so P keeps
//    ~2^-18 relative accuracy. V^T arrives with one transposing LDS read per
//    tile. The accumulators hold full sums over the wave's tokens: lane l
//    holds head l % 16 at columns 16 T + 4 (l / 16) .. +3.
template <int DT, int G, int D>
// The arguments the prologue needs first come as leading scalars, so that
// the hardware can preload them into SGPRs at wave launch (gfx950 kernel
// argument preloading) instead of the first instructions waiting for a
// load from the argument segment; the rest stay in `rest`, loaded when used.
// (At most 256 registers per lane, two waves per SIMD: measured faster than
// the compiler's own choice even with one workgroup per CU.)
__global__ __launch_bounds__(kThreads, 2) void partial_kernel(
    const uint16_t* __restrict__ q, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const Item* __restrict__ items, int32_t mode,
    int32_t num_splits, int32_t split_chunk, int32_t num_kv_heads, int32_t stride,
    int32_t num_q_heads, PartialParams rest) {
  PartialParams a = rest;
  a.q = q;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.items = items;
  a.mode = mode;
  a.num_splits = num_splits;
  a.split_chunk = split_chunk;
  a.num_kv_heads = num_kv_heads;
  a.stride = stride;
  a.num_q_heads = num_q_heads;
  constexpr int W = kWavesPerGroup;
  constexpr int P = kPageTokens;
  constexpr int NKI = D / 32;     // K: 1 KiB DMA runs per page = MFMA steps
  constexpr int RB = D * 2;       // bytes per token row
  constexpr int NCH = RB / 16;    // 16-byte chunks per token row
  constexpr int VL = D / 8;       // 16-byte pieces (lanes) per token row
  constexpr int TPI = 64 / VL;    // token rows per 1 KiB load instruction
  constexpr int NVI = P / TPI;    // V loads per lane per page
  constexpr int TILE = P * D;     // elements of one (page, KV head) tile
  constexpr int NT = D / 16;      // 16-column tiles of the P.V product
  static_assert(G <= 16, "one MFMA tile of heads");

  constexpr int LPP = NKI + NVI;         // 16-byte load instructions per page
  constexpr int NB = kRingSlots;         // ring slots per wave (pages)
  constexpr int SLOT_WORDS = LPP * 256;  // one slot: LPP x 64 lanes x 16 B

  // K/V ring: each wave owns NB slots. One LDS array per slot (not one
  // array indexed by slot) lets the compiler tell slots apart. At the end a
  // wave's slot in the first array holds its state for the cross-wave
  // combine.
  static_assert(NB >= 2 && NB <= 4, "two to four slot arrays");
  __shared__ __attribute__((aligned(16))) uint32_t s_ring0[W * SLOT_WORDS];
  __shared__ __attribute__((aligned(16))) uint32_t s_ring1[W * SLOT_WORDS];
  __shared__ __attribute__((aligned(16))) uint32_t s_ring2[NB > 2 ? W * SLOT_WORDS : 4];
  __shared__ __attribute__((aligned(16))) uint32_t s_ring3[NB > 3 ? W * SLOT_WORDS : 4];
  __shared__ float s_m[W][G];
  __shared__ float s_l[W][G];
  static_assert(G * D <= SLOT_WORDS, "a wave's combine state fits in one ring slot");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads;

  // ---- which range this workgroup owns ----
  int b, g, pb, pe, slot = 0;
  bool early = false;  // range known before the row length
  SeqMeta row;         // (first slot, range count) of (b, g), for the merge
  if (a.mode == PKV_MODE_WORKQUEUE) {
    const Item it = a.items[blockIdx.x];
    b = it.b;
    g = it.g;
    pb = it.page_begin;
    pe = it.page_end;
    slot = it.slot;
    row = {it.row_base, it.row_count};
    early = true;
  } else if (a.mode == PKV_MODE_SPLIT) {
    // Grid S x Hkv x B, so (range, KV head, sequence) come without a
    // division; the linear workgroup order is still range-fastest.
    const int S = a.num_splits;
    const int s = blockIdx.x;
    g = blockIdx.y;
    b = blockIdx.z;
    const int bg = b * Hkv + g;
    const int cell = bg * S + s;
    if (a.split_chunk > 0) {  // every row has this range size
      pb = s * a.split_chunk;
      pe = pb + a.split_chunk;
      early = true;
    } else {
      const int pages = (a.seq_lens[b] + (a.k_new ? 1 : 0) + P - 1) / P;
      const int chunk = pages > 0 ? (pages + S - 1) / S : 1;  // row-local
      pb = s * chunk;
      pe = min(pb + chunk, pages);
    }
    slot = cell;
    row = {bg * S, S};
  } else {
    b = blockIdx.x / Hkv;
    g = blockIdx.x - b * Hkv;
    pb = 0;
    pe = 0x7fffffff;
    row = {0, 0};  // unsplit: no merge
  }
  // Lane roles: in the logits product this lane loads K row (token) t16;
  // in the S^T and O^T results it holds head t16, and tokens 4 hq .. +3
  // (S^T) or columns 16 T + 4 hq .. +3 (O^T); in MFMA operands hq picks the
  // lane's block along k. vr: the token row of the lane's 16-byte piece in
  // a 1 KiB row-major load (the new token's pool write).
  const int t16 = lane & 15;
  const int hq = lane >> 4;
  const int vr = lane / VL;

  // Q^T as the MFMA B operand: column t16 = head t16 of the group, k = d in
  // steps of 32: this lane holds d = 32 kk + 8 hq .. +7. Columns past G
  // repeat real heads (their logits are masked out), so every lane loads
  // unconditionally and the loads overlap the table and length loads below.
  u32x4 qa[NKI];
  {
    const uint16_t* qrow = a.q + ((int64_t)b * a.num_q_heads + g * G + (t16 % G)) * D;
#pragma unroll
    for (int kk = 0; kk < NKI; ++kk) qa[kk] = *(const u32x4*)(qrow + 32 * kk + 8 * hq);
  }

  // Block-table entries of the range are staged in LDS, kBtChunk at a time,
  // and read back with a broadcast LDS read: an in-loop vector load of the
  // table would make the compiler drain every outstanding K/V load. When the
  // range is known without the row length, the first chunk is fetched right
  // away (entries inside the table row only), overlapping the length load.
  __shared__ int32_t s_bt[kBtChunk];
  const int32_t* bt_row = a.block_table + (int64_t)b * a.stride;
  constexpr int U = kBtChunk / kThreads;
  int st_v[U];  // this thread's entries of the chunk being staged
  auto stage_load = [&](int c0, int span) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = threadIdx.x + u * kThreads;
      st_v[u] = i < span ? bt_row[c0 + i] : 0;
    }
  };
  auto stage_store = [&](int span) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = threadIdx.x + u * kThreads;
      if (i < span) s_bt[i] = st_v[u];
    }
  };
  // Row length, with the folded append's new token (at position n - 1).
  const int n = a.seq_lens[b] + (a.k_new ? 1 : 0);
  // With the range known early, the first pages' entries of this wave (see
  // the page loop) are loaded now too, in flight with the staging loads;
  // the staged entries are written to LDS only after the first K/V loads
  // have gone out.
  int e_first[kRingSlots];
  if (early) {
    const int span0 = min(min(pe, a.stride) - pb, kBtChunk);
#pragma unroll
    for (int i = 0; i < kRingSlots; ++i)
      e_first[i] = span0 > 0 ? bt_row[pb + min(wave + kWavesPerGroup * i, span0 - 1)] : 0;
    stage_load(pb, span0);
  }
  // Never past the device's own length, nor past the block-table row.
  pe = min(pe, min((n + P - 1) / P, a.stride));

  // Folded append: the workgroup whose range holds the new token's page
  // (exactly one per (row, KV head)) swaps the token into its operand
  // registers when it computes that page, and writes it to the pools at the
  // end (no other workgroup reads that page in this launch).
  const int app_page = a.k_new && n > 0 ? (n - 1) / P : -1;
  const bool app_owner = app_page >= pb && app_page < pe;  // workgroup-uniform
  const int app_slot = (n - 1) % P;
  int app_phys = 0;
  u32x4 k_tok[NKI], v_tok;  // this lane's pieces of the new token, in operand layout
  uint32_t v_col[NT];       // the new token's V at columns 16 T + t16 (V^T operand)
  if (app_owner) {
    app_phys = bt_row[app_page];
    const uint16_t* kn = a.k_new + ((int64_t)b * Hkv + g) * D;
    const uint16_t* vn = a.v_new + ((int64_t)b * Hkv + g) * D;
#pragma unroll
    for (int kk = 0; kk < NKI; ++kk) k_tok[kk] = *(const u32x4*)(kn + 32 * kk + 8 * hq);
    v_tok = *(const u32x4*)(vn + (lane % VL) * 8);
#pragma unroll
    for (int T = 0; T < NT; ++T) v_col[T] = vn[16 * T + t16];
  }

  // Wave w's combined acc goes to the start of its own first ring slot once
  // its page loop is over (its own loads and reads are done by then: no
  // barrier needed before the write).
  float* s_acc = reinterpret_cast<float*>(s_ring0);  // wave w at w * SLOT_WORDS
  if (pb >= pe) {
    // Empty range: read nothing; with neutral wave states the tail below
    // stores a neutral state (or zeros for a row with no tokens). One tail
    // for both cases keeps the kernel's code, and its cold end, small.
    for (int e = threadIdx.x; e < W * G * D; e += kThreads)
      s_acc[(e / (G * D)) * SLOT_WORDS + e % (G * D)] = 0.0f;
    if (threadIdx.x < W * G) {
      s_m[threadIdx.x / G][threadIdx.x % G] = kNoMax;
      s_l[threadIdx.x / G][threadIdx.x % G] = 0.0f;
    }
  } else {
  // This lane's K operand bytes inside a slot (rotated chunks), and the
  // global element offset its K DMA lanes fetch.
  uint32_t kofs[NKI];
  int kdma[NKI];
  // V in a slot: token-major rows of RB bytes, the 16-byte chunks of token t
  // rotated by vrot(t) positions, so that the 16 token rows one transposing
  // read touches (32 bytes each) spread over all banks. DMA lane `lane` of V
  // load i fills chunk position 64 i + lane.
  constexpr int TPB = 256 / RB;  // token rows per 256 bytes
  auto vrot = [&](int t) { return 2 * ((t / TPB) % (NCH / 2)); };
  int vdma[NVI];
#pragma unroll
  for (int i = 0; i < NVI; ++i) {
    const int pos = 64 * i + lane;
    const int t = pos / NCH, c = (pos % NCH - vrot(t) + NCH) % NCH;
    vdma[i] = t * D + c * 8;
  }
  // This lane's transposing-read address for tile T: the 8 bytes of token
  // 4 hq + t16 / 4 at columns 16 T + 4 (t16 % 4) .. +3.
  uint32_t vofs[NT];
#pragma unroll
  for (int T = 0; T < NT; ++T) {
    const int t = 4 * hq + t16 / 4, c = 2 * T + (t16 % 4) / 2;
    vofs[T] = NKI * 1024 + t * RB + ((c + vrot(t)) % NCH) * 16 + 8 * (t16 % 2);
  }
#pragma unroll
  for (int kk = 0; kk < NKI; ++kk) {
    kofs[kk] = t16 * RB + ((4 * kk + hq + t16) % NCH) * 16;
    const int pos = kk * 1024 + lane * 16;  // where DMA lane `lane` lands
    const int t = pos / RB, pch = (pos % RB) / 16;
    kdma[kk] = t * D + (((pch - t) % NCH + NCH) % NCH) * 8;  // t may exceed NCH
  }

  // O^T tiles: acc[T][i] = output of head t16 at column 16 T + 4 hq + i.
  floatx4 acc[NT];
  float lsum = 0.0f, mref = kNoMax;  // head t16; lsum over this lane's tokens
#pragma unroll
  for (int T = 0; T < NT; ++T) acc[T] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

  struct Page {
    u32x4 kb[NKI];
    uint32_t vt[NT][2];
    int ntok;  // valid tokens of the page (0 if its table entry is bad)
    int lp;    // page index in the row
  };

  int cb = pb;  // first page of the staged chunk
  int cnt = 0;  // pages of the chunk this wave computes
  int ntok_ring[NB];
  int lp_ring[NB];
  auto slot_base = [&](int sl) -> uint32_t* {
    uint32_t* base = sl == 0 ? s_ring0 : sl == 1 ? s_ring1 : sl == 2 ? s_ring2 : s_ring3;
    return base + wave * SLOT_WORDS;
  };

  // Issue page k of this wave's share of the chunk (k < cnt): its LPP
  // direct-to-LDS loads into ring slot `sl`. With `given`, `phys_in` is the
  // page's table entry, already in hand (the first pages of a chunk);
  // otherwise the entry is read from the staged table. Only real pages are
  // ever issued, so the loads in flight behind the page being computed are
  // those of its min(NB - 1, cnt - 1 - k) younger pages, always LPP each.
  auto issue_page = [&](int sl, int k, bool given = false, int phys_in = 0) {
    const int lp = cb + wave + W * k;
    int phys = given ? phys_in : __builtin_amdgcn_readfirstlane(s_bt[wave + W * k]);
    const bool ok = (uint64_t)(uint32_t)phys < (uint64_t)a.num_pages;
    ntok_ring[sl] = ok ? min(P, n - lp * P) : 0;
    lp_ring[sl] = lp;
    phys = ok ? phys : 0;
    const int64_t tile = ((int64_t)phys * Hkv + g) * TILE;
    const uint16_t* kp = a.k_pool + tile;
    const uint16_t* vp = a.v_pool + tile;
    uint32_t* dst = slot_base(sl);
#pragma unroll
    for (int kk = 0; kk < NKI; ++kk)
      __builtin_amdgcn_global_load_lds(GPTR(kp + kdma[kk]), LPTR(dst + kk * 256), 16, 0,
                                       kLoadNontemporal);
#pragma unroll
    for (int i = 0; i < NVI; ++i)
      __builtin_amdgcn_global_load_lds(GPTR(vp + vdma[i]),
                                       LPTR(dst + (NKI + i) * 256), 16, 0, kLoadNontemporal);
  };

  // Wait until slot `sl` has landed, with the loads of `younger` later pages
  // left in flight, then read this lane's operands back. The wait and the
  // LDS reads are one asm block: left to itself the compiler cannot tell the
  // ring slots apart at the loop back-edge and drains every load in flight.
  auto fetch_page = [&](int sl, int younger) -> Page {
    Page r;
    const uint32_t base = (uint32_t)(uintptr_t)LPTR(slot_base(sl));
    uint32_t ka[NKI];
#pragma unroll
    for (int i = 0; i < NKI; ++i) ka[i] = base + kofs[i];
    uint32_t va[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) va[T] = base + vofs[T];
    if (younger == NB - 1) {
      read_slot<LPP, (NB - 1) * LPP>(ka, va, r.kb, r.vt);
    } else if (NB > 2 && younger == 1) {
      read_slot<LPP, LPP>(ka, va, r.kb, r.vt);
    } else if (NB > 3 && younger == 2) {
      read_slot<LPP, 2 * LPP>(ka, va, r.kb, r.vt);
    } else {
      read_slot<LPP, 0>(ka, va, r.kb, r.vt);
    }
    r.ntok = ntok_ring[sl];
    r.lp = lp_ring[sl];
    return r;
  };

  auto compute_page = [&](Page& r) {
    if (app_owner && r.lp == app_page) {  // the new token's page: its slot from registers
#pragma unroll
      for (int kk = 0; kk < NKI; ++kk) r.kb[kk] = t16 == app_slot ? k_tok[kk] : r.kb[kk];
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t& w = r.vt[T][j / 2];
          const uint32_t keep = (j & 1) ? 0x0000ffffu : 0xffff0000u;
          const uint32_t put = (j & 1) ? (v_col[T] << 16) : v_col[T];
          w = 4 * hq + j == app_slot ? ((w & keep) | put) : w;
        }
    }
    // S^T = K Q^T: lane l gets head t16 and tokens 4 hq .. +3.
    floatx4 c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NKI; ++kk) c = mfma_16x16x32<DT>(r.kb[kk], qa[kk], c);
    // logits, log2 domain, masked by select (never by multiply: tails may
    // hold NaN); padding heads (t16 >= G) are masked too
    const bool head_ok = t16 < G;
    float x[4];
    bool need = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = head_ok && 4 * hq + i < r.ntok;
      x[i] = ok ? c[i] * a.scale_log2 : -INFINITY;
      need |= x[i] > mref + kTau;
    }
    if (__any(need)) {
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = swap32_max(swap16_max(mx));  // over the head's 16 tokens
      const float mn = fmaxf(mref, mx);
      const float al = fast_exp2(mref - mn);
      lsum *= al;
      mref = mn;
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[T][i] *= al;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = fast_exp2(x[i] - mref);
      lsum += p[i];
    }
    // P^T in the B-operand layout of the 16x16x32 product, as two 16-bit
    // parts: k = 8 hq + j holds the rounded weight of token 4 hq + j (j < 4)
    // or its rounding residual (j >= 4), so the product carries P to ~2^-18.
    const uint32_t h01 = pack2<DT>(p[0], p[1]), h23 = pack2<DT>(p[2], p[3]);
    float r0, r1, r2, r3;
    unpack2<DT>(h01, r0, r1);
    unpack2<DT>(h23, r2, r3);
    const u32x4 pt = {h01, h23, pack2<DT>(p[0] - r0, p[1] - r1), pack2<DT>(p[2] - r2, p[3] - r3)};
    if (r.ntok < P) {  // wave-uniform: only a row's last page is partial
#pragma unroll
      for (int T = 0; T < NT; ++T)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t& w = r.vt[T][j / 2];
          const uint32_t keep = (j & 1) ? 0x0000ffffu : 0xffff0000u;
          w = 4 * hq + j < r.ntok ? w : (w & keep);
        }
    }
#pragma unroll
    for (int T = 0; T < NT; ++T)
      acc[T] = mfma_16x16x32<DT>(u32x4{r.vt[T][0], r.vt[T][1], r.vt[T][0], r.vt[T][1]}, pt, acc[T]);
  };

  // Software pipeline over the LDS ring: the loads of the next NB-1 pages
  // are in flight while the current page is computed. Pages of the chunk
  // [cb, cb + kBtChunk) go to wave w in the order cb + w, cb + w + W, ...
  for (; cb < pe; cb += kBtChunk) {
    const int span = min(pe - cb, kBtChunk);
    const bool first_early = cb == pb && early;  // staging loads already in flight
    if (cb != pb) __syncthreads();  // every wave is done with the last chunk
    if (!first_early) {
      stage_load(cb, span);
      stage_store(span);
    }
    cnt = span > wave ? (span - wave + W - 1) / W : 0;
    // The first NB pages of this wave take their table entries straight from
    // memory (scalar loads, in flight with the staging), so the first K/V
    // loads go out before the barrier that publishes the staged table; the
    // wave then waits at that barrier with them in flight. Every wave passes
    // exactly one such barrier per chunk (a wave with no pages here too).
    if (cnt == 0) {
      if (first_early) stage_store(span);
      lds_barrier();
      continue;
    }
    int e[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i)
      e[i] = first_early ? e_first[i] : bt_row[cb + min(wave + W * i, span - 1)];
    // Everything older than the first pages' loads (q, the staging loads)
    // must have landed by the wait below, on every path: that keeps the
    // compiler from guarding the q registers inside the ring. The first
    // chunk of an early range waits after issuing its first pages (NB - 1
    // of them, or all at once when it has fewer), the others before.
    if (!first_early || cnt < NB - 1) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
      if (i < cnt) issue_page(i, i, true, e[i]);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NB - 1) * LPP));
    if (first_early) stage_store(span);  // the staged entries go to LDS now
    for (int k = 0; k < cnt; k += NB) {
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        const int kk = k + r;
        if (kk >= cnt) break;
        const bool more = kk + NB - 1 < cnt;  // wave-uniform
        if (kk == 0) {
          if (more) issue_page(NB - 1, NB - 1, true, e[NB - 1]);
          lds_barrier();  // the staged table is complete (K/V loads stay in flight)
        } else if (more) {
          issue_page((r + NB - 1) % NB, kk + NB - 1);
        }
        Page pg = fetch_page(r, more ? NB - 1 : cnt - 1 - kk);
        compute_page(pg);
      }
    }
  }

  // ---- combine the wave states, then the workgroup's waves ----
  // l: sum over the four token rows of head t16; the O^T tiles already hold
  // full sums over the wave's tokens. Lanes of real heads write their state.
  lsum = swap32_add(swap16_add(lsum));
  if (t16 < G) {
    if (hq == 0) {
      s_m[wave][t16] = mref;
      s_l[wave][t16] = lsum;
    }
#pragma unroll
    for (int T = 0; T < NT; ++T)
      *reinterpret_cast<floatx4*>(s_acc + wave * SLOT_WORDS + t16 * D + 16 * T + 4 * hq) = acc[T];
  }
  }  // non-empty range
  __syncthreads();
  // Combine the W wave states: each thread takes four consecutive columns of
  // one head (one float4 of the G x D state, one pass for G x D <= 4 x 256):
  // M = max of the waves' references, wave w weighted by 2^(m_w - M), summed
  // in wave order.
  for (int e4 = threadIdx.x; e4 < G * D / 4; e4 += kThreads) {
    const int h = (e4 * 4) / D, dd = e4 * 4 - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.0f;
    float4 A = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const float sc = fast_exp2(s_m[w][h] - M);
      const float4 x = *reinterpret_cast<const float4*>(s_acc + w * SLOT_WORDS + e4 * 4);
      L = fmaf(sc, s_l[w][h], L);
      A.x = fmaf(sc, x.x, A.x);
      A.y = fmaf(sc, x.y, A.y);
      A.z = fmaf(sc, x.z, A.z);
      A.w = fmaf(sc, x.w, A.w);
    }
    if (a.mode == PKV_MODE_UNSPLIT || slot < 0) {  // slot < 0: a row with no tokens
      const bool any = L > 0.0f;
      const uint32_t lo = pack1<DT>(any ? A.x / L : 0.0f) | ((uint32_t)pack1<DT>(any ? A.y / L : 0.0f) << 16);
      const uint32_t hi = pack1<DT>(any ? A.z / L : 0.0f) | ((uint32_t)pack1<DT>(any ? A.w / L : 0.0f) << 16);
      *(uint2*)(a.out + ((int64_t)b * a.num_q_heads + g * G + h) * D + dd) = make_uint2(lo, hi);
    } else {
      st_agent16(raw_rsrc(a.ws_acc + (int64_t)slot * G * D, G * D * 4), (uint32_t)(h * D + dd) * 4u, A);
      if (dd == 0) {
        st_agent(a.ws_m + (int64_t)slot * G + h, L > 0.0f ? M : -INFINITY);
        st_agent(a.ws_l + (int64_t)slot * G + h, L);
      }
    }
  }
  // Folded append: the owner writes the new token to the pools (for later
  // steps; a table entry outside the pool writes nothing, as in pkv_append),
  // and the row's first range of KV head 0 reports the new length.
  if (app_owner && wave == 0 && (uint64_t)(uint32_t)app_phys < (uint64_t)a.num_pages) {
    const int64_t row0 = (((int64_t)app_phys * Hkv + g) * P + app_slot) * D;
    if (t16 == 0) {
      uint16_t* kp = const_cast<uint16_t*>(a.k_pool) + row0;
#pragma unroll
      for (int kk = 0; kk < NKI; ++kk) *(u32x4*)(kp + 32 * kk + 8 * hq) = k_tok[kk];
    }
    if (vr == 0) *(u32x4*)(const_cast<uint16_t*>(a.v_pool) + row0 + lane * 8) = v_tok;
  }
  if (a.k_new && a.new_seq_lens && g == 0 && pb == 0 && threadIdx.x == 0)
    a.new_seq_lens[b] = n;
  if (a.mode != PKV_MODE_UNSPLIT && a.fused && slot >= 0)
    finish_group<DT, G, D>(a, b, g, row);
}

// ------------------------------------------------------------ merge kernel
//
// The separate merge launch: one workgroup per (sequence b, KV head g),
// running the same merge_row as the fused tail.
template <int DT, int G, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(MergeParams a) {
  const int bg = blockIdx.x;
  int b = bg / a.num_kv_heads;
  const int g = bg - b * a.num_kv_heads;
  if (a.rows) b = a.rows[b];
  int base, count;
  if (a.mode == PKV_MODE_WORKQUEUE) {
    const SeqMeta sm = a.meta[b];
    count = sm.splits;
    base = sm.slot_base + g * count;
  } else {
    count = a.num_splits;
    base = bg * count;
  }
  merge_row<DT, G, D>(a.ws_m, a.ws_l, a.ws_acc, base, count,
                      a.out + ((int64_t)b * a.num_q_heads + g * G) * D);
}

// -------------------------------------------------------------- dispatch

using PartialLaunch = void (*)(dim3, hipStream_t, const PartialParams&);
using MergeLaunch = void (*)(dim3, hipStream_t, const MergeParams&);

template <int DT, int G, int D>
void launch_partial(dim3 grid, hipStream_t s, const PartialParams& p) {
  hipLaunchKernelGGL((partial_kernel<DT, G, D>), grid, dim3(kThreads), 0, s, p.q,
                     p.block_table, p.seq_lens, p.items, p.mode, p.num_splits, p.split_chunk,
                     p.num_kv_heads, p.stride, p.num_q_heads, p);
}

template <int DT, int G, int D>
void launch_merge(dim3 grid, hipStream_t s, const MergeParams& p) {
  hipLaunchKernelGGL((merge_kernel<DT, G, D>), grid, dim3(kThreads), 0, s, p);
}

template <int DT, int D>
PartialLaunch pick_partial_g(int G) {
  switch (G) {
    case 1: return launch_partial<DT, 1, D>;
    case 2: return launch_partial<DT, 2, D>;
    case 4: return launch_partial<DT, 4, D>;
    case 8: return launch_partial<DT, 8, D>;
    default: return nullptr;
  }
}

PartialLaunch pick_partial(int dt, int G, int D) {
  if (dt == PKV_BF16) return D == 128 ? pick_partial_g<PKV_BF16, 128>(G) : pick_partial_g<PKV_BF16, 64>(G);
  return D == 128 ? pick_partial_g<PKV_F16, 128>(G) : pick_partial_g<PKV_F16, 64>(G);
}

template <int DT, int D>
MergeLaunch pick_merge_g(int G) {
  switch (G) {
    case 1: return launch_merge<DT, 1, D>;
    case 2: return launch_merge<DT, 2, D>;
    case 4: return launch_merge<DT, 4, D>;
    case 8: return launch_merge<DT, 8, D>;
    default: return nullptr;
  }
}

MergeLaunch pick_merge(int dt, int G, int D) {
  if (dt == PKV_BF16) return D == 128 ? pick_merge_g<PKV_BF16, 128>(G) : pick_merge_g<PKV_BF16, 64>(G);
  return D == 128 ? pick_merge_g<PKV_F16, 128>(G) : pick_merge_g<PKV_F16, 64>(G);
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

pkv_status hip_fail(const char* what, hipError_t e) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return PKV_ERR_HIP;
}

// One folded append (the new tokens and where the new lengths go), or none.
struct AppendArgs {
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int32_t* new_seq_lens = nullptr;
};

// `ws_static`: the workspace to use instead of the plan's bound one (the
// library's own scratch, already holding the plan's image), or null.
pkv_status decode_impl(const pkv_plan* p, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* seq_lens, void* out,
                       hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1, hipEvent_t ev2,
                       const AppendArgs& app = AppendArgs{}, void* ws_static = nullptr) {
  clear_error();
  if (!p) {
    set_error("plan is NULL");
    return PKV_ERR_INVALID;
  }
  if (app.k_new || app.v_new) {
    if (!app.k_new || !app.v_new) {
      set_error("k_new and v_new must both be given");
      return PKV_ERR_INVALID;
    }
    if (!aligned(app.k_new, 16) || !aligned(app.v_new, 16) || !aligned(app.new_seq_lens, 4)) {
      set_error("k_new/v_new must be 16-byte and new_seq_lens 4-byte aligned");
      return PKV_ERR_INVALID;
    }
    if (app.new_seq_lens && (const void*)app.new_seq_lens == (const void*)seq_lens) {
      set_error("new_seq_lens must not alias seq_lens (other workgroups still read it)");
      return PKV_ERR_INVALID;
    }
  }
  const pkv_shape& s = p->shape;
  if (s.batch == 0) {
    hipError_t e = hipSuccess;
    for (hipEvent_t ev : {ev0, ev1, ev2})
      if (ev && (e = hipEventRecord(ev, stream)) != hipSuccess) return hip_fail("hipEventRecord", e);
    return PKV_OK;
  }
  if (!q || !out || !seq_lens || (p->kv_tokens > 0 && (!k_pool || !v_pool || !block_table))) {
    set_error("a required device pointer is NULL");
    return PKV_ERR_INVALID;
  }
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4)) {
    set_error("q/out/k_pool/v_pool must be 16-byte and block_table/seq_lens 4-byte aligned");
    return PKV_ERR_INVALID;
  }
  if (p->mode != PKV_MODE_UNSPLIT && !p->uploaded && !ws_static) {
    set_error("plan has not been uploaded (pkv_plan_upload) since it was built");
    return PKV_ERR_STATE;
  }
  const int G = p->group, D = s.head_dim;
  PartialLaunch lp = pick_partial(s.dtype, G, D);
  MergeLaunch lm = pick_merge(s.dtype, G, D);
  if (!lp || !lm) {
    set_error("no kernel for head_dim %d, G %d", D, G);
    return PKV_ERR_UNSUPPORTED;
  }
  char* ws = (char*)(ws_static ? ws_static : p->workspace);
  const pkv_workspace_layout& L = p->layout;

  PartialParams pp{};
  pp.q = (const uint16_t*)q;
  pp.k_pool = (const uint16_t*)k_pool;
  pp.v_pool = (const uint16_t*)v_pool;
  pp.block_table = block_table;
  pp.seq_lens = seq_lens;
  pp.out = (uint16_t*)out;
  if (ws) {
    pp.items = (const Item*)(ws + L.items_offset);
    pp.meta = (const SeqMeta*)(ws + L.meta_offset);
    pp.counters = (int32_t*)(ws + L.counters_offset);
    pp.ws_m = (float*)(ws + L.m_offset);
    pp.ws_l = (float*)(ws + L.l_offset);
    pp.ws_acc = (float*)(ws + L.acc_offset);
  }
  pp.fused = p->fused;
  pp.num_pages = s.num_pages;
  pp.stride = s.block_table_stride;
  pp.num_kv_heads = s.num_kv_heads;
  pp.num_q_heads = s.num_q_heads;
  pp.mode = p->mode;
  pp.num_splits = p->num_splits;
  pp.split_chunk = p->split_chunk;
  pp.scale_log2 = s.sm_scale * kLog2e;
  pp.k_new = (const uint16_t*)app.k_new;
  pp.v_new = (const uint16_t*)app.v_new;
  pp.new_seq_lens = app.new_seq_lens;

  MergeParams mp{};
  mp.ws_m = pp.ws_m;
  mp.ws_l = pp.ws_l;
  mp.ws_acc = pp.ws_acc;
  mp.meta = (const SeqMeta*)(ws + L.meta_offset);
  mp.out = (uint16_t*)out;
  mp.num_kv_heads = s.num_kv_heads;
  mp.num_q_heads = s.num_q_heads;
  mp.group = G;
  mp.mode = p->mode;
  mp.num_splits = p->num_splits;

  hipError_t e;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return hip_fail("hipEventRecord", e);
  if (p->mode == PKV_MODE_BUCKETED) {
    // One partial launch per exact-length bucket (its items are a work
    // queue of their own) and, with the separate merge, one merge launch
    // over the bucket's sequences.
    pp.mode = PKV_MODE_WORKQUEUE;
    mp.mode = PKV_MODE_WORKQUEUE;
    const Item* items = pp.items;
    const int32_t* rows = (const int32_t*)(ws + L.meta_offset + sizeof(SeqMeta) * s.batch);
    for (const Bucket& bk : p->buckets) {
      if (bk.item_count > 0) {
        pp.items = items + bk.item_begin;
        lp(dim3(bk.item_count), stream, pp);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail("partial kernel launch", e);
      }
      if (!p->fused && bk.row_count > 0) {
        mp.rows = rows + bk.row_begin;
        lm(dim3(bk.row_count * s.num_kv_heads), stream, mp);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail("merge kernel launch", e);
      }
    }
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return hip_fail("hipEventRecord", e);
  } else {
    if (p->grid > 0) {
      const dim3 grid = p->mode == PKV_MODE_SPLIT
                            ? dim3(p->num_splits, s.num_kv_heads, s.batch)  // = p->grid workgroups
                            : dim3(p->grid);
      lp(grid, stream, pp);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail("partial kernel launch", e);
    }
    if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return hip_fail("hipEventRecord", e);
    if (p->mode != PKV_MODE_UNSPLIT && !p->fused) {
      lm(dim3(s.batch * s.num_kv_heads), stream, mp);
      if ((e = hipGetLastError()) != hipSuccess) return hip_fail("merge kernel launch", e);
    }
  }
  if (ev2 && (e = hipEventRecord(ev2, stream)) != hipSuccess) return hip_fail("hipEventRecord", e);
  return PKV_OK;
}

}  // namespace

pkv_status query_num_cus(int32_t* num_cus) {
  int dev = 0, v = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || v <= 0) {
    set_error("cannot query the device's compute-unit count (pass opts.num_cus): %s",
              hipGetErrorString(e));
    return PKV_ERR_HIP;
  }
  *num_cus = v;
  return PKV_OK;
}

void wait_upload(pkv_plan* p) {
  if (p && p->upload_event) (void)hipEventSynchronize((hipEvent_t)p->upload_event);
}

void release_device_resources(pkv_plan* p) {
  if (!p) return;
  if (p->upload_event) {
    (void)hipEventSynchronize((hipEvent_t)p->upload_event);
    (void)hipEventDestroy((hipEvent_t)p->upload_event);
    p->upload_event = nullptr;
  }
  if (p->pinned) {
    (void)hipHostFree(p->pinned);
    p->pinned = nullptr;
    p->pinned_bytes = 0;
  }
}

// ------------------------------------------------ allocation-free entry
//
// The library's own device scratch for pkv_decode_static: one copy per
// device (a __device__ array), holding a plan's workspace (queue image,
// merge counters, partial states). Host code never passes the array's name
// to a kernel or copy: hipGetSymbolAddress gives each device's address,
// looked up once per device with that device current, and only that
// address is used.
constexpr size_t kStaticScratchBytes = PKV_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace pkv

static __device__ __align__(256) unsigned char scratch[pkv::kStaticScratchBytes];

namespace pkv {

pkv_status static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device %d: the static scratch is kept for devices 0 .. %d", dev, kMaxDevices - 1);
    return PKV_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (!ptr || (uintptr_t)ptr % 256) {
      set_error("static scratch address %p is not 256-byte aligned", ptr);
      return PKV_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

pkv_status pkv_decode_static(const pkv_plan* p, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, hipStream_t stream) {
  pkv::clear_error();
  if (!p) {
    pkv::set_error("plan is NULL");
    return PKV_ERR_INVALID;
  }
  const size_t need = (size_t)p->layout.total_bytes;
  if (need > pkv::kStaticScratchBytes) {
    pkv::set_error("the plan needs a %zu-byte workspace; the static scratch holds %zu bytes",
                   need, pkv::kStaticScratchBytes);
    return PKV_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  if (need > 0) {
    pkv_status st = pkv::static_scratch(&ws);
    if (st != PKV_OK) return st;
    // The queue image and zeroed merge counters go in first, on the stream,
    // from host memory the plan owns: the scratch holds whatever the
    // previous call on this device left.
    if (p->upload_bytes > 0) {
      const hipError_t e = hipMemcpyAsync(ws, p->static_image.data(), (size_t)p->upload_bytes,
                                          hipMemcpyHostToDevice, stream);
      if (e != hipSuccess) return pkv::hip_fail("hipMemcpyAsync(static scratch)", e);
    }
  }
  // (a plan that needs no workspace, unsplit, needs no upload either)
  return pkv::decode_impl(p, q, k_pool, v_pool, block_table, seq_lens, out, stream, nullptr,
                          nullptr, nullptr, pkv::AppendArgs{}, ws);
}

pkv_status pkv_plan_upload(pkv_plan* p, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  pkv::clear_error();
  if (!p) {
    pkv::set_error("plan is NULL");
    return PKV_ERR_INVALID;
  }
  const size_t need = (size_t)p->layout.total_bytes;
  if (need > 0) {
    if (!workspace) {
      pkv::set_error("workspace is NULL but the plan needs %zu bytes", need);
      return PKV_ERR_WORKSPACE;
    }
    if (workspace_bytes < need) {
      pkv::set_error("workspace of %zu bytes is smaller than the %zu the plan needs",
                     workspace_bytes, need);
      return PKV_ERR_WORKSPACE;
    }
    if ((uintptr_t)workspace % 256) {
      pkv::set_error("workspace must be 256-byte aligned");
      return PKV_ERR_WORKSPACE;
    }
  }
  // A plan that needs no workspace keeps none bound: a later re-plan that
  // needs one then asks for a new upload instead of trusting an unchecked
  // pointer.
  p->workspace = need > 0 ? workspace : nullptr;
  p->workspace_bytes = need > 0 ? workspace_bytes : 0;
  hipError_t e;
  if (p->upload_bytes > 0) {
    const size_t nb = (size_t)p->upload_bytes;
    if (p->upload_event) (void)hipEventSynchronize((hipEvent_t)p->upload_event);
    if (p->pinned_bytes < nb) {
      if (p->pinned) (void)hipHostFree(p->pinned);
      p->pinned = nullptr;
      p->pinned_bytes = 0;
      if ((e = hipHostMalloc(&p->pinned, nb, hipHostMallocDefault)) != hipSuccess)
        return pkv::hip_fail("hipHostMalloc", e);
      p->pinned_bytes = nb;
    }
    char* st = (char*)p->pinned;
    pkv::write_upload_image(*p, st);
    if ((e = hipMemcpyAsync(workspace, st, nb, hipMemcpyHostToDevice, stream)) != hipSuccess)
      return pkv::hip_fail("hipMemcpyAsync", e);
    if (!p->upload_event) {
      hipEvent_t ev;
      if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess)
        return pkv::hip_fail("hipEventCreate", e);
      p->upload_event = ev;
    }
    if ((e = hipEventRecord((hipEvent_t)p->upload_event, stream)) != hipSuccess)
      return pkv::hip_fail("hipEventRecord", e);
  }
  p->copied_bytes = p->upload_bytes;
  p->uploaded = true;
  return PKV_OK;
}

pkv_status pkv_decode(const pkv_plan* p, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens, void* out,
                      hipStream_t stream) {
  return pkv::decode_impl(p, q, k_pool, v_pool, block_table, seq_lens, out, stream, nullptr,
                          nullptr, nullptr);
}

pkv_status pkv_decode_append(const pkv_plan* p, const void* q, const void* k_new,
                             const void* v_new, void* k_pool, void* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int32_t* new_seq_lens, void* out, hipStream_t stream) {
  pkv::AppendArgs app;
  app.k_new = k_new;
  app.v_new = v_new;
  app.new_seq_lens = new_seq_lens;
  if (!k_new || !v_new) {
    pkv::clear_error();
    pkv::set_error("k_new and v_new are required");
    return PKV_ERR_INVALID;
  }
  return pkv::decode_impl(p, q, k_pool, v_pool, block_table, seq_lens, out, stream, nullptr,
                          nullptr, nullptr, app);
}

pkv_status pkv_decode_marked(const pkv_plan* p, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, hipStream_t stream,
                             hipEvent_t before, hipEvent_t after_partial, hipEvent_t after_merge) {
  return pkv::decode_impl(p, q, k_pool, v_pool, block_table, seq_lens, out, stream, before,
                          after_partial, after_merge);
}

}  // extern "C"
