// Internal declarations shared by the host planner (plan.cpp, HIP-free) and
// the device side (decode.hip). Not part of the ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "pkv.h"

namespace pkv {

// Tokens per KV page. The pages name 16-token blocks as the usual size
// (LLM Primer ch. 8, section 8.1); the kernels are built for exactly that.
constexpr int kPageTokens = 16;

// Waves (64 lanes each) in one partial-kernel workgroup. A workgroup owns
// one (sequence, KV head, page range) item; its waves take the range's
// pages round-robin and merge their states in LDS at the end.
#ifndef PKV_WAVES_PER_GROUP
#define PKV_WAVES_PER_GROUP 4
#endif
constexpr int kWavesPerGroup = PKV_WAVES_PER_GROUP;

// Work-queue item as the partial kernel reads it (32 bytes, one scalar
// load). It also names its row's slots (first slot of (b, g) and the row's
// range count), so the merge in the partial kernel's tail needs no other
// table.
struct Item {
  int32_t bg;          // b * Hkv + g
  int32_t page_begin;  // first page of the range (logical page index)
  int32_t page_end;    // one past the last page
  int32_t slot;        // partial-state slot this range writes (-1: zero-fill item)
  int32_t row_base;    // first slot of (b, g)
  int32_t row_count;   // ranges of (b, g)
  int32_t b, g;        // bg split, so the kernel needs no division for it
};
static_assert(sizeof(Item) == 32, "item layout");

struct SeqMeta {
  int32_t slot_base;  // first slot of sequence b
  int32_t splits;     // S_b: ranges per KV head of sequence b
};

// One exact-length bucket (BUCKETED mode): its items and its rows, as
// ranges of the plan's item and row lists.
struct Bucket {
  int32_t item_begin, item_count;
  int32_t row_begin, row_count;
};

}  // namespace pkv

struct pkv_plan {
  pkv_shape shape{};
  pkv_opts opts{};
  int32_t group = 0;       // G
  int32_t num_cus = 0;
  int32_t fused = 1;       // merge inside the partial kernel

  // Resolved schedule.
  int32_t mode = PKV_MODE_UNSPLIT;
  int32_t num_splits = 1;  // S
  int32_t chunk_pages = 0;
  int32_t split_chunk = 0;  // SPLIT with one page count for every row: its range size
  int32_t grid = 0;
  int32_t num_items = 0;
  int32_t empty_items = 0;
  int32_t num_slots = 0;
  int32_t bucket_launches = 0;
  int64_t kv_tokens = 0;
  int64_t algorithmic_bytes = 0;
  int64_t partial_bytes = 0;
  int64_t upload_bytes = 0;

  std::vector<int32_t> seq_lens;
  std::vector<pkv::Item> items;
  std::vector<pkv::SeqMeta> meta;
  std::vector<int32_t> rows;            // BUCKETED: sequences, bucket by bucket
  std::vector<pkv::Bucket> buckets;     // BUCKETED

  pkv_workspace_layout layout{};

  // Device binding (decode.hip owns these).
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  bool uploaded = false;
  void* pinned = nullptr;  // pinned staging of [items | meta]: the image last copied
  size_t pinned_bytes = 0;
  int64_t copied_bytes = 0;         // length of that image (0: none copied yet)
  std::vector<char> static_image;  // the upload image as last built (pkv_decode_static copies
                                   // it; a re-plan compares it with the copied one)
  void* upload_event = nullptr;  // hipEvent_t of the last upload copy
  int device = -1;
};

namespace pkv {

// Fill `dst` (upload_bytes long) with the workspace image the upload sends:
// items, per-row table, zeroed counters (plan.cpp).
void write_upload_image(const pkv_plan& p, void* dst);

// Thread-local error text (plan.cpp).
void set_error(const char* fmt, ...);
void clear_error();

// Device-side hooks implemented in decode.hip.
pkv_status query_num_cus(int32_t* num_cus);
void wait_upload(pkv_plan* plan);           // block until staging is free
void release_device_resources(pkv_plan* plan);

// Shapes the kernels are instantiated for (decode.hip dispatches exactly
// these): head_dim 64 or 128, G in {1, 2, 4, 8}.
inline bool kernel_supported(int32_t head_dim, int32_t group) {
  return (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

}  // namespace pkv
