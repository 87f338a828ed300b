// Host planner for one paged GQA decode step: policy, row-local page ranges,
// compact work queue, workspace layout and scheduler counters.
//
// Integer work only, and no HIP calls (except asking the device for its CU
// count when the caller does not supply one), so it runs and is tested on a
// machine without a GPU.
//
// Method (PersistentKV explainer, Technical summary > Methodology):
//  * sequence splitting: the token axis of each (sequence, KV head) is cut
//    into disjoint ranges, each producing a partial online-softmax state that
//    a merge kernel combines exactly (Methodology 1);
//  * row-local bounds: range counts and boundaries come from each row's true
//    length, not a padded one; a split with no tokens produces the neutral
//    state and reads nothing (Methodology 1);
//  * compact work queue: a 1-D grid over the non-empty
//    (row, KV head, range) items only, so a ragged batch costs one partial
//    and one merge launch instead of launches per distinct length
//    (Methodology 1; Results, launch fan-out);
//  * a calibrated policy chooses the path from the batch size and the
//    lengths (Methodology 2). The pages' thresholds were fitted to a 28-SM
//    consumer GPU; the rule here is stated in terms of the MI355X's compute
//    units and workgroup residency instead.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <new>

#include "pkv_internal.h"

namespace pkv {
namespace {

thread_local std::string g_error;

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// --- Policy constants (MI355X) -------------------------------------------
// Measured on an MI355X (256 CUs) with the calibration seed (20260622) over
// the long, mixed B=8, B=4 and B=64 workloads: the step is fastest when every
// CU runs at most one work item (a single split-S row: S = 32 beat 64 by 10%;
// on ragged B=4 and B=8 batches the best range size was the smallest one
// whose item count, after rounding each row up, fits the CUs: items of a
// second workgroup on some CUs finish late). Batches too large for that
// want items of at most ~512 pages so the longest-first queue stays
// balanced (within 2% from 256 to 1024; a whole-row unsplit launch of the
// B=64 batch was 2x slower).
constexpr int kTargetItemsPerCU = 1;
constexpr int kMaxChunkPages = 512;
// Smallest range worth a workgroup (pages): two pages per wave.
constexpr int kMinChunkPages = 2 * kWavesPerGroup;
// The split grid's y and z dimensions (KV heads, sequences) stay within the
// smallest grid-dimension limit HIP devices report.
constexpr int32_t kMaxGridYZ = 65535;

int32_t pages_of(int32_t n) { return (int32_t)ceil_div(n, kPageTokens); }

// Work items (ranges of at most c pages, per row and KV head) of rows `lens`.
int64_t items_at(const std::vector<int32_t>& lens, int32_t Hkv, int64_t c) {
  int64_t n = 0;
  for (int32_t len : lens) n += ceil_div(pages_of(len), c);
  return n * Hkv;
}

// Range size for rows `lens`: the smallest multiple of the wave count, from
// the even share of their page-heads per CU up to kMaxChunkPages, whose
// items (each row rounded up separately) fit one per CU.
int32_t auto_chunk(const std::vector<int32_t>& lens, int32_t Hkv, int32_t num_cus) {
  const int64_t target = std::max<int64_t>(1, (int64_t)num_cus * kTargetItemsPerCU);
  int64_t total_pages = 0;
  for (int32_t len : lens) total_pages += pages_of(len);
  const int64_t work = total_pages * Hkv;
  int64_t c = std::min<int64_t>(std::max<int64_t>(ceil_div(work, target), kMinChunkPages),
                                kMaxChunkPages);
  c = align_up(c, kWavesPerGroup);
  while (c < kMaxChunkPages && items_at(lens, Hkv, c) > target) c += kWavesPerGroup;
  return (int32_t)c;
}

// Stable order by range length, longest first (items of one length keep
// their order): a counting placement, since lengths are bounded by the
// range size; very long ranges fall back to a stable sort.
void longest_first(std::vector<Item>& items) {
  constexpr int32_t kCountingMax = 4096;
  int32_t maxlen = 0;
  for (const Item& it : items) maxlen = std::max(maxlen, it.page_end - it.page_begin);
  if (maxlen > kCountingMax) {
    std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
      return (a.page_end - a.page_begin) > (b.page_end - b.page_begin);
    });
    return;
  }
  thread_local std::vector<int32_t> start;
  thread_local std::vector<Item> sorted;
  start.assign((size_t)maxlen + 1, 0);
  for (const Item& it : items) ++start[it.page_end - it.page_begin];
  int32_t off = 0;
  for (int32_t len = maxlen; len >= 0; --len) {
    const int32_t c = start[len];
    start[len] = off;
    off += c;
  }
  sorted.resize(items.size());
  for (const Item& it : items) sorted[start[it.page_end - it.page_begin]++] = it;
  items.swap(sorted);
}

uint64_t splitmix64(uint64_t& s) {
  uint64_t z = (s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

pkv_status validate(const pkv_shape* s, const int32_t* lens) {
  if (!s) {
    set_error("shape is NULL");
    return PKV_ERR_INVALID;
  }
  if (s->batch < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 ||
      s->head_dim <= 0 || s->page_size <= 0 || s->block_table_stride < 0 ||
      s->num_pages < 0) {
    set_error("shape has a negative or zero size");
    return PKV_ERR_INVALID;
  }
  if (s->num_q_heads % s->num_kv_heads != 0) {
    set_error("num_q_heads (%d) is not a multiple of num_kv_heads (%d)",
              s->num_q_heads, s->num_kv_heads);
    return PKV_ERR_INVALID;
  }
  if (!(s->sm_scale >= 0.0f) || std::isinf(s->sm_scale)) {
    set_error("sm_scale must be finite and >= 0");
    return PKV_ERR_INVALID;
  }
  if (s->dtype != PKV_F16 && s->dtype != PKV_BF16) {
    set_error("unsupported dtype %d", s->dtype);
    return PKV_ERR_UNSUPPORTED;
  }
  if (s->page_size != kPageTokens) {
    set_error("page_size %d unsupported (built for %d)", s->page_size, kPageTokens);
    return PKV_ERR_UNSUPPORTED;
  }
  int32_t G = s->num_q_heads / s->num_kv_heads;
  if (!kernel_supported(s->head_dim, G)) {
    set_error("no kernel for head_dim %d with G = %d", s->head_dim, G);
    return PKV_ERR_UNSUPPORTED;
  }
  if ((int64_t)s->batch * s->num_q_heads > INT32_MAX / 2) {
    set_error("batch * num_q_heads too large");
    return PKV_ERR_INVALID;
  }
  if (s->batch > 0 && !lens) {
    set_error("seq_lens_host is NULL");
    return PKV_ERR_INVALID;
  }
  const int64_t cap = (int64_t)s->block_table_stride * s->page_size;
  for (int32_t b = 0; b < s->batch; ++b) {
    if (lens[b] < 0 || lens[b] > cap) {
      set_error("seq_lens[%d] = %d outside [0, %lld]", b, lens[b], (long long)cap);
      return PKV_ERR_INVALID;
    }
    if (lens[b] > 0 && s->num_pages <= 0) {
      set_error("num_pages is 0 but seq_lens[%d] = %d", b, lens[b]);
      return PKV_ERR_INVALID;
    }
  }
  return PKV_OK;
}

// Build the schedule for p.seq_lens under p.opts.
pkv_status build(pkv_plan& p) {
  const pkv_shape& s = p.shape;
  const int32_t B = s.batch, Hkv = s.num_kv_heads, G = p.group, d = s.head_dim;

  int64_t total_pages = 0, kv_tokens = 0;
  int32_t max_pages = 0, active = 0;
  // Re-planning runs every step: scratch buffers keep their capacity per
  // thread, so a re-plan allocates nothing once warmed up.
  thread_local std::vector<int32_t> nonzero;
  nonzero.clear();
  bool same_len = true;
  for (int32_t b = 0; b < B; ++b) {
    int32_t n = p.seq_lens[b];
    total_pages += pages_of(n);
    kv_tokens += n;
    max_pages = std::max(max_pages, pages_of(n));
    if (n > 0) {
      ++active;
      nonzero.push_back(n);
    }
    if (pages_of(n) != pages_of(p.seq_lens[0])) same_len = false;
  }
  std::sort(nonzero.begin(), nonzero.end());
  const int32_t distinct_lengths =
      (int32_t)(std::unique(nonzero.begin(), nonzero.end()) - nonzero.begin());

  // ---- mode ----
  int32_t mode = p.opts.mode;
  if (mode < PKV_MODE_AUTO || mode > PKV_MODE_BUCKETED) {
    set_error("unknown mode %d", mode);
    return PKV_ERR_INVALID;
  }
  if (p.opts.num_splits < 0 || p.opts.chunk_pages < 0) {
    set_error("num_splits and chunk_pages must be >= 0");
    return PKV_ERR_INVALID;
  }
  if (p.opts.merge != PKV_MERGE_FUSED && p.opts.merge != PKV_MERGE_KERNEL) {
    set_error("unknown merge %d", p.opts.merge);
    return PKV_ERR_INVALID;
  }
  p.fused = p.opts.merge == PKV_MERGE_FUSED;
  int32_t chunk = p.opts.chunk_pages > 0 ? p.opts.chunk_pages
                                         : auto_chunk(p.seq_lens, Hkv, p.num_cus);
  if (mode == PKV_MODE_AUTO) {
    if (active == 0 || max_pages <= chunk) {
      mode = PKV_MODE_UNSPLIT;  // every row fits in one item: nothing to merge
    } else if (same_len && B <= kMaxGridYZ && Hkv <= kMaxGridYZ) {
      mode = PKV_MODE_SPLIT;  // equal rows: the rectangular grid wastes nothing
    } else {
      mode = PKV_MODE_WORKQUEUE;  // ragged rows: only non-empty ranges
    }
  }

  if (mode == PKV_MODE_SPLIT && (B > kMaxGridYZ || Hkv > kMaxGridYZ)) {
    set_error("split grid: batch and KV heads must be at most %d each (the work queue has no "
              "such limit)", kMaxGridYZ);
    return PKV_ERR_UNSUPPORTED;
  }

  p.items.clear();
  p.meta.clear();
  p.rows.clear();
  p.buckets.clear();
  p.mode = mode;
  p.split_chunk = 0;
  p.kv_tokens = kv_tokens;
  p.bucket_launches = 2 * distinct_lengths;

  int64_t num_slots = 0;
  if (mode == PKV_MODE_UNSPLIT) {
    p.num_splits = 1;
    p.chunk_pages = max_pages;
    p.grid = B * Hkv;
    p.num_items = active * Hkv;
    p.empty_items = p.grid - p.num_items;
  } else if (mode == PKV_MODE_SPLIT) {
    int32_t S = p.opts.num_splits > 0
                    ? p.opts.num_splits
                    : (int32_t)std::max<int64_t>(1, ceil_div(max_pages, chunk));
    if (max_pages > 0) S = std::min(S, max_pages);
    S = std::max(S, 1);
    int64_t grid = (int64_t)B * Hkv * S;
    if (grid > INT32_MAX / 2) {
      set_error("split grid too large");
      return PKV_ERR_INVALID;
    }
    int32_t items = 0, cmax = 0;
    for (int32_t b = 0; b < B; ++b) {
      int32_t pg = pages_of(p.seq_lens[b]);
      if (pg == 0) continue;
      int32_t cb = (int32_t)ceil_div(pg, S);
      cmax = std::max(cmax, cb);
      items += (int32_t)ceil_div(pg, cb) * Hkv;
    }
    p.num_splits = S;
    p.chunk_pages = cmax;
    // Rows of one page count share one range size, known here: the kernel
    // can then fetch its block-table entries before the row length.
    p.split_chunk = same_len ? cmax : 0;
    p.grid = (int32_t)grid;
    p.num_items = items;
    p.empty_items = p.grid - items;
    num_slots = grid;
  } else if (mode == PKV_MODE_BUCKETED) {
    // Exact-length buckets, longest first; empty rows last, as a bucket
    // that only writes zeros.
    std::map<int32_t, std::vector<int32_t>, std::greater<int32_t>> by_len;
    for (int32_t b = 0; b < B; ++b) by_len[p.seq_lens[b]].push_back(b);
    p.meta.assign(B, SeqMeta{0, 0});
    int32_t smax = 0, cmax = 0, fills = 0;
    for (const auto& kv : by_len) {
      const int32_t len = kv.first, pg = pages_of(len);
      const std::vector<int32_t>& rows = kv.second;
      Bucket bk{(int32_t)p.items.size(), 0, (int32_t)p.rows.size(), (int32_t)rows.size()};
      if (pg > 0) {
        // Planned as if the bucket ran alone: its own range size.
        const std::vector<int32_t> lens(rows.size(), len);
        const int32_t c = p.opts.chunk_pages > 0 ? p.opts.chunk_pages
                                                 : auto_chunk(lens, Hkv, p.num_cus);
        const int32_t Sb = (int32_t)ceil_div(pg, c);
        for (int32_t b : rows) {
          p.meta[b] = {(int32_t)num_slots, Sb};
          for (int32_t g = 0; g < Hkv; ++g)
            for (int32_t si = 0; si < Sb; ++si)
              p.items.push_back({b * Hkv + g, si * c, std::min(pg, (si + 1) * c),
                                 (int32_t)(num_slots + (int64_t)g * Sb + si),
                                 (int32_t)(num_slots + (int64_t)g * Sb), Sb, b, g});
          num_slots += (int64_t)Hkv * Sb;
          if (num_slots > INT32_MAX / 2) {
            set_error("bucket plan too large");
            return PKV_ERR_INVALID;
          }
        }
        smax = std::max(smax, Sb);
        cmax = std::max(cmax, c);
      } else if (p.fused) {
        for (int32_t b : rows)
          for (int32_t g = 0; g < Hkv; ++g) p.items.push_back({b * Hkv + g, 0, 0, -1, 0, 0, b, g});
        fills += (int32_t)rows.size() * Hkv;
      }
      for (int32_t b : rows) p.rows.push_back(b);
      bk.item_count = (int32_t)p.items.size() - bk.item_begin;
      p.buckets.push_back(bk);
    }
    p.num_splits = std::max(smax, 1);
    p.chunk_pages = cmax;
    p.grid = (int32_t)p.items.size();
    p.num_items = p.grid - fills;
    p.empty_items = fills;
  } else {  // WORKQUEUE
    if (chunk <= 0) chunk = kMinChunkPages;
    int32_t smax = 0;
    int64_t n_full = 0, n_short = 0, n_fill = 0;
    p.meta.resize(B);
    for (int32_t b = 0; b < B; ++b) {
      const int32_t pg = pages_of(p.seq_lens[b]);
      const int32_t Sb = (int32_t)ceil_div(pg, chunk);
      p.meta[b] = {(int32_t)num_slots, Sb};
      const bool short_last = pg % chunk != 0;  // Sb > 0 then
      n_full += (int64_t)Hkv * (Sb - (short_last ? 1 : 0));
      n_short += short_last ? Hkv : 0;
      n_fill += (Sb == 0 && p.fused) ? Hkv : 0;
      num_slots += (int64_t)Hkv * Sb;
      smax = std::max(smax, Sb);
      if (num_slots > INT32_MAX / 2) {
        set_error("work queue too large");
        return PKV_ERR_INVALID;
      }
    }
    // The queue is written in place, longest range first with ranges of one
    // length in (b, g, range) order: the hardware hands workgroups out in
    // launch order, so this is greedy longest-processing-time scheduling.
    // Every range but a row's last is `chunk` pages long, so the order is the
    // full ranges as generated, then the short last ranges by length, then
    // the zero-fill items. (An empty row has no range; with the merge fused
    // into the partial kernel nothing else would write its zero output, so it
    // gets one zero-fill item per KV head: slot -1, no pages.) Only the short
    // ranges, at most one per (b, g), are sorted.
    p.items.resize((size_t)(n_full + n_short + n_fill));
    thread_local std::vector<Item> tails;
    tails.clear();
    Item* full = p.items.data();
    Item* fill = full + n_full + n_short;
    for (int32_t b = 0; b < B; ++b) {
      const int32_t pg = pages_of(p.seq_lens[b]);
      const int32_t Sb = p.meta[b].splits;
      for (int32_t g = 0; g < Hkv; ++g) {
        const int32_t base = p.meta[b].slot_base + g * Sb;
        for (int32_t si = 0; si < Sb; ++si) {
          const Item it{b * Hkv + g, si * chunk, std::min(pg, (si + 1) * chunk), base + si, base,
                        Sb, b, g};
          if (it.page_end - it.page_begin == chunk)
            *full++ = it;
          else
            tails.push_back(it);
        }
        if (Sb == 0 && p.fused) *fill++ = {b * Hkv + g, 0, 0, -1, 0, 0, b, g};
      }
    }
    longest_first(tails);
    std::copy(tails.begin(), tails.end(), full);
    if (p.opts.queue_seed != 0) {  // a seeded shuffle of the queue (tests: order independence)
      uint64_t st = p.opts.queue_seed;
      for (size_t i = p.items.size(); i > 1; --i)
        std::swap(p.items[i - 1], p.items[splitmix64(st) % i]);
    }
    int32_t fills = 0;
    for (const Item& it : p.items) fills += it.slot < 0;
    p.num_splits = smax;
    p.chunk_pages = chunk;
    p.grid = (int32_t)p.items.size();
    p.num_items = p.grid - fills;
    p.empty_items = fills;
  }
  p.num_slots = (int32_t)num_slots;
  // The merge addresses one row's states with 32-bit byte offsets.
  if (mode != PKV_MODE_UNSPLIT && (int64_t)p.num_splits * G * d * 4 > INT32_MAX) {
    set_error("too many ranges per row (%d)", p.num_splits);
    return PKV_ERR_INVALID;
  }

  // ---- workspace layout ----
  pkv_workspace_layout& L = p.layout;
  L = pkv_workspace_layout{};
  int64_t off = 0;
  L.items_offset = off;
  off = align_up(off + (int64_t)p.items.size() * (int64_t)sizeof(Item), kAlign);
  L.meta_offset = off;
  const int64_t meta_end =
      off + (int64_t)p.meta.size() * (int64_t)sizeof(SeqMeta) + (int64_t)p.rows.size() * 4;
  off = align_up(meta_end, kAlign);
  L.counters_offset = off;
  const bool counters = mode != PKV_MODE_UNSPLIT && p.fused;
  const int64_t counters_end = off + (counters ? (int64_t)B * Hkv * PKV_COUNTER_STRIDE : 0);
  off = align_up(counters_end, kAlign);
  L.m_offset = off;
  off = align_up(off + num_slots * G * 4, kAlign);
  L.l_offset = off;
  off = align_up(off + num_slots * G * 4, kAlign);
  L.acc_offset = off;
  off = align_up(off + num_slots * G * d * 4, kAlign);
  L.total_bytes = (mode == PKV_MODE_UNSPLIT) ? 0 : off;
  L.num_items = (int32_t)p.items.size();
  L.num_slots = p.num_slots;
  L.group = G;
  L.num_splits = p.num_splits;

  // ---- counters ----
  const int64_t e = 2;  // fp16 / bf16
  p.algorithmic_bytes = kv_tokens * Hkv * d * 2 * e + 2 * (int64_t)B * s.num_q_heads * d * e +
                        total_pages * 4 + (int64_t)B * 4;
  p.partial_bytes = 2 * num_slots * G * (int64_t)(d + 2) * 4;
  // Upload image: [items | meta | zeroed counters]; nothing when no table
  // or counter is used.
  if (mode == PKV_MODE_UNSPLIT)
    p.upload_bytes = 0;
  else if (counters)
    p.upload_bytes = counters_end;
  else if (mode == PKV_MODE_WORKQUEUE || mode == PKV_MODE_BUCKETED)
    p.upload_bytes = meta_end;
  else
    p.upload_bytes = 0;
  // The same image in host memory the plan owns, for the entry point that
  // copies it into the library's own device scratch on every call (and
  // allocates nothing there).
  p.static_image.resize((size_t)p.upload_bytes);
  if (p.upload_bytes > 0) write_upload_image(p, p.static_image.data());
  p.uploaded = false;
  return PKV_OK;
}

}  // namespace

void write_upload_image(const pkv_plan& p, void* dst) {
  char* d = (char*)dst;
  std::memset(d, 0, (size_t)p.upload_bytes);
  if (!p.items.empty())
    std::memcpy(d + p.layout.items_offset, p.items.data(), p.items.size() * sizeof(Item));
  if (!p.meta.empty())
    std::memcpy(d + p.layout.meta_offset, p.meta.data(), p.meta.size() * sizeof(SeqMeta));
  if (!p.rows.empty())
    std::memcpy(d + p.layout.meta_offset + p.meta.size() * sizeof(SeqMeta), p.rows.data(),
                p.rows.size() * sizeof(int32_t));
}

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  try {
    g_error = buf;
  } catch (...) {  // out of host memory: the message is lost, nothing is thrown
    g_error.clear();
  }
}

void clear_error() { g_error.clear(); }

}  // namespace pkv

extern "C" {

pkv_status pkv_plan_create(const pkv_shape* shape, const int32_t* seq_lens_host,
                           const pkv_opts* opts, pkv_plan** out_plan) {
  pkv::clear_error();
  if (!out_plan) {
    pkv::set_error("out_plan is NULL");
    return PKV_ERR_INVALID;
  }
  *out_plan = nullptr;
  pkv_status st = pkv::validate(shape, seq_lens_host);
  if (st != PKV_OK) return st;
  pkv_plan* p = new (std::nothrow) pkv_plan();
  if (!p) {
    pkv::set_error("out of host memory");
    return PKV_ERR_INVALID;
  }
  p->shape = *shape;
  if (p->shape.sm_scale == 0.0f) p->shape.sm_scale = 1.0f / std::sqrt((float)shape->head_dim);
  if (opts) p->opts = *opts;
  p->group = shape->num_q_heads / shape->num_kv_heads;
  p->num_cus = p->opts.num_cus;
  if (p->num_cus <= 0) {
    st = pkv::query_num_cus(&p->num_cus);
    if (st != PKV_OK) {
      delete p;
      return st;
    }
  }
  try {  // host vectors grow here; no exception crosses the C ABI
    p->seq_lens.assign(seq_lens_host, seq_lens_host + shape->batch);
    st = pkv::build(*p);
  } catch (const std::bad_alloc&) {
    pkv::set_error("out of host memory");
    st = PKV_ERR_INVALID;
  }
  if (st != PKV_OK) {
    delete p;
    return st;
  }
  *out_plan = p;
  return PKV_OK;
}

pkv_status pkv_plan_update(pkv_plan* p, const int32_t* seq_lens_host) {
  pkv::clear_error();
  if (!p) {
    pkv::set_error("plan is NULL");
    return PKV_ERR_INVALID;
  }
  pkv_status st = pkv::validate(&p->shape, seq_lens_host);
  if (st != PKV_OK) return st;
  pkv::wait_upload(p);
  const bool was_uploaded = p->uploaded;
  p->uploaded = false;  // also after a failed re-plan: decode refuses until a new upload
  try {  // host vectors may grow here; no exception crosses the C ABI
    p->seq_lens.assign(seq_lens_host, seq_lens_host + p->shape.batch);
    st = pkv::build(*p);
  } catch (const std::bad_alloc&) {
    pkv::set_error("out of host memory");
    st = PKV_ERR_INVALID;
  }
  if (st != PKV_OK || !was_uploaded) return st;
  // The workspace still holds the previous image. When the new plan's image
  // is byte for byte the same (the usual case when no row gained or lost a
  // page: ranges are whole pages and the kernels read the exact lengths
  // from the device) and the workspace is large enough, the plan stays
  // uploaded and the next decode needs no copy.
  const int64_t nb = p->upload_bytes;
  if (nb != p->copied_bytes) return st;
  // The bound workspace must also serve the new plan: present, aligned and
  // large enough whenever the plan needs one. (A plan that needed none, such
  // as an unsplit one, may have been bound to anything or to nothing.)
  const int64_t need = p->layout.total_bytes;
  if (need > 0 && (!p->workspace || (uintptr_t)p->workspace % 256 != 0 ||
                   need > (int64_t)p->workspace_bytes))
    return st;
  // build() has just written the new image (static_image).
  if (nb > 0 && std::memcmp(p->static_image.data(), p->pinned, (size_t)nb) != 0) return st;
  p->uploaded = true;
  return st;
}

pkv_status pkv_plan_upload_needed(const pkv_plan* p, int32_t* needed) {
  pkv::clear_error();
  if (!p || !needed) {
    pkv::set_error("plan or needed is NULL");
    return PKV_ERR_INVALID;
  }
  *needed = p->uploaded ? 0 : 1;
  return PKV_OK;
}

size_t pkv_plan_workspace_bytes(const pkv_plan* p) {
  return p ? (size_t)p->layout.total_bytes : 0;
}

pkv_status pkv_plan_stats_get(const pkv_plan* p, pkv_plan_stats* s) {
  pkv::clear_error();
  if (!p || !s) {
    pkv::set_error("plan or stats is NULL");
    return PKV_ERR_INVALID;
  }
  *s = pkv_plan_stats{};
  s->mode = p->mode;
  s->num_splits = p->num_splits;
  s->chunk_pages = p->chunk_pages;
  s->grid = p->grid;
  s->num_items = p->num_items;
  s->empty_items = p->empty_items;
  s->num_slots = p->num_slots;
  const int32_t per = (p->mode == PKV_MODE_UNSPLIT || p->fused) ? 1 : 2;
  s->launches = p->mode == PKV_MODE_BUCKETED ? per * (int32_t)p->buckets.size() : per;
  s->bucket_launches = p->bucket_launches;
  s->kv_tokens = p->kv_tokens;
  s->algorithmic_bytes = p->algorithmic_bytes;
  s->partial_bytes = p->partial_bytes;
  s->upload_bytes = p->upload_bytes;
  s->workspace_bytes = p->layout.total_bytes;
  return PKV_OK;
}

pkv_status pkv_plan_layout_get(const pkv_plan* p, pkv_workspace_layout* l) {
  pkv::clear_error();
  if (!p || !l) {
    pkv::set_error("plan or layout is NULL");
    return PKV_ERR_INVALID;
  }
  *l = p->layout;
  return PKV_OK;
}

pkv_status pkv_plan_queue_get(const pkv_plan* p, void* dst, size_t bytes) {
  pkv::clear_error();
  if (!p) {
    pkv::set_error("plan is NULL");
    return PKV_ERR_INVALID;
  }
  const size_t need = (size_t)p->upload_bytes;
  if (need == 0) return PKV_OK;
  if (!dst || bytes < need) {
    pkv::set_error("queue image needs %zu bytes", need);
    return PKV_ERR_INVALID;
  }
  pkv::write_upload_image(*p, dst);
  return PKV_OK;
}

void pkv_plan_destroy(pkv_plan* p) {
  if (!p) return;
  pkv::release_device_resources(p);
  delete p;
}

const char* pkv_status_string(int32_t st) {
  switch (st) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID: return "PKV_ERR_INVALID";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_STATE: return "PKV_ERR_STATE";
    case PKV_ERR_POOL: return "PKV_ERR_POOL";
    default: return "PKV_ERR_UNKNOWN";
  }
}

const char* pkv_last_error(void) { return pkv::g_error.c_str(); }

int32_t pkv_version(void) { return 100; }

}  // extern "C"
