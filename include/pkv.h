/*
 * pkv.h -- C ABI of a paged grouped-query-attention (GQA) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * One decode step: every sequence b contributes one query token per query
 * head; it attends over the N_b tokens already in a paged KV cache. The cache
 * is read in place through a block table, never repacked (PersistentKV
 * explainer, Technical summary > Methodology 1, layout). Query heads are
 * grouped: G = Hq / Hkv query heads share one KV head, head h reading KV head
 * h / G (same section, the GQA definition).
 *
 * The step is planned on the host and run by hand-written HIP kernels:
 *
 *   pkv_plan_create / pkv_plan_update   host, integer only: pick the mode
 *       (unsplit, split-S, work queue), cut each (sequence, KV head) into
 *       page-aligned ranges from the real per-row lengths, and build the
 *       compact work queue (Methodology 1, sequence splitting, row-local
 *       bounds, compact workqueue; Methodology 2, calibrated policy).
 *   pkv_plan_upload    binds the caller's workspace and copies the queue.
 *   pkv_decode         launches the partial kernel (one workgroup per range;
 *       each writes a partial online-softmax state (m, l, acc) or, unsplit,
 *       the output) and, when ranges were split, the merge kernel that
 *       combines the states exactly.
 *
 * Data layouts (all device memory, row-major, owned by the caller):
 *   q, out        [B, Hq, d]                 dtype (fp16 or bf16)
 *   k_pool,v_pool [num_pages, Hkv, P, d]     dtype; P = 16 tokens per page.
 *                 One (page, KV head) tile is P*d contiguous elements.
 *   block_table   int32 [B, block_table_stride]; entry j of row b is the
 *                 physical page holding logical tokens [j*P, (j+1)*P) of
 *                 sequence b (LLM Primer ch. 8, section 8.1). Entries at or
 *                 beyond ceil(N_b / P) never affect the result (they may be
 *                 loaded, never past the row's block_table_stride entries).
 *   seq_lens      int32 [B]; N_b >= 0. Must hold the same values as the host
 *                 array the plan was built from.
 * Tail slots of a sequence's last page (t >= N_b) may hold anything,
 * including NaN: they never reach the arithmetic.
 *
 * Numerics: products and sums in fp32; out = acc / l rounded to nearest even
 * in the storage dtype. sm_scale multiplies q.k before the softmax.
 *
 * Errors: every call returns a pkv_status; nothing aborts and no C++
 * exception crosses the ABI. pkv_last_error() gives a thread-local message
 * for the last failing call on the calling thread.
 *
 * Threading and streams: plans are host objects, not internally locked; use
 * one plan from one thread at a time. pkv_decode is asynchronous on the
 * caller's stream and does not synchronise. Decodes of different plans with
 * different workspaces may overlap; two decodes sharing one workspace must be
 * ordered by the caller (the same stream does that).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,     /* bad argument: null, negative, inconsistent */
  PKV_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, G, page size */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned */
  PKV_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  PKV_ERR_STATE = -5,       /* call out of order (e.g. decode before upload) */
  PKV_ERR_POOL = -6         /* page pool exhausted (nothing was taken) */
} pkv_status;

/* Storage dtype shared by q, the K/V pools and out. */
typedef enum pkv_dtype { PKV_F16 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Dispatch modes (PersistentKV explainer, Methodology 2: the policy routes a
 * step to one of several execution paths by batch size and length).
 *   UNSPLIT    one workgroup per (sequence, KV head); writes out; 1 launch.
 *   SPLIT      rectangular grid S x Hkv x B (x, y, z); row b uses
 *              chunk_b = ceil(pages_b / S) pages per range; cells past the
 *              row's last range write a neutral state; partial + merge.
 *   WORKQUEUE  1-D grid over the non-empty (sequence, KV head, range) items
 *              only, every range chunk_pages pages long (the last one of a
 *              row shorter); partial + merge.
 *   AUTO       the calibrated policy picks one of the three.
 *   BUCKETED   comparator, never chosen by AUTO: exact-length bucketing
 *              (PersistentKV explainer, Methodology 1 and Results, the
 *              launch fan-out the compact work queue avoids). The rows of
 *              each distinct N_b form a bucket planned as if it ran alone
 *              (ranges sized so that the bucket's items fill the CUs), with
 *              a partial launch of its own and, with PKV_MERGE_KERNEL, a
 *              merge launch of its own; empty rows form one more bucket
 *              that only writes zeros. Same results as WORKQUEUE up to the
 *              split points; meant for the ablation counters and timings. */
typedef enum pkv_mode {
  PKV_MODE_AUTO = 0,
  PKV_MODE_UNSPLIT = 1,
  PKV_MODE_SPLIT = 2,
  PKV_MODE_WORKQUEUE = 3,
  PKV_MODE_BUCKETED = 4
} pkv_mode;

/* How split states are merged (SPLIT and WORKQUEUE modes).
 *   FUSED   the partial kernel's last-arriving workgroup of each
 *           (sequence, KV head) merges that row's states and writes out:
 *           one launch per step.
 *   KERNEL  a separate merge kernel runs after the partial kernel: two
 *           launches per step (the pages' design).
 * Both merge the states in split-index order and give identical bits. */
typedef enum pkv_merge { PKV_MERGE_FUSED = 0, PKV_MERGE_KERNEL = 1 } pkv_merge;

/* Problem shape. Supported: page_size 16; head_dim 64 or 128;
 * G = num_q_heads / num_kv_heads in {1, 2, 4, 8}. */
typedef struct pkv_shape {
  int32_t batch;              /* B >= 0 */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;           /* d */
  int32_t page_size;          /* P, tokens per page */
  int32_t block_table_stride; /* int32 entries per block_table row */
  int64_t num_pages;          /* pool capacity in pages (both pools) */
  int32_t dtype;              /* pkv_dtype */
  float sm_scale;             /* softmax scale; 0 selects 1/sqrt(d) */
} pkv_shape;

/* Planning options; zero-initialised means "automatic" everywhere. */
typedef struct pkv_opts {
  int32_t mode;        /* pkv_mode */
  int32_t num_splits;  /* SPLIT: S (0 = policy's choice) */
  int32_t chunk_pages; /* WORKQUEUE: pages per range (0 = policy's choice) */
  int32_t num_cus;     /* compute units to plan for (0 = ask the device) */
  uint32_t queue_seed; /* 0: longest ranges first; else a seeded shuffle of
                          the queue (results do not depend on queue order) */
  int32_t merge;       /* pkv_merge */
  int32_t reserved[2];
} pkv_opts;

/* Scheduler-derived counters of one planned step (PersistentKV explainer,
 * Technical summary > Results: launch fan-out and merge-state traffic). */
typedef struct pkv_plan_stats {
  int32_t mode;            /* resolved pkv_mode (never AUTO) */
  int32_t num_splits;      /* S: most ranges any (sequence, KV head) has */
  int32_t chunk_pages;     /* pages per range (SPLIT: the largest row's) */
  int32_t grid;            /* partial-kernel workgroups launched */
  int32_t num_items;       /* launched workgroups that read KV */
  int32_t empty_items;     /* launched workgroups that read no KV: SPLIT
                              cells past a row's end (neutral state), or,
                              with the fused merge, one zero-fill item per
                              KV head of an empty row (WORKQUEUE, slot -1) */
  int32_t num_slots;       /* partial states written and merged */
  int32_t launches;        /* kernel launches per step: 1 (unsplit, or
                              fused merge) or 2 (separate merge kernel);
                              BUCKETED: that many per bucket */
  int32_t bucket_launches; /* launches exact-length bucketing would issue:
                              one partial + one merge per distinct N_b > 0 */
  int32_t reserved;
  int64_t kv_tokens;         /* sum of N_b */
  int64_t algorithmic_bytes; /* K/V of the N_b tokens + q + out + used
                                block-table entries + seq_lens */
  int64_t partial_bytes;     /* merge-state traffic: bytes of (m, l, acc)
                                written by the partial kernel + read by the
                                merge kernel */
  int64_t upload_bytes;      /* host-to-device bytes per step: the queue,
                                the per-row table and the zeroed merge
                                counters */
  int64_t workspace_bytes;   /* what pkv_plan_workspace_bytes returns */
} pkv_plan_stats;

/* Where the partial states sit in the workspace, for inspection in tests.
 * Slot of (b, g, s): WORKQUEUE, BUCKETED  slot_base[b] + g * S_b + s, with
 * (slot_base[b], S_b) the int32 pair at meta_offset + 8*b;
 * SPLIT  (b * Hkv + g) * S + s. Per slot: m_log2[G] (the reference maximum,
 * in log2 units of the scaled logits: m_log2 = m * log2(e)), l[G] and
 * acc[G][d], all fp32; the state is (m, l, acc) with l = sum exp(x - m) and
 * acc = sum exp(x - m) v over the range; a neutral state is
 * (-inf, 0, 0). m need not be the range's exact maximum: any reference at
 * or above it by a bounded amount represents the same state. */
/* Bytes between two rows' merge counters in the workspace: each counter has
 * its own 128-byte cache line, so that the workgroups of different rows do
 * not queue behind each other's atomic increments. */
#define PKV_COUNTER_STRIDE 128

typedef struct pkv_workspace_layout {
  int64_t items_offset;  /* int32x8 {b*Hkv+g, page_begin, page_end, slot,
                            row_base, row_count, b, g}: row_base / row_count
                            are the first slot and the range count of
                            (b, g); a zero-fill item has slot -1 */
  int64_t meta_offset;   /* int32x2 per sequence (WORKQUEUE, BUCKETED);
                            BUCKETED: then int32 per sequence, the rows of
                            the buckets one bucket after another */
  int64_t counters_offset; /* int32 per (sequence, KV head), PKV_COUNTER_STRIDE
                              bytes apart: arrivals of the current step
                              (fused merge); 0 between steps */
  int64_t m_offset;      /* fp32 [num_slots][G] */
  int64_t l_offset;      /* fp32 [num_slots][G] */
  int64_t acc_offset;    /* fp32 [num_slots][G][d] */
  int64_t total_bytes;
  int32_t num_items;
  int32_t num_slots;
  int32_t group;         /* G */
  int32_t num_splits;    /* S */
} pkv_workspace_layout;

typedef struct pkv_plan pkv_plan; /* opaque; host-owned */

/* Build a plan for one decode step.
 *   shape          problem shape (copied).
 *   seq_lens_host  int32[batch] host array of N_b (copied; may be NULL when
 *                  batch == 0).
 *   opts           may be NULL (all automatic).
 *   out_plan       receives the new plan; *out_plan is NULL on failure.
 * Errors: PKV_ERR_INVALID for null pointers, negative sizes, Hq % Hkv != 0,
 * N_b < 0 or N_b > block_table_stride * page_size; PKV_ERR_UNSUPPORTED for a
 * page size, head_dim, G or dtype this build has no kernel for, and for
 * PKV_MODE_SPLIT with batch or num_kv_heads above 65535 (grid dimensions;
 * AUTO then picks the work queue); PKV_ERR_HIP if num_cus is 0 and the
 * device cannot be queried. Host-only: calls no HIP
 * function unless num_cus is 0. */
pkv_status pkv_plan_create(const pkv_shape* shape, const int32_t* seq_lens_host,
                           const pkv_opts* opts, pkv_plan** out_plan);

/* Re-plan in place for the next step (same shape and options, new lengths);
 * reuses the plan's host buffers. Waits for the plan's previous upload copy
 * to leave its pinned staging buffer. The plan must be uploaded again before
 * the next decode, unless pkv_plan_upload_needed reports otherwise: when the
 * plan was uploaded and the new queue image is byte for byte the one its
 * last upload copied (typically when no row gained or lost a page: ranges
 * are whole pages, and the kernels read the exact lengths from the device
 * seq_lens) and the bound workspace is large enough, the plan stays
 * uploaded. Errors as pkv_plan_create. (Serving re-forms the batch every
 * step: ai-trend study note, "How it works", step four.) */
pkv_status pkv_plan_update(pkv_plan* plan, const int32_t* seq_lens_host);

/* *needed = 1 if the next decode needs pkv_plan_upload first (never
 * uploaded, or the last pkv_plan_update changed the queue image or outgrew
 * the workspace), 0 if the workspace bound by the last upload already holds
 * the plan's image (valid for decodes ordered after that upload's copy, and
 * while the caller leaves the workspace untouched). Host-only, no HIP call.
 * For callers that re-plan every step: skipping the copy saves a
 * host-to-device transfer per step. Errors: PKV_ERR_INVALID for NULL. */
pkv_status pkv_plan_upload_needed(const pkv_plan* plan, int32_t* needed);

/* Device workspace the plan needs (bytes, 0 for UNSPLIT). */
size_t pkv_plan_workspace_bytes(const pkv_plan* plan);

/* Bind a caller-owned device workspace of at least
 * pkv_plan_workspace_bytes() bytes (256-byte aligned) and enqueue the copy of
 * the work queue into it on `stream`. The workspace must stay allocated
 * until every decode that uses it has finished on the device. Errors:
 * PKV_ERR_WORKSPACE (null when needed, too small, misaligned), PKV_ERR_HIP. */
pkv_status pkv_plan_upload(pkv_plan* plan, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Copy the plan's counters. */
pkv_status pkv_plan_stats_get(const pkv_plan* plan, pkv_plan_stats* stats);

/* Describe where the partial states live in the workspace. */
pkv_status pkv_plan_layout_get(const pkv_plan* plan,
                               pkv_workspace_layout* layout);

/* Copy the host image of what pkv_plan_upload sends (upload_bytes of
 * pkv_plan_stats): the work-queue items (int32x8
 * {b*Hkv+g, page_begin, page_end, slot, row_base, row_count, 0, 0} at
 * items_offset), the per-sequence
 * (slot_base, S_b) pairs at meta_offset and the zeroed merge counters at
 * counters_offset, laid out exactly as in the workspace. `bytes` must be at
 * least upload_bytes (0 is fine when the plan uploads nothing). */
pkv_status pkv_plan_queue_get(const pkv_plan* plan, void* dst, size_t bytes);

/* Run one decode step on `stream` (asynchronous).
 *   q, k_pool, v_pool, out: device pointers, 16-byte aligned, layouts above.
 *   block_table, seq_lens:  device int32 arrays, 4-byte aligned.
 * Block-table entries are not trusted blindly: a page index outside
 * [0, num_pages) contributes no tokens instead of being read.
 * Errors: PKV_ERR_INVALID (null or misaligned pointer), PKV_ERR_STATE (plan
 * not uploaded), PKV_ERR_HIP (launch failure). */
pkv_status pkv_decode(const pkv_plan* plan, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table,
                      const int32_t* seq_lens, void* out, hipStream_t stream);

/* pkv_decode with timing marks: records `before` ahead of the partial
 * kernel, `after_partial` after it and `after_merge` after the merge kernel
 * (or after the partial kernel when there is no merge), each on `stream`.
 * Any event may be NULL. Used to time the partial kernel on its own stream. */
pkv_status pkv_decode_marked(const pkv_plan* plan, const void* q,
                             const void* k_pool, const void* v_pool,
                             const int32_t* block_table,
                             const int32_t* seq_lens, void* out,
                             hipStream_t stream, hipEvent_t before,
                             hipEvent_t after_partial, hipEvent_t after_merge);

/* Free a plan (NULL is a no-op). Waits for its last upload copy. */
void pkv_plan_destroy(pkv_plan* plan);

/* ---------------------------------------------------------------------------
 * Paged KV append: the step before decode. Each sequence keeps its cache in
 * fixed-size pages of one shared pool; a sequence takes a new page from the
 * pool when its tail page is full, and a finished sequence's pages go back
 * to the pool at once, for other sequences to reuse (ZimaSpace post, on
 * fixed-size blocks and on blocks released when a request ends; ai-trend
 * study note, "How it works", steps two and four). The token at logical
 * position t of sequence b lives at (block_table[b][t / P], g, t % P).
 * ------------------------------------------------------------------------- */

typedef struct pkv_pool pkv_pool; /* opaque host-side page allocator */

/* A free list over pool pages 0 .. num_pages-1, all free at creation; pages
 * are handed out lowest index first, and freed pages are reused first (last
 * in, first out). Host only. Errors: PKV_ERR_INVALID (num_pages <= 0, null). */
pkv_status pkv_pool_create(int32_t num_pages, pkv_pool** out_pool);

/* Free the allocator (NULL is a no-op). */
void pkv_pool_destroy(pkv_pool* pool);

/* Pages currently free (-1 for a NULL pool). */
int32_t pkv_pool_free_pages(const pkv_pool* pool);

/* Take n pages into pages[0 .. n-1]. Errors: PKV_ERR_POOL when fewer than n
 * are free (nothing taken), PKV_ERR_INVALID (n < 0, null). */
pkv_status pkv_pool_alloc(pkv_pool* pool, int32_t n, int32_t* pages);

/* Return n pages. Errors: PKV_ERR_INVALID, with nothing returned, if a page
 * is outside the pool, not currently taken, or listed twice. */
pkv_status pkv_pool_free(pkv_pool* pool, const int32_t* pages, int32_t n);

/* Host half of one append step for a batch: row b's new token goes to
 * position N_b = seq_lens_host[b]; a row whose position opens a page
 * (N_b % page_size == 0) takes a page from the pool into
 * block_table_host[b * stride + N_b / page_size]. *pages_taken (may be NULL)
 * receives how many pages were taken. Errors: PKV_ERR_INVALID (null, N_b < 0,
 * position past the table row: N_b >= stride * page_size); PKV_ERR_POOL
 * (pool exhausted). On any error nothing is taken and the table is
 * unchanged. */
pkv_status pkv_append_prepare(pkv_pool* pool, int32_t batch, int32_t block_table_stride,
                              int32_t page_size, const int32_t* seq_lens_host,
                              int32_t* block_table_host, int32_t* pages_taken);

/* A sequence has finished: return the pages of its first
 * ceil(seq_len / page_size) table entries to the pool and set those entries
 * to -1. Errors as pkv_pool_free (then nothing is returned and the row is
 * unchanged). Pages shared with another row must not be released while that
 * row still uses them (the allocator keeps no reference counts). */
pkv_status pkv_pool_release_row(pkv_pool* pool, int32_t* block_table_row, int32_t seq_len,
                                int32_t page_size);

/* Device half: write every row's new token on `stream` (asynchronous).
 *   shape        batch, num_kv_heads, head_dim, page_size,
 *                block_table_stride, num_pages and dtype are used.
 *   k_new, v_new device [batch, Hkv, d] in the shape's dtype, 4-byte aligned.
 *   k_pool, v_pool  device [num_pages, Hkv, page_size, d].
 *   block_table  device int32 [batch, stride]; seq_lens device int32 [batch]:
 *                each row's position (its length before the append).
 *   new_seq_lens device int32 [batch] or NULL: receives seq_lens[b] + 1; it
 *                must not alias seq_lens.
 * A row whose position is negative or past the table row, or whose page
 * entry is outside [0, num_pages), writes no K/V (new_seq_lens still gets
 * seq_lens[b] + 1). Errors: PKV_ERR_INVALID (null or misaligned pointer, bad
 * shape), PKV_ERR_UNSUPPORTED (head_dim, page size, dtype), PKV_ERR_HIP. */
pkv_status pkv_append(const pkv_shape* shape, const void* k_new, const void* v_new,
                      void* k_pool, void* v_pool, const int32_t* block_table,
                      const int32_t* seq_lens, int32_t* new_seq_lens, hipStream_t stream);

/* pkv_append and pkv_decode in one launch (ZimaSpace post and ai-trend study
 * note, "How it works": a step first places the new token's K/V through the
 * block table, then decode reads the cache through it). Row b's new token
 * (k_new / v_new as in pkv_append, 16-byte aligned) goes to position
 * seq_lens[b], and the step attends over seq_lens[b] + 1 tokens, so `plan`
 * must have been built (and uploaded) for the lengths seq_lens[b] + 1 and
 * its page must already be in the table (pkv_append_prepare). The token's
 * page is read by no other row in the step (a page shared with another row
 * must not receive the token). k_pool / v_pool are written only at the new
 * tokens' slots; new_seq_lens (or NULL, never aliasing seq_lens) receives
 * seq_lens[b] + 1. The outputs and the pools after the call equal those of
 * pkv_append followed by pkv_decode bit for bit. Errors: those of
 * pkv_decode, and PKV_ERR_INVALID for a null or misaligned k_new / v_new
 * or an aliased new_seq_lens. */
pkv_status pkv_decode_append(const pkv_plan* plan, const void* q, const void* k_new,
                             const void* v_new, void* k_pool, void* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int32_t* new_seq_lens, void* out, hipStream_t stream);

/* pkv_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, with the plan's workspace in the library's own
 * device scratch instead of a caller-bound one. Each call copies the plan's
 * queue image and zeroed merge counters (host memory the plan owns, built
 * by pkv_plan_create / pkv_plan_update) into the scratch on `stream`, then
 * launches exactly as pkv_decode. No pkv_plan_upload is needed; the call
 * makes no device or pinned-host allocation of any kind.
 * Limit: the plan's pkv_plan_workspace_bytes must be at most
 * PKV_STATIC_SCRATCH_BYTES (16 MiB: every configuration up to 64 sequences
 * of 131072 tokens at G = 8); larger plans get PKV_ERR_WORKSPACE. The
 * scratch is one array per device, held until the process ends and shared
 * by every call on that device, which keeps the last call's contents:
 * calls that overlap on one device (other streams, other threads) race,
 * so order them (one stream does). Errors: those of pkv_decode, and
 * PKV_ERR_WORKSPACE as above. */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
pkv_status pkv_decode_static(const pkv_plan* plan, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* out, hipStream_t stream);

/* Measurement aid: one plain streaming read of bytes_each bytes from each of
 * the device buffers a and b (16-byte aligned, bytes_each a multiple of 16),
 * grid workgroups of 256 lanes, nontemporal 16-byte loads, asynchronous on
 * `stream`. Timed on the decode's K/V bytes it gives the HBM ceiling a
 * single read of that many bytes reaches on the device. `sink` is a device
 * word (4-byte aligned) the kernel may write. Errors: PKV_ERR_INVALID,
 * PKV_ERR_HIP. */
pkv_status pkv_stream_read(const void* a, const void* b, int64_t bytes_each, int32_t grid,
                           void* sink, hipStream_t stream);

/* Measurement aid: read every K and V tile that pkv_decode with this plan
 * reads (each item's pages of its (sequence, KV head) row through the block
 * table: PersistentKV explainer, Methodology 1), with the partial kernel's
 * grid and work split and the same kind of load path (nontemporal 16-byte
 * direct-to-LDS loads, a two-slot ring per wave), asynchronous on `stream`,
 * and fold the data into a check word: no q, softmax, state or merge. Timed
 * beside pkv_decode it gives the cost of the paged gather alone. Arguments
 * as pkv_decode (k_pool/v_pool 16-byte, block_table/seq_lens 4-byte aligned
 * device pointers); `sink` is a device word (4-byte aligned) the kernel may
 * write. A work-queue plan must be uploaded. Errors: PKV_ERR_INVALID (null
 * or misaligned pointer), PKV_ERR_STATE (work queue not uploaded),
 * PKV_ERR_UNSUPPORTED (PKV_MODE_BUCKETED, head_dim other than 64 or 128),
 * PKV_ERR_HIP. */
pkv_status pkv_paged_read(const pkv_plan* plan, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const int32_t* seq_lens, void* sink,
                          hipStream_t stream);

/* Static string naming a status code. */
const char* pkv_status_string(int32_t status);

/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
