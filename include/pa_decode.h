/*
 * pa_decode.h — C ABI of the MI355X (gfx950) split-KV paged-attention decode
 * library (libpa.so).
 *
 * The operation (FlyDSL paged-attention decode pages: aiter PR #4332 "Add
 * paged-attention Tile kernel", host wrapper and its review; aiter PR #6617
 * "Extend packed D256 PA decode pipe", summary and validation; aiter PR #7079
 * "Merge gfx1250 PA decode partitions", partition merges and tests):
 *
 *   For sequence s, query row i in [0, QL), q-head h, KV head g = h / (Hq/Hkv):
 *     L = context_lens[s];  pos = L - QL + i (causal) or L - 1;
 *     visible tokens t: 0 <= t < L, t <= pos, and t > pos - W when W > 0;
 *     out[s*QL+i, h, :] = softmax_t(softmax_scale * q . k_t  [+ sink_h]) v_t
 *   with k_t, v_t dequantised from paged caches (FP8 code * scale, or BF16),
 *   a per-head sink logit joining the denominator only, and 0 for a row that
 *   sees no token.
 *
 * Split-KV: pa_plan divides each (sequence, KV head)'s visible tokens into
 * partitions sized to the device's compute-unit count; pa_decode runs one
 * launch over the work list and writes per-partition partial states (or the
 * final rows for a (sequence, KV head) with a single partition); pa_reduce
 * merges partials by the log-sum-exp rule, in partition order.
 *
 * Ownership: the caller allocates every device buffer (query, output, caches,
 * tables, scales, sinks, meta_dev, workspace_dev).  The library allocates only
 * the host plan object; it never allocates device memory and never
 * synchronises the host.  Status codes are returned, never exceptions; the
 * thread-local pa_last_error() explains the last non-OK status.
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* malformed arguments: shapes, nulls, alignment */
  PA_ERR_UNSUPPORTED = 2, /* valid but not implemented (layout/dtype/size) */
  PA_ERR_WORKSPACE = 3,   /* meta/workspace buffer missing or too small */
  PA_ERR_DEVICE = 4       /* a HIP runtime call failed */
} pa_status;

typedef enum { PA_BF16 = 0, PA_FP16 = 1, PA_FP8_E4M3FN = 2 } pa_dtype;
typedef enum { PA_V_PLAIN = 0, PA_V_TRANSPOSED = 1 } pa_v_layout;
typedef enum { PA_SCALE_NONE = 0, PA_SCALE_PER_TENSOR = 1, PA_SCALE_PER_TOKEN = 2 } pa_scale_mode;

/*
 * Problem statement.  Layouts (x = 16 bytes / KV element size: 16 for FP8,
 * 8 for BF16), all contiguous, row-major:
 *   q, out         [num_seqs*query_len, num_q_heads, head_dim]  (q_dtype)
 *   k_cache        [num_pages, num_kv_heads, head_dim/x, page_size, x]  (packed K)
 *   v_cache plain  [num_pages, num_kv_heads, head_dim, page_size]
 *   v_cache trans. [num_pages, num_kv_heads, page_size/x, head_dim, x]
 *   block_tables   int32 [num_seqs, table_stride]
 *   context_lens   int32 [num_seqs]
 *   k/v scales     float [1] (per tensor) or [num_pages, num_kv_heads, page_size]
 *   sinks          float [num_q_heads] (natural-log logits), or NULL
 * token_table = 1: block_tables[s][j] is a physical token slot
 *   (page * page_size + offset) of the j-th attended token and
 *   context_lens[s] counts them (sparse decode; query_len 1, no window).
 */
typedef struct {
  int32_t num_seqs, query_len, num_q_heads, num_kv_heads, head_dim, page_size;
  int32_t num_pages, table_stride;
  int32_t q_dtype;    /* pa_dtype: PA_BF16 or PA_FP16 */
  int32_t kv_dtype;   /* pa_dtype: PA_FP8_E4M3FN or PA_BF16 */
  int32_t v_layout;   /* pa_v_layout */
  int32_t scale_mode; /* pa_scale_mode; FP8 needs PER_TENSOR or PER_TOKEN, BF16 needs NONE */
  int32_t causal, sliding_window, has_sinks, token_table;
  float softmax_scale; /* <= 0: 1/sqrt(head_dim) */
} pa_problem;

typedef struct {
  int32_t cu_count;         /* 0: query the current device */
  int32_t max_partitions;   /* per (sequence, KV head); 0: cu_count, capped at 256 */
  int32_t partition_tokens; /* > 0: fixed partition length (rounded up to 128 tokens) */
  int32_t stage_limit;      /* page/slot ids staged in LDS per work item; 0: 1024 (max) */
  int32_t refreshable;      /* 1: a fixed budget of work items and partial slots (cu_count x resident
                               workgroups, at least one per (sequence, KV head, row group)) and one reduce
                               entry per such unit, so that pa_plan_refresh can re-partition the plan on
                               the device from device context lengths (e.g. between HIP graph replays) */
} pa_plan_opts;

typedef struct pa_plan_s pa_plan_t;

typedef struct {
  int32_t num_items;      /* work items = workgroups of one pa_decode launch */
  int32_t num_slots;      /* partial-state slots in the workspace */
  int32_t num_reduce;     /* (sequence, KV head, row group) entries pa_reduce merges */
  int32_t rows_per_group; /* query rows (QL*G, at most 64) one work item carries */
  int32_t row_groups;     /* row groups per (sequence, KV head) */
  int32_t max_parts;      /* largest partition count of any (sequence, KV head) */
  int32_t total_tiles;    /* 128-token tiles over all work items (planned lengths) */
  int32_t cu_count;       /* compute units the budget was sized for */
} pa_plan_info_t;

/*
 * Build a plan from host context lengths (planning reads only the host copy).
 * Partitions per (sequence, KV head) minimise the longest work item under a
 * budget of (cu_count x resident workgroups per CU) items; empty sequences
 * get one zero-length item that clears their rows.  Returns PA_ERR_INVALID /
 * PA_ERR_UNSUPPORTED for bad problems (see pa_decode), PA_ERR_DEVICE if
 * cu_count is 0 and no device can be queried.  *out is NULL on error.
 */
pa_status pa_plan(const pa_problem* problem, const int32_t* context_lens_host, const pa_plan_opts* opts,
                  pa_plan_t** out);

/* Device bytes the caller must provide: meta_dev (work list, reduce table)
 * and workspace_dev (FP32 partial states).  Either may be 0 bytes. */
pa_status pa_plan_sizes(const pa_plan_t* plan, size_t* meta_bytes, size_t* workspace_bytes);

/* Summary counts of a plan (host only). */
pa_status pa_plan_info(const pa_plan_t* plan, pa_plan_info_t* info);

/* Copy the host work list: 8 int32 per item
 * {seq, kv_head, row_group, tile_begin, tile_end(-1: to the end), slot(-1: direct output), part, nparts},
 * tiles being 128-token blocks from the page-aligned start of the visible span.
 * n_items_capacity limits the copy; returns PA_ERR_INVALID if too small. */
pa_status pa_plan_work(const pa_plan_t* plan, int32_t* out, int32_t n_items_capacity);

void pa_plan_free(pa_plan_t* plan);

/*
 * One launch: every work item of the plan.  Writes partial states to
 * workspace_dev for multi-partition (sequence, KV head) pairs and the final
 * rows of `out` for the others (including cleared rows of empty sequences).
 * The plan metadata is copied to meta_dev on `stream` when meta_dev differs
 * from the last upload.  `stream` is a hipStream_t (NULL: default stream).
 * Device context_lens are authoritative: a sequence longer than planned is
 * still fully processed (its last partition runs to the end, reading page ids
 * past the staged range from the block table directly).
 * Errors: PA_ERR_INVALID for null or misaligned (16 B) pointers,
 * PA_ERR_WORKSPACE for missing meta/workspace, PA_ERR_DEVICE for launch errors.
 */
pa_status pa_decode(const pa_plan_t* plan, void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, const float* k_scale,
                    const float* v_scale, const float* sinks, void* meta_dev, void* workspace_dev, void* stream);

/*
 * Merge the partial states of every multi-partition (sequence, KV head) into
 * `out` (log-sum-exp in partition order; sinks join the denominator; a row
 * with no visible token gets 0).  At most one launch; none if the plan has no
 * multi-partition pair.  Must follow pa_decode of the same plan on the same
 * stream.  A plan with its meta/workspace must not serve two in-flight calls.
 */
pa_status pa_reduce(const pa_plan_t* plan, void* out, const float* sinks, void* meta_dev, void* workspace_dev,
                    void* stream);

/*
 * Re-partition a refreshable plan on the device from the device context
 * lengths (one single-workgroup launch on `stream`, no host synchronisation,
 * no allocation, no host-to-device copy: it can be captured in a HIP graph
 * in front of pa_decode and pa_reduce).  Partition counts follow the host
 * planner's rule (the CU-count budget of aiter PR #4332, "Add paged-attention
 * Tile kernel", work plans): the smallest longest-item length M whose
 * partitions (ceil(tiles / M) per (sequence, KV head, row group), at most
 * max_partitions and at most one per tile) fit the plan's item and slot
 * budget, with each unit's tiles split evenly.  The work list and reduce
 * table in meta_dev are rewritten in full (unused items do nothing); the
 * plan's host copy is not changed, and later pa_decode calls with this
 * meta_dev use the refreshed list.  Must precede pa_decode on the same
 * stream.  Errors: PA_ERR_INVALID for a NULL pointer or a plan made without
 * `refreshable`, PA_ERR_DEVICE for a launch error.
 */
pa_status pa_plan_refresh(const pa_plan_t* plan, const int32_t* context_lens, void* meta_dev, void* stream);

/* Thread-local message for the last non-OK status of this thread. */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
