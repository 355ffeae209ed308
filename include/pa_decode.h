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
 *   with k_t, v_t dequantised from paged caches (FP8 code * scale, MXFP4
 *   code * the power-of-two scale of its 32-element block, or BF16),
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
 * the host plan object and its pinned host copy of the metadata; it never
 * allocates device memory and never synchronises the host.  Status codes are
 * returned, never exceptions; the thread-local pa_last_error() explains the
 * last non-OK status.
 *
 * Call order: pa_plan, pa_plan_sizes, (allocate meta_dev and workspace_dev),
 * pa_plan_upload once, then pa_decode + pa_reduce per step (optionally
 * preceded by pa_plan_refresh for a refreshable plan).
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

typedef enum { PA_BF16 = 0, PA_FP16 = 1, PA_FP8_E4M3FN = 2, PA_MXFP4 = 3 } pa_dtype;
typedef enum { PA_V_PLAIN = 0, PA_V_TRANSPOSED = 1 } pa_v_layout;
typedef enum { PA_SCALE_NONE = 0, PA_SCALE_PER_TENSOR = 1, PA_SCALE_PER_TOKEN = 2, PA_SCALE_MX = 3 } pa_scale_mode;

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
 * token_table = 2: the two-level sparse front end (pa_decode_sparse): row s
 *   attends the logical positions topk[s][0..count_s) of its paged context,
 *   each resolved through block_tables[s] (page = block_tables[s][P / page],
 *   slot = P % page); positions outside [0, table_stride * page_size) are
 *   clamped to it (never read outside the row; such a position attends the
 *   clamped token).  query_len 1, no window.
 * MXFP4 caches (kv_dtype PA_MXFP4, scale_mode PA_SCALE_MX; aiter PR #7079,
 *   merge of #7056, names MXFP4 K/V and its 256-token partitions; the format
 *   is OCP microscaling FP4): every token's K and V row is cut into blocks
 *   of 32 head dims, each of 32 E2M1 codes and one E8M0 scale byte e
 *   (element = code value * 2^(e - 127)); two codes share a byte, the lower
 *   index in the low nibble.
 *     k_cache  uint8 [num_pages, num_kv_heads, head_dim/32, page_size, 16]
 *     v_cache  uint8 [num_pages, num_kv_heads, head_dim, page_size/2]
 *              (row d: the page's tokens in order, two per byte)
 *     k/v scales uint8 [num_pages, num_kv_heads, page_size, head_dim/32],
 *              passed through the k_scale / v_scale pointers, 16-byte
 *              aligned; a scale byte 0xFF (NaN) of a visible token gives
 *              unspecified results.
 *   head_dim 128, page_size 32, 64 or 128, page tables (token_table 0),
 *   v_layout PA_V_PLAIN; partitions are cut at multiples of 256 tokens of
 *   the visible span (pa_plan_opts.partition_tokens 0 or 256); plans are
 *   not refreshable.
 * Built configurations (others: PA_ERR_UNSUPPORTED): head_dim 64, 128,
 * 256 or 512; page_size a power of two from 16 to 1024 (token tables: at
 * most 128; pages above 128 tokens are read as 128-token sub-pages); FP8
 * e4m3fn caches with a per-tensor or per-token scale at any of those head
 * dims (512: page tables only, token_table = 0), BF16 caches (no scale,
 * BF16 queries) at head_dim 64 or 128.
 */
typedef struct {
  int32_t num_seqs, query_len, num_q_heads, num_kv_heads, head_dim, page_size;
  int32_t num_pages, table_stride;
  int32_t q_dtype;    /* pa_dtype: PA_BF16 or PA_FP16 */
  int32_t kv_dtype;   /* pa_dtype: PA_FP8_E4M3FN, PA_BF16 or PA_MXFP4 */
  int32_t v_layout;   /* pa_v_layout */
  int32_t scale_mode; /* pa_scale_mode; FP8 needs PER_TENSOR or PER_TOKEN, BF16 NONE, MXFP4 MX */
  int32_t causal, sliding_window, has_sinks, token_table;
  float softmax_scale;  /* <= 0: 1/sqrt(head_dim) */
  int32_t index_stride; /* token_table = 2: row stride of the top-k index table (pa_decode_sparse) */
} pa_problem;

typedef struct {
  int32_t cu_count;         /* 0: query the current device */
  int32_t max_partitions;   /* per (sequence, KV head); 0: cu_count, capped at 256 */
  int32_t partition_tokens; /* > 0: fixed partition length (rounded up to 128 tokens) */
  int32_t stage_limit;      /* page/slot ids staged in LDS per work item; 0: 1024 (max; the rest of an
                               item's ids are read from the block table with scalar loads).  1024 ids
                               (4 KB) keep two 16-row workgroups within one CU's 160 KB of LDS; the
                               pages' 4096 would not */
  int32_t refreshable;      /* 1: a fixed budget of work items and partial slots (cu_count x resident
                               workgroups, at least one per (sequence, KV head, row group)) and one reduce
                               entry per such unit, so that pa_plan_refresh can re-partition the plan on
                               the device from device context lengths (e.g. between HIP graph replays) */
  int32_t merge;            /* how multi-partition units are merged: 0 the library's choice (the reducer:
                               on gfx950 the agent-scope L2 write-back each arriving item needs makes the
                               in-kernel merge slower on every multi-partition shape measured), 1 the
                               reducer launch (pa_reduce), 2 in the decode launch (aiter PR #7079,
                               "Partition merges": the last-arriving work item of a unit merges its
                               partials, counted on per-unit arrival counters in meta_dev that every call
                               leaves at zero; pa_reduce then does nothing; calls that overlap on one
                               meta_dev race on the counters).  Both give bit-identical outputs */
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
 * The split-KV work plan of aiter PR #4332 "Add paged-attention Tile kernel"
 * (work plans and the commit that defaults the per-sequence partition limit
 * to the CU count): partitions per (sequence, KV head, row group of up to 64
 * query rows) minimise the longest work item under a budget of (cu_count x
 * resident workgroups per CU) items, at most max_partitions (default: the CU
 * count, capped at 256) each, over the 128-token tiles of the union of what
 * the sequence's query rows can see (window and causal MTP rows, aiter PR
 * #6617 "Extend packed D256 PA decode pipe", summary); empty sequences get
 * one zero-length item that clears their rows (aiter PR #7079 "Merge gfx1250
 * PA decode partitions", Partition merges).  Returns PA_ERR_INVALID /
 * PA_ERR_UNSUPPORTED for bad problems (see pa_decode), PA_ERR_DEVICE if
 * cu_count is 0 and no device can be queried.  *out is NULL on error.  The
 * plan is a host object owned by the caller (pa_plan_free).
 */
pa_status pa_plan(const pa_problem* problem, const int32_t* context_lens_host, const pa_plan_opts* opts,
                  pa_plan_t** out);

/* Device bytes the caller must provide: meta_dev (a 32-byte header, the work
 * list and the reduce table; at least 32 bytes) and workspace_dev (FP32
 * partial states; may be 0 bytes). */
pa_status pa_plan_sizes(const pa_plan_t* plan, size_t* meta_bytes, size_t* workspace_bytes);

/* Summary counts of a plan (host only). */
pa_status pa_plan_info(const pa_plan_t* plan, pa_plan_info_t* info);

/* Copy the host work list: 8 int32 per item
 * {seq, kv_head, row_group, tile_begin, tile_end(-1: to the end), slot(-1: direct output), part, nparts},
 * tiles being 128-token blocks from the page-aligned start of the visible span.
 * n_items_capacity limits the copy; returns PA_ERR_INVALID if too small. */
pa_status pa_plan_work(const pa_plan_t* plan, int32_t* out, int32_t n_items_capacity);

/*
 * Copy the plan's metadata (header, work list, reduce table: meta_bytes of
 * pa_plan_sizes) into the caller's device buffer meta_dev with one
 * asynchronous copy on `stream`, from a pinned host copy that the first call
 * allocates and pa_plan_free releases.  Required once per (plan, buffer)
 * before pa_decode / pa_reduce use the buffer, and again whenever the buffer
 * has held another plan's list (pa_decode and pa_reduce return
 * PA_ERR_WORKSPACE for a buffer whose last upload or refresh was another
 * plan's).  The header carries a per-plan serial that every kernel checks:
 * a buffer reallocated or overwritten after its upload makes the kernels do
 * nothing (the output is left untouched) instead of following a foreign
 * list.  Errors: PA_ERR_INVALID (NULL plan, meta_dev not 16-byte aligned),
 * PA_ERR_WORKSPACE (NULL meta_dev), PA_ERR_DEVICE (pinned allocation or copy
 * failed).
 */
pa_status pa_plan_upload(const pa_plan_t* plan, void* meta_dev, void* stream);

void pa_plan_free(pa_plan_t* plan);

/*
 * One launch over every work item of the plan: the decode of aiter PR #4332
 * "Add paged-attention Tile kernel" (host wrapper: query, paged caches,
 * block tables, context lengths, scales; partials pmax / psum / pout for
 * split-KV): page-id staging, K/V page gather, QK^T with the dequant scales
 * applied before the mask (aiter PR #6617, review), masked online softmax,
 * PV, and the partition epilogue.  Writes partial states to workspace_dev
 * for multi-partition (sequence, KV head) pairs and the final rows of `out`
 * for the others (including cleared rows of empty sequences).
 * Arguments: device pointers in the layouts of pa_problem; meta_dev filled
 * by pa_plan_upload (or pa_plan_refresh) for this plan; workspace_dev of
 * workspace_bytes; `stream` a hipStream_t (NULL: default stream).  Never
 * allocates, copies or synchronises: it can be captured in a HIP graph.
 * Device context_lens are authoritative: a sequence longer than planned is
 * still fully processed (its last partition runs to the end, reading page ids
 * past the staged range from the block table directly); lengths below 0
 * count as 0 and lengths past table_stride pages (slots) as that capacity.
 * Errors: PA_ERR_INVALID for null or misaligned (16 B) pointers,
 * PA_ERR_WORKSPACE for missing meta/workspace or a meta_dev that does not
 * hold this plan's metadata, PA_ERR_DEVICE for launch errors.
 */
pa_status pa_decode(const pa_plan_t* plan, void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, const float* k_scale,
                    const float* v_scale, const float* sinks, void* meta_dev, void* workspace_dev, void* stream);

/*
 * The partition merge (aiter PR #7079 "Merge gfx1250 PA decode partitions",
 * Launch and reducer latency; sinks at the merge, Partition merges): merge
 * the partial states of every multi-partition (sequence, KV head) into `out`
 * by the log-sum-exp rule, partitions added in a fixed order (run-to-run
 * bit-identical); sinks join the denominator; a row with no visible token
 * gets 0.  At most one launch; none if the plan has no multi-partition pair.
 * Must follow pa_decode of the same plan on the same stream.  A plan with
 * its meta/workspace must not serve two in-flight calls.  Errors as
 * pa_decode.
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

/*
 * The sparse decode of aiter PR #7079 (summary and Performance setup: rows
 * attending their top-k tokens of a paged context) with two-level indices,
 * for plans of problems with token_table = 2: row s attends
 * topk_indices[s][0..topk_counts[s]) (int32 logical positions, row stride
 * index_stride), resolved through block_tables[s] (int32 page ids, row
 * stride table_stride) to physical page slots.  Otherwise as pa_decode,
 * followed by pa_reduce as usual.  PA_ERR_INVALID for a plan whose problem is
 * not token_table = 2 (and pa_decode refuses those plans).
 */
pa_status pa_decode_sparse(const pa_plan_t* plan, void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* topk_indices, const int32_t* topk_counts,
                           const float* k_scale, const float* v_scale, const float* sinks, void* meta_dev,
                           void* workspace_dev, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): pa_decode
 * followed by pa_reduce, with the plan metadata and the partial states kept
 * in a static device array of this library instead of meta_dev and
 * workspace_dev.  Each GPU holds its own array of PA_STATIC_SCRATCH_BYTES
 * until the process ends; a plan needing more (its meta_bytes rounded up to
 * 256, plus workspace_bytes) is refused with PA_ERR_WORKSPACE.  No call
 * allocates: the metadata is copied into the array (asynchronously on
 * `stream`, from the plan's pinned copy when pa_plan_upload made one) only
 * when the array does not already hold this plan's.  All calls on one GPU
 * share the array and it keeps the last call's contents: calls that overlap
 * on one GPU (other streams, other threads) race.  The other arguments and
 * errors are those of pa_decode.
 */
#define PA_STATIC_SCRATCH_BYTES (32u << 20)
pa_status pa_attend_static(const pa_plan_t* plan, void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* context_lens, const float* k_scale,
                           const float* v_scale, const float* sinks, void* stream);

/* Thread-local message for the last non-OK status of this thread. */
const char* pa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
