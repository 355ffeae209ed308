/*
 * Sparse front end of the decode: the indexer whose top-k token positions the
 * two-level sparse decode (pa_decode_sparse) consumes.
 *
 * The FlyDSL pages describe it in two places: the fp8_mqa_logits kernel
 * (aiter PR "LDS-staged fp8_mqa_logits for gfx942", Summary, Changes and
 * Performance: per-row scores over a KV window, a ReLU x weight epilogue
 * reduced over the heads, -inf outside each row's window under clean_logits,
 * shapes of rows x KV tokens at 16-128 heads), and the sparse decode of
 * aiter PR #7079 (Summary: a top-k index stage selects the token positions
 * that a block-table stage maps to physical KV).
 *
 * Both calls are asynchronous on `stream` (a hipStream_t; NULL: the null
 * stream), take device pointers the caller owns, allocate nothing, and
 * return PA_OK, PA_ERR_INVALID (a NULL pointer or a size out of range,
 * checked before any launch), PA_ERR_UNSUPPORTED (a head count or head dim
 * the kernels do not build) or PA_ERR_DEVICE (a launch failed);
 * pa_last_error describes the last failure of the calling thread.
 */
#ifndef PA_INDEXER_H_
#define PA_INDEXER_H_

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * FP8 MQA logits: for every query row r and KV token t of the row's window
 * ks[r] <= t < ke[r] (both clamped into [0, num_kv]),
 *
 *   logits[r * logits_stride + t] = sum_h weights[r * num_heads + h]
 *                                   * relu(kv_scale[t] * dot(q[r, h, :], kv[t, :]))
 *
 * and, when clean != 0, -inf at every other t < num_kv (clean == 0 leaves
 * those entries unspecified: they may or may not be written).
 *
 *   q        FP8 e4m3fn [rows, num_heads, head_dim], row-major
 *   kv       FP8 e4m3fn [num_kv, head_dim] (the index keys of the KV tokens)
 *   kv_scale FP32 [num_kv], each >= 0 (a dequantisation scale)
 *   weights  FP32 [rows, num_heads] (any query scale folded in by the caller)
 *   ks, ke   int32 [rows]
 *   logits   FP32, rows of logits_stride >= num_kv elements
 *
 * head_dim 128; num_heads 16, 32, 64 or 128.  rows >= 0 and num_kv >= 0
 * (either 0: nothing to do).  Accumulation is FP32 (products of FP8 values
 * are exact; at most 128 + 128 sums round): |error| stays within 2^-16 of
 * sum_h |weights[r, h]| kv_scale[t] sum_d |q[r, h, d] kv[t, d]|.
 */
pa_status pa_mqa_logits(float* logits, const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                        const float* weights, const int32_t* ks, const int32_t* ke, int32_t rows, int32_t num_kv,
                        int32_t num_heads, int32_t head_dim, int64_t logits_stride, int32_t clean, void* stream);

/*
 * Top-k of each row's window: the k largest logits[r * logits_stride + t] for
 * t in [ks[r], ke[r]) (clamped into [0, num_kv]), ties broken by the lower
 * position, -0.0 equal to +0.0 (NaN logits are outside the contract).
 *
 *   indices  int32 [rows, k]: the selected positions relative to ks[r]
 *            (t - ks[r]), ascending, -1 past the row's count
 *   counts   int32 [rows]: min(k, window length)
 *
 * indices and counts are what pa_decode_sparse takes as topk_indices (with
 * index_stride = k) and topk_counts when ks[r] is the first index key of
 * row r's sequence.  k >= 1.
 *
 * With few rows the windows are first cut into segments whose own top k
 * are kept as candidates (every key of the row's top k is in its segment's
 * top k), then each row selects from its candidates: workspace (16-byte
 * aligned, caller-owned, contents irrelevant) holds them, of at least the
 * bytes pa_topk_workspace_size returns for (rows, num_kv, k) (0: no
 * workspace needed, NULL allowed); too small: PA_ERR_WORKSPACE.
 */
pa_status pa_topk(int32_t* indices, int32_t* counts, const float* logits, const int32_t* ks, const int32_t* ke,
                  int32_t rows, int32_t num_kv, int64_t logits_stride, int32_t k, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Workspace bytes pa_topk needs for (rows, num_kv, k). */
pa_status pa_topk_workspace_size(int32_t rows, int32_t num_kv, int32_t k, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* PA_INDEXER_H_ */
