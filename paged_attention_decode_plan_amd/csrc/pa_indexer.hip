// gfx950 indexer of the sparse decode: FP8 MQA logits and the per-row top-k
// (the fp8_mqa_logits indexer of aiter PR "LDS-staged fp8_mqa_logits for
// gfx942", Summary and Changes; the top-k index stage of aiter PR #7079,
// Summary).
//
// Logits (one workgroup = 8 waves = 8 query rows x 256 KV tokens):
//  * the 256 tokens' FP8 index keys (32 KB) are staged once in LDS, their
//    16-byte chunks XOR-swizzled by token so that the per-lane operand reads
//    of 32 consecutive tokens spread over the banks; each wave then keeps its
//    row's FP8 query (H x 128) in registers as the MFMA A operand;
//  * scores run on v_mfma_scale_f32_32x32x64_f8f6f4 (block scales 1): heads
//    are the MFMA rows and tokens the columns, so a lane's 16 accumulator
//    values are 16 heads of one token and the head reduction is in-lane:
//    sum_h w_h * max(s, 0) over the lane's heads, then one permlane32 swap
//    adds the other half of the heads;
//  * the per-token key scale multiplies the head sum (scales are
//    non-negative, so it commutes with the ReLU); the window mask and the
//    -inf fill are applied at the store, and a wave whose row's window misses
//    the whole tile only writes the fill.
//
// Top-k (one workgroup of 1024 threads per row, the window read in
// coalesced batches of 16 keys per thread with every load in flight): the
// bin of order-preserving 32-bit keys that holds the k-th largest by a
// radix select of up to four 8-bit passes (LDS histograms in 32
// bank-staggered copies, lane & 31, so that clustered keys do not
// serialise on one word; it stops once the whole bin is taken), then one
// pass in position order that writes every key above the bin and the first
// keys inside it (lower positions first) until k are taken, ascending.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>

#include "pa_device.h"
#include "pa_indexer.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int LG_TOK = 256;  // KV tokens per logits workgroup
constexpr int LG_ROWS = 8;   // query rows per logits workgroup (one per wave)
constexpr int LG_D = 128;    // index head dim

struct LogitsArgs {
  float* logits;
  const uint8_t* q;
  const uint8_t* kv;
  const float* kv_scale;
  const float* weights;
  const int32_t* ks;
  const int32_t* ke;
  long long stride;
  int rows, num_kv, clean;
};

// max(x, 0) as one integer max on the bits (a negative float, -0.0
// included, is a negative int32; a non-negative one keeps its bits): fmaxf
// would also quieten NaNs first, one more instruction per score.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int H>
__global__ __launch_bounds__(512) void mqa_logits_kernel(LogitsArgs a) {
  constexpr int D = LG_D;
  constexpr int MB = (H + 31) / 32;  // 32-head blocks (16 heads: one block, rows 16..31 zero)
  __shared__ __attribute__((aligned(16))) uint8_t kt[LG_TOK * D];
  __shared__ float sc[LG_TOK];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hh = lane >> 5;
  const long t0 = (long)blockIdx.x * LG_TOK;
  const int r = blockIdx.y * LG_ROWS + w;
  const bool row_ok = r < a.rows;
  const int N = a.num_kv;

  // ---- stage the tile's keys (chunk c of token t at 16-byte slot t*8 + (c ^ (t & 7))) and scales ----
#pragma unroll
  for (int j = 0; j < (LG_TOK * D / 16) / 512; ++j) {
    const int u = tid + 512 * j;
    const int tok = u >> 3, pc = u & 7, lc = pc ^ (tok & 7);
    const long src = min(t0 + tok, (long)N - 1);  // past the end: the last token (never stored)
    *(u32x4*)(kt + u * 16) = *(const u32x4*)(a.kv + src * D + lc * 16);
  }
  if (tid < LG_TOK) sc[tid] = a.kv_scale[min(t0 + tid, (long)N - 1)];

  // ---- the wave's row: window, query operand, weights ----
  int lo = 0, hi = 0;
  if (row_ok) {
    lo = min(max(a.ks[r], 0), N);
    hi = min(max(a.ke[r], lo), N);
  }
  // A operand of head block mb, k-step ks: head 32 mb + n, dims 64 ks + 32 hh .. +31
  i32x8 qa[MB][2];
  // weight of accumulator slot j of head block mb: head 32 mb + 8 (j / 4) + 4 hh + j % 4
  float wv[MB][16];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = 32 * mb + n;
    const bool hq = row_ok && head < H;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t* src = a.q + (((long)(hq ? r : 0) * H + (hq ? head : 0)) * D + 64 * ks + 32 * hh);
      const u32x4 lo4 = hq ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
      const u32x4 hi4 = hq ? *(const u32x4*)(src + 16) : u32x4{0, 0, 0, 0};
      qa[mb][ks] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int jq = 0; jq < 4; ++jq) {
      const int h0 = 32 * mb + 8 * jq + 4 * hh;
      const bool hw = row_ok && h0 < H;
      const f4 v = hw ? *(const f4*)(a.weights + (long)r * H + h0) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) wv[mb][4 * jq + e] = v[e];
    }
  }
  __syncthreads();  // keys and scales staged

  const bool any = row_ok && lo < hi && t0 < hi && t0 + LG_TOK > lo;  // wave-uniform
  float* orow = a.logits + (long)(row_ok ? r : 0) * a.stride;
  if (!row_ok || (!any && !a.clean)) return;
#pragma unroll 2
  for (int sb = 0; sb < LG_TOK / 32; ++sb) {
    const long t = t0 + 32 * sb + n;
    float logit = -INFINITY;
    if (any) {
      const int tok = 32 * sb + n;
      i32x8 kb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c0 = 4 * ks + 2 * hh;
        const u32x4 x0 = *(const u32x4*)(kt + (tok * 8 + (c0 ^ (tok & 7))) * 16);
        const u32x4 x1 = *(const u32x4*)(kt + (tok * 8 + ((c0 + 1) ^ (tok & 7))) * 16);
        kb[ks] = __builtin_bit_cast(i32x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      float part0 = 0.f, part1 = 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f32x16 acc = {};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][0], kb[0], acc, 0, 0, 0, 127, 0, 127);
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[mb][1], kb[1], acc, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          part0 += wv[mb][j] * relu_bits(acc[j]);
          part1 += wv[mb][j + 1] * relu_bits(acc[j + 1]);
        }
      }
      const float part = part0 + part1;
      const float total = fadd_swap32(part);  // + the other 16 heads of each block (lanes n and n + 32)
      logit = total * sc[tok];
      if (t < lo || t >= hi) logit = -INFINITY;
    }
    if (hh == 0 && t < N && (a.clean || (t >= lo && t < hi))) orow[t] = logit;
  }
}

// ---- top-k ----
constexpr int TK_T = 1024;             // threads of a top-k workgroup
constexpr int TK_W = TK_T / 64;        // its waves
constexpr int TK_E = 16;               // keys per thread per batch, loaded together
constexpr int TK_CHUNK = TK_T * TK_E;  // keys of one batch (thread t: c0 + t + TK_T j)
constexpr int TK_NE = TK_E * TK_W;     // (slot j, wave w) entries of one batch, in position order
constexpr int TK_SUB = 32;             // histogram copies (lane & 31): at most two lanes meet on one word
constexpr int TK_HROW = 257;           // padded copy stride: copies of one bin sit in different banks

struct TopkArgs {
  int32_t* indices;
  int32_t* counts;
  const float* logits;
  const int32_t* ks;
  const int32_t* ke;
  long long stride;
  int rows, num_kv, k;
  int segs;          // segments per row of the first stage (1: a single stage)
  uint32_t* ckey;    // candidates [rows][segs][k]: keys, positions, counts
  int32_t* cpos;
  int32_t* ccount;
};

// Order-preserving key: larger float <-> larger unsigned key; -0.0 is made
// +0.0 first so that the two compare equal.
__device__ __forceinline__ uint32_t fkey(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the wave (lane order).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Top-k modes: the whole window of a row to its final positions; one
// segment of a row's window to k candidates (first stage); a row's
// candidates to its final positions (second stage).
enum TopkMode { TK_ROW = 0, TK_SEG = 1, TK_CAND = 2 };

// One workgroup selects the k largest keys of n elements in position order
// (ties: the lower position).  Element i: key(i) and validity come from the
// mode's source; selected elements are written in ascending position order.
template <int MODE>
__global__ __launch_bounds__(TK_T) void topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[TK_SUB * TK_HROW];
  __shared__ uint32_t tot[256];
  __shared__ uint32_t scan[2][TK_NE + TK_W];  // per (j, w) counts, then their exclusive scan
  __shared__ uint32_t sel[3];
  __shared__ int32_t seg_cnt[16];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int K = a.k, N = a.num_kv;
  const int r = MODE == TK_SEG ? blockIdx.x / a.segs : blockIdx.x;
  const int seg = MODE == TK_SEG ? blockIdx.x % a.segs : 0;
  const int lo = min(max(a.ks[r], 0), N);
  const int hi = min(max(a.ke[r], lo), N);
  const int nw = hi - lo;  // window length
  // the elements this workgroup selects from
  int base = 0, n = nw;
  if (MODE == TK_SEG) {
    const int sl = (nw + a.segs - 1) / a.segs;
    base = min(seg * sl, nw);
    n = min(nw - base, sl);
  } else if (MODE == TK_CAND) {
    n = a.segs * K;
    if (tid < a.segs) seg_cnt[tid] = a.ccount[r * a.segs + tid];
    __syncthreads();
  }
  const float* row = a.logits + (long)r * a.stride + lo + base;
  const uint32_t* crow_k = a.ckey + (long)r * a.segs * K;
  const int32_t* crow_p = a.cpos + (long)r * a.segs * K;
  // outputs: final positions of the row, or this segment's candidates
  int32_t* out = MODE == TK_SEG ? a.cpos + ((long)r * a.segs + seg) * K : a.indices + (long)r * K;
  uint32_t* outk = a.ckey + ((long)r * a.segs + seg) * K;  // first stage only
  // validity of element i (candidates: inside its segment's count); the
  // quotient by k runs through a float reciprocal with an exact correction
  // (i < 2^24), not an integer division per element
  const float inv_k = 1.0f / (float)K;
  auto valid_at = [&](int i) {
    if (MODE == TK_CAND) {
      if (i >= n) return false;
      int q = (int)((float)i * inv_k);
      q -= q * K > i ? 1 : 0;
      q += (q + 1) * K <= i ? 1 : 0;
      return i - q * K < seg_cnt[q];
    }
    return i < n;
  };
  auto emit = [&](uint32_t pos, int32_t position, uint32_t key) {
    out[pos] = position;
    if (MODE == TK_SEG) outk[pos] = key;
  };

  // The thread's keys of the batch at c0 (element c0 + tid + TK_T j in slot
  // j: each load instruction of a wave reads 64 consecutive keys).  Every
  // load is unconditional (an index past the elements reads the last one;
  // valid_at marks the slot), so all of them are in flight together.
  uint32_t key[TK_E];
  int32_t cpos[MODE == TK_CAND ? TK_E : 1];  // candidates: their positions, loaded with the keys
  uint32_t vbits = 0;  // bit j: slot j holds an element of the batch
  const bool resident = n <= TK_CHUNK;  // one batch: its keys stay in registers through every pass
  auto load_keys = [&](int c0) {
    vbits = 0;
#pragma unroll
    for (int j = 0; j < TK_E; ++j) vbits |= valid_at(c0 + tid + TK_T * j) ? (1u << j) : 0u;
    if (MODE == TK_CAND) {
#pragma unroll
      for (int j = 0; j < TK_E; ++j) key[j] = crow_k[min(c0 + tid + TK_T * j, n - 1)];
      // the positions now, so that writing a selected candidate waits for
      // no load of its own
#pragma unroll
      for (int j = 0; j < (MODE == TK_CAND ? TK_E : 0); ++j) cpos[j] = crow_p[min(c0 + tid + TK_T * j, n - 1)];
    } else {
      float v[TK_E];
#pragma unroll
      for (int j = 0; j < TK_E; ++j) v[j] = row[min(c0 + tid + TK_T * j, n - 1)];
#pragma unroll
      for (int j = 0; j < TK_E; ++j) key[j] = fkey(v[j]);
    }
  };

  if (MODE != TK_CAND && n <= K) {  // every element is taken
    if (MODE == TK_SEG) {
      for (int i = tid; i < n; i += TK_T) emit(i, base + i, fkey(row[i]));
      if (tid == 0) a.ccount[r * a.segs + seg] = n;
    } else {
      for (int i = tid; i < K; i += TK_T) out[i] = i < n ? i : -1;
      if (tid == 0) a.counts[r] = n;
    }
    return;
  }

  if (resident) load_keys(0);

  // second stage of a row whose window held at most k keys: every candidate
  int total = K + 1;
  if (MODE == TK_CAND) {
    total = 0;
    for (int x = 0; x < a.segs; ++x) total += seg_cnt[x];
  }
  const bool take_all = total <= K;  // workgroup-uniform

  // ---- radix select, 8 bits a pass from the top: the bin [tlo, thi] of
  // keys that holds the k-th largest, and how many of its keys are taken
  // (need; the rest of the k are the keys above thi).  Stops early once
  // every key of the bin is taken.  (Taking every candidate: an empty bin
  // below every key.) ----
  uint32_t prefix = 0, need = take_all ? 0u : (uint32_t)K, tlo = take_all ? 1u : 0u, thi = take_all ? 0u : 0xFFFFFFFFu;
  for (int pass = 0; pass < (take_all ? 0 : 4); ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < TK_SUB * TK_HROW; i += TK_T) hist[i] = 0;
    if (tid == 0) {  // overwritten by the lane that finds the bin
      sel[0] = 0;
      sel[1] = need;
      sel[2] = 0;
    }
    __syncthreads();
    uint32_t* hl = hist + (lane & (TK_SUB - 1)) * TK_HROW;
    for (int c0 = 0; c0 < n; c0 += TK_CHUNK) {
      if (!resident) load_keys(c0);
#pragma unroll
      for (int j = 0; j < TK_E; ++j) {
        if (((vbits >> j) & 1u) && (pass == 0 || (key[j] >> (shift + 8)) == prefix))
          atomicAdd(hl + ((key[j] >> shift) & 255u), 1u);
      }
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t s = 0;
#pragma unroll 8
      for (int x = 0; x < TK_SUB; ++x) s += hist[x * TK_HROW + tid];
      tot[tid] = s;
    }
    __syncthreads();
    if (w == 0) {
      // bins from the top: lane l holds bins 255 - 4l - j, j = 0..3
      uint32_t c[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = tot[255 - 4 * lane - j];
        s += c[j];
      }
      const uint32_t before = wave_incl_scan(s, lane) - s;  // keys in higher bins than the lane's
      uint32_t cum = before;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (cum < need && cum + c[j] >= need) {
          sel[0] = 255u - 4u * lane - j;
          sel[1] = need - cum;
          sel[2] = c[j];
        }
        cum += c[j];
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | sel[0];
    need = sel[1];
    tlo = prefix << shift;
    thi = tlo | ((1u << shift) - 1u);
    const bool whole_bin = sel[2] == need;
    __syncthreads();  // sel read by every thread before the next pass writes it
    if (whole_bin) break;  // workgroup-uniform
  }

  // ---- take the keys above thi, and the first `need` keys of [tlo, thi],
  // in position order: element c0 + TK_T j + 64 w + lane, so (j, w) runs in
  // position order and one scan over the batch's (j, w) counts places them,
  // ascending ----
  const uint64_t below = (1ull << lane) - 1;  // lanes before this one
  uint32_t run_gt = 0, run_eq = 0;            // keys above / inside the bin in earlier batches
  for (int c0 = 0; c0 < n; c0 += TK_CHUNK) {
    if (!resident) load_keys(c0);
#pragma unroll
    for (int j = 0; j < TK_E; ++j) {
      const bool valid = (vbits >> j) & 1u;
      const uint64_t bg = __builtin_amdgcn_ballot_w64(valid && key[j] > thi);
      const uint64_t be = __builtin_amdgcn_ballot_w64(valid && key[j] >= tlo && key[j] <= thi);
      if (lane == 0) {
        scan[0][j * TK_W + w] = (uint32_t)__builtin_popcountll(bg);
        scan[1][j * TK_W + w] = (uint32_t)__builtin_popcountll(be);
      }
    }
    __syncthreads();
    // exclusive scan of the TK_NE entries, one per thread of the first
    // TK_NE / 64 waves
    constexpr int SW = TK_NE / 64;
    const uint32_t vg = tid < TK_NE ? scan[0][tid] : 0u, ve = tid < TK_NE ? scan[1][tid] : 0u;
    const uint32_t ig = wave_incl_scan(vg, lane), ie = wave_incl_scan(ve, lane);
    if (lane == 63 && w < SW) {
      scan[0][TK_NE + w] = ig;
      scan[1][TK_NE + w] = ie;
    }
    __syncthreads();
    uint32_t og = 0, oe = 0, cg = 0, ce = 0;
#pragma unroll
    for (int x = 0; x < SW; ++x) {
      const uint32_t g = scan[0][TK_NE + x], q = scan[1][TK_NE + x];
      og += x < w ? g : 0u;
      oe += x < w ? q : 0u;
      cg += g;
      ce += q;
    }
    __syncthreads();  // every thread has read the entries it scans
    if (tid < TK_NE) {
      scan[0][tid] = run_gt + og + ig - vg;
      scan[1][tid] = run_eq + oe + ie - ve;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TK_E; ++j) {
      const int i = c0 + tid + TK_T * j;
      const bool valid = (vbits >> j) & 1u;
      const bool gt = valid && key[j] > thi, eq = valid && key[j] >= tlo && key[j] <= thi;
      const uint64_t bg = __builtin_amdgcn_ballot_w64(gt);
      const uint64_t be = __builtin_amdgcn_ballot_w64(eq);
      if (bg | be) {  // wave-uniform: most (j, w) blocks hold no selected key
        const uint32_t gt_before = scan[0][j * TK_W + w] + (uint32_t)__builtin_popcountll(bg & below);
        const uint32_t eq_before = scan[1][j * TK_W + w] + (uint32_t)__builtin_popcountll(be & below);
        const uint32_t pos = gt_before + min(eq_before, need);
        if ((gt || (eq && eq_before < need)) && pos < (uint32_t)K) emit(pos, MODE == TK_CAND ? cpos[j % (MODE == TK_CAND ? TK_E : 1)] : base + i, key[j]);
      }
    }
    run_gt += cg;
    run_eq += ce;
    __syncthreads();  // scan read before the next batch writes it
  }
  if (MODE == TK_CAND && take_all)
    for (int i = total + tid; i < K; i += TK_T) out[i] = -1;
  if (tid == 0) {
    if (MODE == TK_SEG)
      a.ccount[r * a.segs + seg] = K;
    else
      a.counts[r] = take_all ? total : K;
  }
}

}  // namespace
}  // namespace pa

using namespace pa;

namespace pa {
namespace {
// First-stage segments per row: enough workgroups for the CUs (about 256)
// when rows are few, each segment at least 4k keys, at most 16.
int topk_segments(int rows, int num_kv, int k) {
  if (rows <= 0) return 1;
  int s = (256 + rows - 1) / rows;
  s = std::min(s, std::max(1, num_kv / (4 * k)));
  return std::max(1, std::min(s, 16));
}
}  // namespace
}  // namespace pa

extern "C" pa_status pa_mqa_logits(float* logits, const uint8_t* q, const uint8_t* kv, const float* kv_scale,
                                   const float* weights, const int32_t* ks, const int32_t* ke, int32_t rows,
                                   int32_t num_kv, int32_t num_heads, int32_t head_dim, int64_t logits_stride,
                                   int32_t clean, void* stream) {
  if (rows < 0 || num_kv < 0) return set_error(PA_ERR_INVALID, "rows and num_kv must be >= 0");
  if (head_dim != LG_D) return set_error(PA_ERR_UNSUPPORTED, "pa_mqa_logits supports head_dim 128");
  if (num_heads != 16 && num_heads != 32 && num_heads != 64 && num_heads != 128)
    return set_error(PA_ERR_UNSUPPORTED, "pa_mqa_logits supports 16, 32, 64 or 128 heads");
  if (rows == 0 || num_kv == 0) return PA_OK;
  if (!logits || !q || !kv || !kv_scale || !weights || !ks || !ke)
    return set_error(PA_ERR_INVALID, "a pointer argument is NULL");
  if (logits_stride < num_kv) return set_error(PA_ERR_INVALID, "logits_stride must be >= num_kv");
  if (((uintptr_t)q | (uintptr_t)kv | (uintptr_t)weights) & 15)
    return set_error(PA_ERR_INVALID, "q, kv and weights must be 16-byte aligned");
  const long gy = ((long)rows + LG_ROWS - 1) / LG_ROWS;
  if (gy > 65535) return set_error(PA_ERR_INVALID, "rows must be at most 524280");
  LogitsArgs a{logits, q, kv, kv_scale, weights, ks, ke, (long long)logits_stride, rows, num_kv, clean != 0};
  const dim3 grid((unsigned)(((long)num_kv + LG_TOK - 1) / LG_TOK), (unsigned)gy);
  auto launch = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(512), 0, (hipStream_t)stream, a); };
  switch (num_heads) {
    case 16: launch(mqa_logits_kernel<16>); break;
    case 32: launch(mqa_logits_kernel<32>); break;
    case 64: launch(mqa_logits_kernel<64>); break;
    default: launch(mqa_logits_kernel<128>); break;
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("logits launch failed: ") + hipGetErrorString(err));
  return PA_OK;
}

extern "C" pa_status pa_topk_workspace_size(int32_t rows, int32_t num_kv, int32_t k, size_t* bytes) {
  if (rows < 0 || num_kv < 0 || k < 1 || !bytes) return set_error(PA_ERR_INVALID, "rows, num_kv >= 0, k >= 1 and bytes required");
  const int segs = topk_segments(rows, num_kv, k);
  *bytes = segs > 1 ? (size_t)rows * segs * ((size_t)k * 8 + 4) : 0;
  return PA_OK;
}

extern "C" pa_status pa_topk(int32_t* indices, int32_t* counts, const float* logits, const int32_t* ks,
                             const int32_t* ke, int32_t rows, int32_t num_kv, int64_t logits_stride, int32_t k,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 0 || num_kv < 0 || k < 1) return set_error(PA_ERR_INVALID, "rows, num_kv >= 0 and k >= 1 required");
  if (rows == 0) return PA_OK;
  if (!indices || !counts || !ks || !ke || (num_kv > 0 && !logits))
    return set_error(PA_ERR_INVALID, "a pointer argument is NULL");
  if (logits_stride < num_kv) return set_error(PA_ERR_INVALID, "logits_stride must be >= num_kv");
  size_t need = 0;
  pa_topk_workspace_size(rows, num_kv, k, &need);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 15)))
    return set_error(PA_ERR_WORKSPACE, "top-k needs a 16-byte aligned workspace of " + std::to_string(need) +
                                           " bytes (pa_topk_workspace_size)");
  const int segs = topk_segments(rows, num_kv, k);
  TopkArgs a{indices, counts, logits, ks, ke, (long long)logits_stride, rows, num_kv, k, segs, nullptr, nullptr,
             nullptr};
  if (segs > 1) {
    a.ckey = (uint32_t*)workspace;
    a.cpos = (int32_t*)((uint8_t*)workspace + (size_t)rows * segs * k * 4);
    a.ccount = (int32_t*)((uint8_t*)workspace + (size_t)rows * segs * k * 8);
    hipLaunchKernelGGL(topk_kernel<TK_SEG>, dim3((unsigned)(rows * segs)), dim3(TK_T), 0, (hipStream_t)stream, a);
    hipLaunchKernelGGL(topk_kernel<TK_CAND>, dim3((unsigned)rows), dim3(TK_T), 0, (hipStream_t)stream, a);
  } else {
    hipLaunchKernelGGL(topk_kernel<TK_ROW>, dim3((unsigned)rows), dim3(TK_T), 0, (hipStream_t)stream, a);
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("top-k launch failed: ") + hipGetErrorString(err));
  return PA_OK;
}
