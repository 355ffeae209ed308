// gfx950 split-KV paged-attention decode: the tile kernel, the partition
// reducer and the pa_decode / pa_reduce entry points.
//
// Method (FlyDSL paged-attention decode pages): each work item runs an online
// softmax over its token range and writes (max, sum, partial O) per query row
// (aiter PR #4332 "Add paged-attention Tile kernel", launch with pmax/psum/pout
// partials); a reducer merges partitions in a fixed order (aiter PR #7079,
// "Launch and reducer latency"); the score scale is multiplied in before the
// -inf mask and fully masked rows use a safe exponent (aiter PR #6617, summary
// and review: scale-before-mask); table entries past a sequence's extent are
// never dereferenced and garbage V bytes past the extent cannot reach the
// output (aiter PR #4332 follow-up commit: pinning stale entries, 0*NaN).
//
// gfx950 design (not the pages' FlyDSL tiling):
//  * a workgroup of 4 waves owns one work item = (sequence, KV head, row
//    group of up to 64 query rows, a contiguous range of 128-token tiles);
//  * K/V pages of a tile are staged in LDS through registers with 16-byte
//    coalesced loads, double-buffered so tile j+1 loads while tile j computes;
//  * each wave takes 32 tokens of every tile for all of the item's query rows,
//    so every K/V byte is read from LDS and converted exactly once; the four
//    waves keep independent online-softmax states merged once at the end;
//  * QK^T is computed as S^T = K Q^T and PV as O^T = V^T P^T with
//    v_mfma_f32_16x16x32_{f16,bf16}: FP8 K/V convert exactly to FP16 in
//    registers (v_cvt_scalef32_pk_f16_fp8), BF16 queries are scaled by a
//    per-row power of two into FP16 (exact), probabilities go from the QK
//    accumulator to the PV operand in registers (the QK rows are read in the
//    token order PV contracts), FP16 P keeps 11 significant bits;
//  * row max/sum across the 4 lane groups of a row use v_permlane16/32_swap;
//  * rescaling of the accumulator is lazy: only when a row maximum grows by
//    more than 2^8, or the per-token V-scale reference leaves its band.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "pa_internal.h"

namespace pa {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int TT = kTileTokens;  // 128 tokens per tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr float TAU = 8.0f;  // lazy-rescale band (log2 units): probabilities stay <= 2^8

struct KernelArgs {
  void* out;
  const void* q;
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const float* k_scale;
  const float* v_scale;
  const float* sinks;
  const WorkItem* items;
  float* workspace;
  long long page_stride;  // bytes between physical pages (Hkv * D * page * elem)
  long long head_stride;  // bytes between KV heads of a page (D * page * elem)
  int QL, Hq, G, page_size, table_stride, window, causal;
  int v_transposed, scale_mode, q_fp16, has_sinks, rows_total, rows_per_group, stage_limit;
  float scale_log2;  // softmax_scale * log2(e)
};

__device__ __forceinline__ float fmax_swap16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fmax_swap32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fadd_swap16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float fadd_swap32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// max / sum over the four 16-lane groups (lanes c, c+16, c+32, c+48)
__device__ __forceinline__ float group_max(float x) { return fmax_swap32(fmax_swap16(x)); }
__device__ __forceinline__ float group_sum(float x) { return fadd_swap32(fadd_swap16(x)); }

__device__ __forceinline__ half8 fp8x8_to_half8(u32x2 v) {
  h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[0], 1.0f, false);
  h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[0], 1.0f, true);
  h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[1], 1.0f, false);
  h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[1], 1.0f, true);
  return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Token position of a K row inside the LDS K tile (16-byte rows).  The XOR
// spreads the QK operand reads of one lane group over all bank quads.
__device__ __forceinline__ int kswz(int t) { return t ^ (((t >> 3) & 1) << 2); }

// Row d of a staged V tile holds TT tokens; with FP8 its 8-byte units are
// stored at unit ^ (d & 15), with BF16 its 16-byte units likewise, so the 16
// lanes reading one unit column from 16 rows hit distinct banks.

template <int D, bool FP8>
struct Tile {
  static constexpr int E = FP8 ? 1 : 2;      // bytes per KV element
  static constexpr int X = 16 / E;           // elements per 16-byte chunk
  static constexpr int KBYTES = D * TT * E;  // K tile bytes
  static constexpr int VROW = TT * E;        // bytes per V row
  static constexpr int VBYTES = D * VROW;
  static constexpr int SBYTES = FP8 ? 2 * TT * 4 : 0;  // per-token k and v scales
  static constexpr int STAGE = KBYTES + VBYTES + SBYTES;
  static constexpr int KUNITS = KBYTES / 16;
  static constexpr int VUNITS = VBYTES / 16;
  static constexpr int KPT = KUNITS / NTHREADS;  // 16-byte K units per thread per tile
  static constexpr int VPT = VUNITS / NTHREADS;
  static constexpr int NM = D / 32;               // MFMA k-steps over the head dim
  static constexpr int NDT = D / 16;              // 16-wide d tiles of O
};

template <int D, bool FP8, int NRT>
struct Smem {
  static constexpr int STAGES = 2;
  static constexpr int STAGE = Tile<D, FP8>::STAGE;
  static constexpr int MERGE = 2 * NRT * 16 * (D + 4) * 4;  // two O buffers with padded rows
  static constexpr int MAIN = (STAGES * STAGE > MERGE) ? STAGES * STAGE : MERGE;
  static constexpr int IDS = kStageCap * 4;
  static constexpr int STATS = NWAVES * NRT * 16 * 2 * 4 + NWAVES * 4 + NRT * 16 * 4 * 4;
  static constexpr int TOTAL = MAIN + IDS + STATS;
};

// Staging registers of one tile for one thread.
template <int D, bool FP8>
struct Staged {
  u32x4 k[Tile<D, FP8>::KPT];
  u32x4 v[Tile<D, FP8>::VPT];
  u32x4 s;  // 4 per-token scales (threads 0..63: K scales, 64..127: V scales)
  uint32_t kmask, vmask;
  int sdst;
};

template <int D, bool FP8, int NRT, bool SPARSE>
__global__ __launch_bounds__(NTHREADS) void pa_decode_kernel(KernelArgs a) {
  using T = Tile<D, FP8>;
  using S = Smem<D, FP8, NRT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* stage_base = smem;
  int32_t* ids = (int32_t*)(smem + S::MAIN);
  float* stats = (float*)(smem + S::MAIN + S::IDS);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;
  const int g = lane >> 4;

  const WorkItem it = a.items[blockIdx.x];
  const int s = it.seq, kvh = it.kvh, rg = it.rg;
  const int ps = a.page_size;
  const long cap = SPARSE ? (long)a.table_stride : (long)a.table_stride * ps;
  const int L = (int)min(max((long)a.context_lens[s], 0L), cap);

  // Visible span of the sequence (union over its query rows).
  int lo_u = 0, hi_u = L;
  if (!SPARSE && L > 0 && a.window > 0) {
    int first_pos = a.causal ? L - a.QL : L - 1;
    lo_u = max(0, first_pos - a.window + 1);
  }
  const int t0 = SPARSE ? 0 : (lo_u / ps) * ps;
  const int ntiles = hi_u > lo_u ? (hi_u - t0 + TT - 1) / TT : 0;
  const int tb = min(it.tile_begin, ntiles);
  const int te = it.tile_end < 0 ? ntiles : min(it.tile_end, ntiles);

  // Rows of this item.
  const int rpg = a.rows_per_group;
  const int row0 = rg * kMaxRowsPerItem;
  const int nrows = min(rpg, a.rows_total - row0);
  int lo_r[NRT], hi_r[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    int r = rt * 16 + c;
    if (r < nrows) {
      int gr = row0 + r, i = gr / a.G;
      int pos = a.causal ? L - a.QL + i : L - 1;
      hi_r[rt] = min(pos, L - 1);
      lo_r[rt] = a.window > 0 ? max(0, pos - a.window + 1) : 0;
    } else {
      lo_r[rt] = 1;
      hi_r[rt] = 0;
    }
  }
  // Bounds shared by all rows: a tile inside [lo_max, hi_min] needs no mask.
  int lo_max, hi_min;
  {
    int i_first = row0 / a.G, i_last = (row0 + nrows - 1) / a.G;
    int pos_first = a.causal ? L - a.QL + i_first : L - 1;
    int pos_last = a.causal ? L - a.QL + i_last : L - 1;
    hi_min = min(pos_first, L - 1);
    lo_max = a.window > 0 ? max(0, pos_last - a.window + 1) : 0;
  }

  // ---- stage page ids (or token slots) of the item in LDS ----
  const int ppt = SPARSE ? TT : TT / ps;  // ids per tile
  const long id0 = SPARSE ? (long)tb * TT : (long)t0 / ps + (long)tb * ppt;
  const long id_end = SPARSE ? (long)hi_u : ((long)hi_u + ps - 1) / ps;  // one past the last valid id
  const int nstaged = (int)max(0L, min((long)a.stage_limit, min((long)(te - tb) * ppt, id_end - id0)));
  const int32_t* bt_row = a.block_tables + (long)s * a.table_stride;
  for (int k = tid; k < nstaged; k += NTHREADS) ids[k] = bt_row[id0 + k];

  // ---- query fragments ----
  // FP8 caches: d of MFMA step m, lane group g, slot p is 64(m/2)+16g+8(m%2)+p;
  // BF16 caches: 32m+8g+p.  Both read 8 contiguous d per (m, g).
  constexpr int NM = T::NM;
  constexpr int NDT = T::NDT;
  using QFrag = typename std::conditional<FP8, half8, bf16x8>::type;
  QFrag qf[NRT][NM];
  float crow[NRT];  // log2-domain score scale of the row (incl. query pre-scale)
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    int r = rt * 16 + c;
    bool valid = r < nrows;
    int gr = row0 + (valid ? r : 0);
    int i = gr / a.G, hl = gr % a.G;
    long qoff = (((long)s * a.QL + i) * a.Hq + (long)kvh * a.G + hl) * D;
    const uint16_t* qrow = (const uint16_t*)a.q + qoff;
    u32x4 raw[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      int d0 = FP8 ? 64 * (m >> 1) + 16 * g + 8 * (m & 1) : 32 * m + 8 * g;
      raw[m] = valid ? *(const u32x4*)(qrow + d0) : u32x4{0, 0, 0, 0};
    }
    if constexpr (FP8) {
      float amax = 0.f;
      float qv[NM][8];
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          uint32_t word = raw[m][p >> 1];
          uint16_t bits = (p & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFF);
          float f;
          if (a.q_fp16) {
            f = (float)__builtin_bit_cast(_Float16, bits);
          } else {
            f = __uint_as_float((uint32_t)bits << 16);
          }
          qv[m][p] = f;
          amax = fmaxf(amax, fabsf(f));
        }
      amax = group_max(amax);
      // BF16 rows are scaled by 2^e so |q| lands in [2^14, 2^15): exact in FP16.
      int e = 0;
      if (!a.q_fp16 && amax > 0.f && amax < INFINITY) {
        int ex;
        frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
        e = 15 - ex;
      }
      float mul = ldexpf(1.0f, e);
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int p = 0; p < 8; ++p) qf[rt][m][p] = (_Float16)(qv[m][p] * mul);
      crow[rt] = a.scale_log2 * ldexpf(1.0f, -e);
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m) qf[rt][m] = __builtin_bit_cast(bf16x8, raw[m]);
      crow[rt] = a.scale_log2;
    }
  }
  const bool per_token = FP8 && a.scale_mode == PA_SCALE_PER_TOKEN;
  float vs_ref = 1.0f;  // O holds sum p*v / vs_ref (per-token V scales)
  if (FP8 && !per_token) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) crow[rt] *= a.k_scale[0];
    vs_ref = a.v_scale[0];
  }
  if (per_token) vs_ref = 0.f;
  float inv_ref = per_token ? 0.f : 1.0f;

  // ---- online softmax state (lane holds row rt*16+c) ----
  float m_ref[NRT], l_part[NRT];
  f4 o[NRT][NDT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    m_ref[rt] = -INFINITY;
    l_part[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = f4{0.f, 0.f, 0.f, 0.f};
  }

  const uint8_t* kbase = a.k_cache + (long long)kvh * a.head_stride;
  const uint8_t* vbase = a.v_cache + (long long)kvh * a.head_stride;

  __syncthreads();  // staged ids visible

  // Page id (dense) or token slot (sparse) number j of the item.
  auto item_id = [&](long j) -> long {
    return j < nstaged ? (long)ids[j] : (long)bt_row[id0 + j];
  };

  // ---- tile loader: global -> registers ----
  auto load_tile = [&](int tile, Staged<D, FP8>& st) {
    const int ts = t0 + tile * TT;          // first token (index) of the tile
    const long jt = (long)(tile - tb) * ppt;  // first id of the tile within the item
    if constexpr (!SPARSE) {
      // K: unit u -> chunk cc = u / TT, token t = u % TT
      st.kmask = 0;
#pragma unroll
      for (int k = 0; k < T::KPT; ++k) {
        int u = tid + k * NTHREADS;
        int cc = u / TT, t = u % TT;
        int j = t / ps, slot = t % ps;
        int tok0 = ts + j * ps;
        bool ok = tok0 < hi_u && tok0 + ps > lo_u;
        st.k[k] = u32x4{0, 0, 0, 0};
        if (ok) {
          long pid = item_id(jt + j);
          const uint8_t* src = kbase + pid * a.page_stride + ((long)cc * ps + slot) * 16;
          st.k[k] = *(const u32x4*)src;
          st.kmask |= 1u << k;
        }
      }
      // V: unit u -> page j, row d, 16-byte unit within the row of the page
      const int n16 = ps * T::E / 16;  // 16-byte units per (row, page)
      st.vmask = 0;
#pragma unroll
      for (int k = 0; k < T::VPT; ++k) {
        int u = tid + k * NTHREADS;
        int per_page = D * n16;
        int j = u / per_page, rem = u % per_page;
        int d, s16;
        if (a.v_transposed) {
          s16 = rem / D;
          d = rem % D;
        } else {
          d = rem / n16;
          s16 = rem % n16;
        }
        int tok0 = ts + j * ps;
        bool ok = tok0 < hi_u && tok0 + ps > lo_u;
        st.v[k] = u32x4{0, 0, 0, 0};
        if (ok) {
          long pid = item_id(jt + j);
          long off = a.v_transposed ? ((long)s16 * D + d) * 16 : (long)d * ps * T::E + s16 * 16;
          st.v[k] = *(const u32x4*)(vbase + pid * a.page_stride + off);
          st.vmask |= 1u << k;
        }
      }
      if (FP8 && per_token && tid < 2 * TT / 4) {
        int which = tid / (TT / 4);  // 0: K scales, 1: V scales
        int t = (tid % (TT / 4)) * 4;
        int j = t / ps, slot = t % ps;
        int tok0 = ts + j * ps;
        st.s = u32x4{0, 0, 0, 0};
        st.sdst = which * TT + t;
        if (tok0 < hi_u && tok0 + ps > lo_u) {
          long pid = item_id(jt + j);
          const float* sc = which ? a.v_scale : a.k_scale;
          st.s = *(const u32x4*)(sc + (pid * (a.page_stride / (D * ps * T::E)) + kvh) * ps + slot);
        }
      }
    } else {
      // Sparse: every token has its own physical slot.
      const int nh = (int)(a.page_stride / a.head_stride);  // KV heads
      st.kmask = 0;
#pragma unroll
      for (int k = 0; k < T::KPT; ++k) {
        int u = tid + k * NTHREADS;
        int cc = u / TT, t = u % TT;
        st.k[k] = u32x4{0, 0, 0, 0};
        if (ts + t < hi_u) {
          long S = item_id(jt + t);
          long pid = S / ps;
          int slot = (int)(S % ps);
          st.k[k] = *(const u32x4*)(kbase + pid * a.page_stride + ((long)cc * ps + slot) * 16);
          st.kmask |= 1u << k;
        }
      }
      // V: unit u -> row d, 16 consecutive tokens (gathered element by element)
      st.vmask = 0;
#pragma unroll
      for (int k = 0; k < T::VPT; ++k) {
        int u = tid + k * NTHREADS;
        int upr = TT * T::E / 16;  // units per row
        int d = u / upr, t0u = (u % upr) * (16 / T::E);
        uint8_t bytes[16];
#pragma unroll
        for (int e = 0; e < 16 / T::E; ++e) {
          int t = t0u + e;
          if (ts + t < hi_u) {
            long S = item_id(jt + t);
            long pid = S / ps;
            int slot = (int)(S % ps);
            long off = a.v_transposed ? ((long)(slot / T::X) * D + d) * 16 + (slot % T::X) * T::E
                                      : ((long)d * ps + slot) * T::E;
            const uint8_t* src = vbase + pid * a.page_stride + off;
#pragma unroll
            for (int b = 0; b < T::E; ++b) bytes[e * T::E + b] = src[b];
          } else {
#pragma unroll
            for (int b = 0; b < T::E; ++b) bytes[e * T::E + b] = 0;
          }
        }
        std::memcpy(&st.v[k], bytes, 16);
        st.vmask |= 1u << k;
      }
      if (FP8 && per_token && tid < 2 * TT / 4) {
        int which = tid / (TT / 4);
        int t = (tid % (TT / 4)) * 4;
        st.sdst = which * TT + t;
        const float* sc = which ? a.v_scale : a.k_scale;
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = 0.f;
          if (ts + t + e < hi_u) {
            long S = item_id(jt + t + e);
            long pid = S / ps;
            int slot = (int)(S % ps);
            f[e] = sc[(pid * nh + kvh) * ps + slot];
          }
        }
        st.s = u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
      }
    }
  };

  // ---- registers -> LDS stage ----
  auto store_tile = [&](const Staged<D, FP8>& st, uint8_t* stg) {
    uint8_t* kl = stg;
    uint8_t* vl = stg + T::KBYTES;
    float* sl = (float*)(stg + T::KBYTES + T::VBYTES);
#pragma unroll
    for (int k = 0; k < T::KPT; ++k) {
      if (!(st.kmask & (1u << k))) continue;
      int u = tid + k * NTHREADS;
      int cc = u / TT, t = u % TT;
      *(u32x4*)(kl + cc * TT * 16 + kswz(t) * 16) = st.k[k];
    }
#pragma unroll
    for (int k = 0; k < T::VPT; ++k) {
      if (!(st.vmask & (1u << k))) continue;
      int u = tid + k * NTHREADS;
      int d, unit;  // destination row and 16-byte unit within the row
      if constexpr (SPARSE) {
        int upr = TT * T::E / 16;
        d = u / upr;
        unit = u % upr;
      } else {
        const int n16 = ps * T::E / 16;
        int per_page = D * n16;
        int j = u / per_page, rem = u % per_page, s16;
        if (a.v_transposed) {
          s16 = rem / D;
          d = rem % D;
        } else {
          d = rem / n16;
          s16 = rem % n16;
        }
        unit = j * n16 + s16;
      }
      uint8_t* row = vl + d * T::VROW;
      if constexpr (FP8) {
        int e = d & 15;
        u32x4 val = st.v[k];
        if (e & 1) val = u32x4{val[2], val[3], val[0], val[1]};
        *(u32x4*)(row + ((2 * unit) ^ (e & 14)) * 8) = val;
      } else {
        *(u32x4*)(row + (unit ^ (d & 15)) * 16) = st.v[k];
      }
    }
    if (FP8 && per_token && tid < 2 * TT / 4) *(u32x4*)(sl + st.sdst) = st.s;
  };

  // ---- main loop ----
  Staged<D, FP8> st;
  if (tb < te) {
    load_tile(tb, st);
    store_tile(st, stage_base);
  }
  for (int tile = tb; tile < te; ++tile) {
    __syncthreads();
    const int cur = (tile - tb) & 1;
    uint8_t* stg = stage_base + cur * T::STAGE;
    const bool more = tile + 1 < te;
    if (more) load_tile(tile + 1, st);

    const int ts = t0 + tile * TT;
    const int wt = ts + 32 * w;  // first token of this wave's 32
    const uint8_t* kl = stg;
    const uint8_t* vl = stg + T::KBYTES;
    const float* sl = (const float*)(stg + T::KBYTES + T::VBYTES);
    const bool interior = ts >= lo_max && ts + TT - 1 <= hi_min;

    if (wt < hi_u && wt + 32 > lo_u) {
      // --- S^T = K Q^T for the wave's 32 tokens: block b, row i <-> token 8(i/4)+4b+(i%4)
      f4 sacc[NRT][2];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) sacc[rt][0] = sacc[rt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        int tok = 32 * w + 8 * (c >> 2) + 4 * b + (c & 3);
        const uint8_t* krow = kl + kswz(tok) * 16;
        if constexpr (FP8) {
#pragma unroll
          for (int kk = 0; kk < D / 64; ++kk) {
            u32x4 raw = *(const u32x4*)(krow + (4 * kk + g) * TT * 16);
            half8 k0 = fp8x8_to_half8(u32x2{raw[0], raw[1]});
            half8 k1 = fp8x8_to_half8(u32x2{raw[2], raw[3]});
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt) {
              sacc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[rt][2 * kk], sacc[rt][b], 0, 0, 0);
              sacc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[rt][2 * kk + 1], sacc[rt][b], 0, 0, 0);
            }
          }
        } else {
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            u32x4 raw = *(const u32x4*)(krow + (4 * m + g) * TT * 16);
            bf16x8 kf = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
            for (int rt = 0; rt < NRT; ++rt)
              sacc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rt][m], sacc[rt][b], 0, 0, 0);
          }
        }
      }

      // --- per-token scales of the lane's 8 tokens (slot p = 4b + r <-> token 8g + p)
      const int tl = 32 * w + 8 * g;  // first of the lane's 8 tokens (tile-relative)
      float ks[8], vsn[8];
      if (per_token) {
        f4 k0 = *(const f4*)(sl + tl), k1 = *(const f4*)(sl + tl + 4);
        f4 v0 = *(const f4*)(sl + TT + tl), v1 = *(const f4*)(sl + TT + tl + 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ks[r] = k0[r];
          ks[4 + r] = k1[r];
          vsn[r] = v0[r];
          vsn[4 + r] = v1[r];
        }
      }
      // union validity of the lane's tokens (garbage outside it)
      const int tv = ts + tl;
      const int va = min(max(lo_u - tv, 0), 8), vb = min(max(hi_u - tv, 0), 8);  // valid slots [va, vb)
      if (per_token) {
#pragma unroll
        for (int p = 0; p < 8; ++p)
          if (p < va || p >= vb) vsn[p] = 0.f;
        float vmax = 0.f;
#pragma unroll
        for (int p = 0; p < 8; ++p) vmax = fmaxf(vmax, vsn[p]);
        vmax = group_max(vmax);
        // wave-uniform: every lane sees the same 32 tokens after the group max
        if (vmax > 0.f && (vmax > vs_ref * 16.f || vmax < vs_ref * (1.0f / 1024.f))) {
          float alpha = vs_ref / vmax;  // 0 on the first visit
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[rt][dt] *= alpha;
          vs_ref = vmax;
          inv_ref = 1.0f / vmax;
        }
      }

      // --- scale, mask, row max
      float x[NRT][8];
      float mx[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        mx[rt] = -INFINITY;
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          float v = sacc[rt][p >> 2][p & 3] * crow[rt];
          if (per_token) v *= ks[p];
          if (!interior) {
            int t = tv + p;
            if (t < lo_r[rt] || t > hi_r[rt]) v = -INFINITY;
          }
          x[rt][p] = v;
          mx[rt] = fmaxf(mx[rt], v);
        }
        mx[rt] = group_max(mx[rt]);
      }
      // --- lazy rescale when a row max grows past the band
      bool need = false;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) need |= mx[rt] > m_ref[rt] + TAU;
      if (__builtin_amdgcn_ballot_w64(need)) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          float alpha = 1.0f;
          if (mx[rt] > m_ref[rt] + TAU) {
            alpha = exp2f(m_ref[rt] - mx[rt]);  // 0 when m_ref is -inf
            m_ref[rt] = mx[rt];
          }
          l_part[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[rt][dt] *= alpha;
        }
      }
      // --- probabilities -> PV operand (registers only)
      using PFrag = typename std::conditional<FP8, half8, bf16x8>::type;
      PFrag pf[NRT];
      PFrag pl[NRT];  // BF16 caches: low part of a two-term split of P
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        float msafe = m_ref[rt] == -INFINITY ? 0.f : m_ref[rt];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          float pr = exp2f(x[rt][p] - msafe);
          l_part[rt] += pr;
          float u = per_token ? pr * (vsn[p] * inv_ref) : pr;
          if constexpr (FP8) {
            pf[rt][p] = (_Float16)u;
          } else {
            __bf16 hi = (__bf16)u;
            pf[rt][p] = hi;
            pl[rt][p] = (__bf16)(u - (float)hi);
          }
        }
      }
      // --- O^T += V^T P^T: V row d = 16dt + c, tokens 8g..8g+7 of the wave
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        int d = 16 * dt + c;
        const uint8_t* vrow = vl + d * T::VROW;
        if constexpr (FP8) {
          int unit = (4 * w + g) ^ c;
          u32x2 raw = *(const u32x2*)(vrow + unit * 8);
          if (va > 0 || vb < 8) {
            // bytes [va, vb) hold valid tokens; no shift by 64 (va or vb may be 8)
            uint64_t below_vb = vb >= 8 ? ~0ull : ((1ull << (8 * vb)) - 1);
            uint64_t below_va = va >= 8 ? ~0ull : ((1ull << (8 * va)) - 1);
            uint64_t keep = below_vb & ~below_va;
            raw[0] &= (uint32_t)keep;
            raw[1] &= (uint32_t)(keep >> 32);
          }
          half8 vf = fp8x8_to_half8(raw);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[rt], o[rt][dt], 0, 0, 0);
        } else {
          int unit = (4 * w + g) ^ c;
          u32x4 raw = *(const u32x4*)(vrow + unit * 16);
          if (va > 0 || vb < 8) {
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
              uint32_t keep = 0;
              if (2 * q2 >= va && 2 * q2 < vb) keep |= 0xFFFFu;
              if (2 * q2 + 1 >= va && 2 * q2 + 1 < vb) keep |= 0xFFFF0000u;
              raw[q2] &= keep;
            }
          }
          bf16x8 vf = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rt], o[rt][dt], 0, 0, 0);
            o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[rt], o[rt][dt], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_tile(st, stage_base + (cur ^ 1) * T::STAGE);
  }

  // ---- merge the four waves' states ----
  float l_row[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) l_row[rt] = group_sum(l_part[rt]);
  __syncthreads();  // all waves done with the stages (merge buffers alias them)
  float* wm = stats;                         // [NWAVES][NRT*16] m_ref
  float* wl = stats + NWAVES * NRT * 16;     // [NWAVES][NRT*16] l
  float* wr = stats + 2 * NWAVES * NRT * 16; // [NWAVES] v-scale reference
  float* rowinfo = wr + NWAVES;              // [NRT*16][4]: M, Ltot, out factor, flag
  if (g == 0) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      wm[w * NRT * 16 + rt * 16 + c] = m_ref[rt];
      wl[w * NRT * 16 + rt * 16 + c] = l_row[rt];
    }
  }
  if (lane == 0) wr[w] = vs_ref;
  __syncthreads();
  // weight of this wave's O for each of its rows
  float fw[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    int r = rt * 16 + c;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < NWAVES; ++ww)
      if (wl[ww * NRT * 16 + r] > 0.f) M = fmaxf(M, wm[ww * NRT * 16 + r]);
    fw[rt] = (l_row[rt] > 0.f) ? exp2f(m_ref[rt] - M) * vs_ref : 0.f;
  }
  if (tid < NRT * 16) {
    int r = tid;
    float M = -INFINITY, Lt = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWAVES; ++ww)
      if (wl[ww * NRT * 16 + r] > 0.f) M = fmaxf(M, wm[ww * NRT * 16 + r]);
#pragma unroll
    for (int ww = 0; ww < NWAVES; ++ww) {
      float lw = wl[ww * NRT * 16 + r];
      if (lw > 0.f) Lt += lw * exp2f(wm[ww * NRT * 16 + r] - M);
    }
    float factor = 0.f;  // direct output: out = O * factor
    if (Lt > 0.f) {
      if (a.has_sinks) {
        int gr = row0 + (r < nrows ? r : 0);
        int h = kvh * a.G + gr % a.G;
        float sk = a.sinks[h] * 1.4426950408889634f;
        float M2 = fmaxf(M, sk);
        float sc = exp2f(M - M2);
        factor = sc / (Lt * sc + exp2f(sk - M2));
      } else {
        factor = 1.0f / Lt;
      }
    }
    rowinfo[r * 4 + 0] = M;
    rowinfo[r * 4 + 1] = Lt;
    rowinfo[r * 4 + 2] = factor;
  }
  // O buffers: waves 0/1 write, waves 2/3 add
  constexpr int OROW = D + 4;
  float* obuf = (float*)stage_base;
  float* mine = obuf + (w & 1) * (NRT * 16 * OROW);
  if (w < 2) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *(f4*)(mine + (rt * 16 + c) * OROW + 16 * dt + 4 * g) = o[rt][dt] * fw[rt];
  }
  __syncthreads();
  if (w >= 2) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        f4* dst = (f4*)(mine + (rt * 16 + c) * OROW + 16 * dt + 4 * g);
        *dst = *dst + o[rt][dt] * fw[rt];
      }
  }
  __syncthreads();

  // ---- write: partial state or final rows ----
  const float* ob0 = obuf;
  const float* ob1 = obuf + NRT * 16 * OROW;
  if (it.slot >= 0) {
    float* sp = a.workspace + (size_t)it.slot * rpg * (2 + D);
    float* pm = sp;
    float* pl_ = sp + rpg;
    float* po = sp + 2 * rpg;
    if (tid < nrows) {
      pm[tid] = rowinfo[tid * 4 + 0];
      pl_[tid] = rowinfo[tid * 4 + 1];
    }
    for (int e = tid; e < nrows * (D / 4); e += NTHREADS) {
      int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
      f4 v = *(const f4*)(ob0 + r * OROW + d4) + *(const f4*)(ob1 + r * OROW + d4);
      *(f4*)(po + (size_t)r * D + d4) = v;
    }
  } else {
    for (int e = tid; e < nrows * (D / 4); e += NTHREADS) {
      int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
      f4 v = *(const f4*)(ob0 + r * OROW + d4) + *(const f4*)(ob1 + r * OROW + d4);
      v *= rowinfo[r * 4 + 2];
      int gr = row0 + r, i = gr / a.G, hl = gr % a.G;
      long ooff = (((long)s * a.QL + i) * a.Hq + (long)kvh * a.G + hl) * D + d4;
      uint16_t hv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (a.q_fp16)
          hv[k] = __builtin_bit_cast(uint16_t, (_Float16)v[k]);
        else
          hv[k] = __builtin_bit_cast(uint16_t, (__bf16)v[k]);
      }
      u32x2 packed = u32x2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
      *(u32x2*)((uint16_t*)a.out + ooff) = packed;
    }
  }
}

// ---------------------------------------------------------------------------
// Partition reducer: out = sum_p w_p O_p / (sum_p w_p l_p + [sink]), with
// w_p = 2^(m_p - M), M = max(m_p over parts with l_p > 0, sink), partitions
// added in order (deterministic).
// ---------------------------------------------------------------------------
struct ReduceArgs {
  void* out;
  const float* workspace;
  const float* sinks;
  const ReduceItem* entries;
  int QL, Hq, G, D, rows_total, rows_per_group, q_fp16, has_sinks;
};

__global__ __launch_bounds__(256) void pa_reduce_kernel(ReduceArgs a) {
  const ReduceItem e = a.entries[blockIdx.x];
  const int D = a.D, rpg = a.rows_per_group;
  const int row0 = e.rg * kMaxRowsPerItem;
  const int nrows = min(rpg, a.rows_total - row0);
  const size_t slot_f = (size_t)rpg * (2 + D);
  for (int idx = threadIdx.x; idx < nrows * (D / 4); idx += blockDim.x) {
    int r = idx / (D / 4), d4 = (idx % (D / 4)) * 4;
    float M = -INFINITY;
    for (int p = 0; p < e.nparts; ++p) {
      const float* sp = a.workspace + (size_t)(e.first_slot + p) * slot_f;
      if (sp[rpg + r] > 0.f) M = fmaxf(M, sp[r]);
    }
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (M > -INFINITY) {
      for (int p = 0; p < e.nparts; ++p) {
        const float* sp = a.workspace + (size_t)(e.first_slot + p) * slot_f;
        float lp = sp[rpg + r];
        if (!(lp > 0.f)) continue;
        float wgt = exp2f(sp[r] - M);
        den += wgt * lp;
        acc += wgt * *(const f4*)(sp + 2 * rpg + (size_t)r * D + d4);
      }
    }
    int gr = row0 + r, i = gr / a.G, hl = gr % a.G;
    int h = e.kvh * a.G + hl;
    f4 v = f4{0.f, 0.f, 0.f, 0.f};
    if (den > 0.f) {
      if (a.has_sinks) {
        float sk = a.sinks[h] * 1.4426950408889634f;
        float M2 = fmaxf(M, sk);
        float sc = exp2f(M - M2);
        v = acc * (sc / (den * sc + exp2f(sk - M2)));
      } else {
        v = acc * (1.0f / den);
      }
    }
    long ooff = (((long)e.seq * a.QL + i) * a.Hq + h) * D + d4;
    uint16_t hv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (a.q_fp16)
        hv[k] = __builtin_bit_cast(uint16_t, (_Float16)v[k]);
      else
        hv[k] = __builtin_bit_cast(uint16_t, (__bf16)v[k]);
    }
    *(u32x2*)((uint16_t*)a.out + ooff) =
        u32x2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
  }
}

// ---------------------------------------------------------------------------
// Launch selection
// ---------------------------------------------------------------------------
using KernelFn = void (*)(KernelArgs);

template <int D, bool FP8, int NRT, bool SPARSE>
static pa_status launch_one(const KernelArgs& args, int nblocks, hipStream_t stream) {
  constexpr int bytes = Smem<D, FP8, NRT>::TOTAL;
  static bool configured = false;
  if (!configured) {
    if (hipFuncSetAttribute((const void*)pa_decode_kernel<D, FP8, NRT, SPARSE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "hipFuncSetAttribute failed");
    }
    configured = true;
  }
  hipLaunchKernelGGL((pa_decode_kernel<D, FP8, NRT, SPARSE>), dim3(nblocks), dim3(NTHREADS), bytes, stream, args);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("decode launch failed: ") + hipGetErrorString(err));
  return PA_OK;
}

template <int D, bool FP8, int NRT>
static pa_status launch_sp(bool sparse, const KernelArgs& args, int n, hipStream_t st) {
  return sparse ? launch_one<D, FP8, NRT, true>(args, n, st) : launch_one<D, FP8, NRT, false>(args, n, st);
}
template <int D, bool FP8>
static pa_status launch_nrt(int nrt, bool sparse, const KernelArgs& args, int n, hipStream_t st) {
  if (nrt == 1) return launch_sp<D, FP8, 1>(sparse, args, n, st);
  if (nrt == 2) return launch_sp<D, FP8, 2>(sparse, args, n, st);
  return launch_sp<D, FP8, 4>(sparse, args, n, st);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_decode(const pa_plan_t* plan, void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                               const float* k_scale, const float* v_scale, const float* sinks, void* meta_dev,
                               void* workspace_dev, void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  const Plan& P = plan->plan;
  const pa_problem& p = P.prob;
  if (P.items.empty()) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return set_error(PA_ERR_INVALID, "a required device pointer is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return set_error(PA_ERR_INVALID, "q, out, k_cache and v_cache must be 16-byte aligned");
  if (p.kv_dtype == PA_FP8_E4M3FN) {
    if (!k_scale || !v_scale) return set_error(PA_ERR_INVALID, "FP8 caches need k_scale and v_scale");
    if (p.scale_mode == PA_SCALE_PER_TOKEN && (!aligned16(k_scale) || !aligned16(v_scale)))
      return set_error(PA_ERR_INVALID, "per-token scales must be 16-byte aligned");
  }
  if (p.has_sinks && !sinks) return set_error(PA_ERR_INVALID, "has_sinks set but sinks is NULL");
  if (!meta_dev) return set_error(PA_ERR_WORKSPACE, "meta_dev is NULL");
  if (P.num_slots > 0 && !workspace_dev) return set_error(PA_ERR_WORKSPACE, "workspace_dev is NULL");
  hipStream_t st = (hipStream_t)stream;
  if (P.uploaded_to != meta_dev) {
    if (hipMemcpyAsync(meta_dev, P.meta_host.data(), P.meta_host.size(), hipMemcpyHostToDevice, st) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "metadata upload failed");
    }
    P.uploaded_to = meta_dev;
  }
  const int elem = p.kv_dtype == PA_FP8_E4M3FN ? 1 : 2;
  KernelArgs args;
  args.out = out;
  args.q = q;
  args.k_cache = (const uint8_t*)k_cache;
  args.v_cache = (const uint8_t*)v_cache;
  args.block_tables = block_tables;
  args.context_lens = context_lens;
  args.k_scale = k_scale;
  args.v_scale = v_scale;
  args.sinks = sinks;
  args.items = (const WorkItem*)meta_dev;
  args.workspace = (float*)workspace_dev;
  args.head_stride = (long long)p.head_dim * p.page_size * elem;
  args.page_stride = args.head_stride * p.num_kv_heads;
  args.QL = p.query_len;
  args.Hq = p.num_q_heads;
  args.G = p.num_q_heads / p.num_kv_heads;
  args.page_size = p.page_size;
  args.table_stride = p.table_stride;
  args.window = p.sliding_window;
  args.causal = p.causal;
  args.v_transposed = p.v_layout == PA_V_TRANSPOSED;
  args.scale_mode = p.scale_mode;
  args.q_fp16 = p.q_dtype == PA_FP16;
  args.has_sinks = p.has_sinks;
  args.rows_total = P.rows_total;
  args.rows_per_group = P.rows_per_group;
  args.stage_limit = P.stage_limit;
  args.scale_log2 = P.scale_log2;
  const int n = (int)P.items.size();
  const bool sparse = p.token_table != 0;
  if (p.kv_dtype == PA_FP8_E4M3FN) {
    if (p.head_dim == 128) return launch_nrt<128, true>(P.nrt, sparse, args, n, st);
    return launch_nrt<256, true>(P.nrt, sparse, args, n, st);
  }
  return launch_nrt<128, false>(P.nrt, sparse, args, n, st);
}

extern "C" pa_status pa_reduce(const pa_plan_t* plan, void* out, const float* sinks, void* meta_dev,
                               void* workspace_dev, void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  const Plan& P = plan->plan;
  if (P.reduce.empty()) return PA_OK;
  if (!out) return set_error(PA_ERR_INVALID, "out is NULL");
  if (!aligned16(out)) return set_error(PA_ERR_INVALID, "out must be 16-byte aligned");
  if (P.prob.has_sinks && !sinks) return set_error(PA_ERR_INVALID, "has_sinks set but sinks is NULL");
  if (!meta_dev || !workspace_dev) return set_error(PA_ERR_WORKSPACE, "meta_dev or workspace_dev is NULL");
  if (P.uploaded_to != meta_dev) return set_error(PA_ERR_WORKSPACE, "meta_dev was not filled by pa_decode");
  ReduceArgs ra;
  ra.out = out;
  ra.workspace = (const float*)workspace_dev;
  ra.sinks = sinks;
  ra.entries = (const ReduceItem*)((const uint8_t*)meta_dev + P.items.size() * sizeof(WorkItem));
  ra.QL = P.prob.query_len;
  ra.Hq = P.prob.num_q_heads;
  ra.G = P.prob.num_q_heads / P.prob.num_kv_heads;
  ra.D = P.prob.head_dim;
  ra.rows_total = P.rows_total;
  ra.rows_per_group = P.rows_per_group;
  ra.q_fp16 = P.prob.q_dtype == PA_FP16;
  ra.has_sinks = P.prob.has_sinks;
  hipLaunchKernelGGL(pa_reduce_kernel, dim3((unsigned)P.reduce.size()), dim3(256), 0, (hipStream_t)stream, ra);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("reduce launch failed: ") + hipGetErrorString(err));
  return PA_OK;
}
