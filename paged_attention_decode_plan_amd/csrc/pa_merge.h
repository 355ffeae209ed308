// The partition merge of one (sequence, KV head, row group): out = sum_p w_p
// O_p / (sum_p w_p l_p + [sink]), w_p = 2^(m_p - M), M the largest m_p of the
// partitions with l_p > 0 (and the sink's logit), partitions added in order.
// The log-sum-exp merge of split-KV partials (aiter PR #4332, "Add
// paged-attention Tile kernel", pmax/psum/pout; aiter PR #7079, "Launch and
// reducer latency"), with sinks as in aiter PR #6617.
//
// One code path for both callers: the reducer kernel (one workgroup per
// chunk of rows) and the last-arriving work item of a decode launch with the
// in-kernel merge (the unit's chunks in turn, or a small unit at once).
// Each output gets the same operations in the same order from either (how
// many partitions' loads share a round trip differs, which changes no
// value): the two give bit-identical outputs.
#pragma once

#include "pa_device.h"

namespace pa {

// acc + w * v per component as one fused multiply-add, whatever the code
// around it: every merge variant rounds each partition's term the same way.
__device__ __forceinline__ f4 merge_term(f4 acc, float w, const f4& v) {
  return f4{__builtin_fmaf(w, v[0], acc[0]), __builtin_fmaf(w, v[1], acc[1]), __builtin_fmaf(w, v[2], acc[2]),
            __builtin_fmaf(w, v[3], acc[3])};
}

struct MergeArgs {
  void* out;
  const float* workspace;
  const float* sinks;
  int QL, Hq, G, rows_total, rows_per_group, q_fp16, has_sinks;
};

// Rows per merge chunk: one (row, 4-dim) output per thread of 256.
template <int D>
constexpr int merge_rows() { return 1024 / D; }

// LDS the in-kernel merge needs: weights (merge_chunk: [merge_rows]
// [kMaxPartitions]; merge_small: [64 rows][64 partitions]), row factors
// (64), plus one int that broadcasts the arrival.
template <int D>
constexpr int merge_wgt_floats() {
  return merge_rows<D>() * kMaxPartitions > 64 * 64 ? merge_rows<D>() * kMaxPartitions : 64 * 64;
}
template <int D>
constexpr int merge_lds_bytes() { return (merge_wgt_floats<D>() + 64 + 4) * 4; }

// Merges rows [chunk * RR, chunk * RR + RR) of unit e.  Every thread of the
// workgroup must call it (it holds one barrier); threads 256 and up only take
// part in the barrier.  wgt: RR * kMaxPartitions floats of LDS, rowf: RR.
// RCH: partitions whose loads are in flight per round trip.  The order of
// the operations on each output does not depend on it.
template <int D, int RCH>
__device__ __forceinline__ void merge_chunk(const MergeArgs& a, const ReduceItem& e, int chunk, float* wgt,
                                            float* rowf) {
  // no contraction of a*b+c into FMAs at the compiler's choice, which
  // differs with the surrounding code: the fused operations are explicit
#pragma clang fp contract(off)
  constexpr int RR = merge_rows<D>();
  constexpr int Q4 = D / 4;
  static_assert(RR * Q4 == 256, "one output per thread");
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  const int rpg = a.rows_per_group;
  const int row0 = e.rg * kMaxRowsPerItem;
  const int nrows = min(rpg, a.rows_total - row0);
  const int r0 = chunk * RR;
  const size_t slot_f = (size_t)rpg * (2 + D);
  const int np = e.nparts;
  const float* base = a.workspace + (size_t)e.first_slot * slot_f;
  // The thread's output (row rr, 4 dims d4).  Its partial O for the first RCH
  // partitions is loaded before the weights are known, so that the merge
  // costs one round trip to memory for up to RCH partitions.
  const int rr = act ? tid / Q4 : 0, d4 = (tid % Q4) * 4;
  const int r = r0 + rr;
  const float* po = base + 2 * rpg + (size_t)min(r, nrows - 1) * D + d4;
  f4 v0[RCH];
  if (act) {
#pragma unroll
    for (int j = 0; j < RCH; ++j) v0[j] = *(const f4*)(po + (size_t)min(j, np - 1) * slot_f);
  }
  // per-row weights: wave w takes rows w, w + 4, ..., lanes over partitions
  // (p = lane + 64k); the rows' (max, sum) loads are issued together
  if (act) {
    constexpr int XR = (RR + 3) / 4;  // rows per wave (head dim 512: two rows, waves 2 and 3 idle)
    const int wv = tid >> 6, lane = tid & 63;
    float mv[XR][4], lv[XR][4], skv[XR];
#pragma unroll
    for (int x = 0; x < XR; ++x) {
      const int rx = min(r0 + wv + 4 * x, nrows - 1);
      skv[x] = a.has_sinks ? a.sinks[e.kvh * a.G + (row0 + rx) % a.G] : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float* sp = base + (size_t)min(lane + 64 * k, np - 1) * slot_f;
        mv[x][k] = sp[rx];
        lv[x][k] = sp[rpg + rx];
      }
    }
#pragma unroll
    for (int x = 0; x < XR; ++x) {
      const int rw = wv + 4 * x;
      if (rw >= RR || r0 + rw >= nrows) continue;  // wave-uniform
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (lane + 64 * k < np && lv[x][k] > 0.f) M = fmaxf(M, mv[x][k]);
      M = wave_max(M);
      float den = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int p = lane + 64 * k;
        if (p < np) {
          const float wp = lv[x][k] > 0.f ? __builtin_amdgcn_exp2f(mv[x][k] - M) : 0.f;
          wgt[rw * kMaxPartitions + p] = wp;
          den = __builtin_fmaf(wp, lv[x][k], den);
        }
      }
      den = wave_sum(den);  // fixed-order sum of the denominator terms
      if (lane == 0) {
        float f = 0.f;
        if (den > 0.f) {
          if (a.has_sinks) {
            const float sk = skv[x] * LOG2E;
            const float M2 = fmaxf(M, sk);
            const float sc = __builtin_amdgcn_exp2f(M - M2);
            f = sc / __builtin_fmaf(den, sc, __builtin_amdgcn_exp2f(sk - M2));  // fused in every caller
          } else {
            f = 1.0f / den;
          }
        }
        rowf[rw] = f;
      }
    }
  }
  __syncthreads();
  if (!act || r >= nrows) return;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  const float f = rowf[rr];
  if (f > 0.f) {
    // partitions in order, RCH loads in flight at a time (the first RCH are
    // already in v0); partitions without visible tokens are skipped by a
    // select, not a branch
    for (int p0 = 0; p0 < np; p0 += RCH) {
      f4 v[RCH];
      if (p0 == 0) {
#pragma unroll
        for (int j = 0; j < RCH; ++j) v[j] = v0[j];
      } else {
#pragma unroll
        for (int j = 0; j < RCH; ++j) v[j] = *(const f4*)(po + (size_t)min(p0 + j, np - 1) * slot_f);
      }
#pragma unroll
      for (int j = 0; j < RCH; ++j) {
        const float wp = p0 + j < np ? wgt[rr * kMaxPartitions + p0 + j] : 0.f;
        if (wp != 0.f) acc = merge_term(acc, wp, v[j]);
      }
    }
  }
  const f4 v = acc * f;
  const int gr = row0 + r, i = gr / a.G, hl = gr % a.G;
  const int h = e.kvh * a.G + hl;
  const long ooff = (((long)e.seq * a.QL + i) * a.Hq + h) * D + d4;
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

// merge_chunk with the round-trip width chosen by the partition count (a
// unit of up to 32 partitions in one round trip): the reducer's choice.
template <int D>
__device__ __forceinline__ void merge_chunk_any(const MergeArgs& a, const ReduceItem& e, int chunk, float* wgt,
                                                float* rowf) {
  if (e.nparts <= 16)
    merge_chunk<D, 16>(a, e, chunk, wgt, rowf);
  else
    merge_chunk<D, 32>(a, e, chunk, wgt, rowf);
}

// The whole unit in one round trip to memory, for units of at most 64
// partitions whose partial O fits SMALL_LOADS 16-byte loads per thread:
// every thread loads all partitions of its outputs (output o = tid + 256 j,
// row o / (D/4)) together with the rows' (max, sum), then merges.  Per
// output the operations and their order are merge_chunk's (weights from the
// same wave-wide max and sum over lanes = partitions, partitions added in
// order, zero weights skipped), so the outputs are bit-identical to it.
constexpr int SMALL_LOADS = 8;
template <int D>
__device__ __forceinline__ bool merge_fits_small(int nrows, int np) {
  return np <= 64 && (long)((nrows * (D / 4) + 255) / 256) * np <= SMALL_LOADS;
}
template <int D>
__device__ __forceinline__ void merge_small(const MergeArgs& a, const ReduceItem& e, float* wgt, float* rowf) {
#pragma clang fp contract(off)  // as in merge_chunk
  constexpr int Q4 = D / 4;
  const int tid = threadIdx.x;
  const bool act = tid < 256;
  const int rpg = a.rows_per_group;
  const int row0 = e.rg * kMaxRowsPerItem;
  const int nrows = min(rpg, a.rows_total - row0);
  const size_t slot_f = (size_t)rpg * (2 + D);
  const int np = e.nparts;
  const int nout = nrows * Q4;
  const float* base = a.workspace + (size_t)e.first_slot * slot_f;
  f4 v[SMALL_LOADS];
  if (act) {
#pragma unroll
    for (int k = 0; k < SMALL_LOADS; ++k) {
      const int o = min(tid + 256 * (k / np), nout - 1), p = k % np;
      v[k] = *(const f4*)(base + (size_t)p * slot_f + 2 * rpg + (size_t)(o / Q4) * D + (o % Q4) * 4);
    }
  }
  // per-row weights: wave w takes rows w, w + 4, ..., lane p partition p
  constexpr int XR = kMaxRowsPerItem / 4;
  if (act) {
    const int wv = tid >> 6, lane = tid & 63;
    float mv[XR], lv[XR], skv[XR];
    const float* sp = base + (size_t)min(lane, np - 1) * slot_f;
#pragma unroll
    for (int x = 0; x < XR; ++x) {
      const int rx = min(wv + 4 * x, nrows - 1);
      skv[x] = a.has_sinks ? a.sinks[e.kvh * a.G + (row0 + rx) % a.G] : 0.f;
      mv[x] = sp[rx];
      lv[x] = sp[rpg + rx];
    }
#pragma unroll
    for (int x = 0; x < XR; ++x) {
      const int rw = wv + 4 * x;
      if (rw >= nrows) break;  // wave-uniform
      float M = -INFINITY;
      if (lane < np && lv[x] > 0.f) M = fmaxf(M, mv[x]);
      M = wave_max(M);
      float den = 0.f;
      if (lane < np) {
        const float wp = lv[x] > 0.f ? __builtin_amdgcn_exp2f(mv[x] - M) : 0.f;
        wgt[rw * 64 + lane] = wp;
        den = __builtin_fmaf(wp, lv[x], den);
      }
      den = wave_sum(den);  // fixed-order sum of the denominator terms
      if (lane == 0) {
        float f = 0.f;
        if (den > 0.f) {
          if (a.has_sinks) {
            const float sk = skv[x] * LOG2E;
            const float M2 = fmaxf(M, sk);
            const float sc = __builtin_amdgcn_exp2f(M - M2);
            f = sc / __builtin_fmaf(den, sc, __builtin_amdgcn_exp2f(sk - M2));  // fused in every caller
          } else {
            f = 1.0f / den;
          }
        }
        rowf[rw] = f;
      }
    }
  }
  __syncthreads();
  if (!act) return;
  const int nj = (nout + 255) / 256;
  for (int j = 0; j < nj; ++j) {
    const int o = tid + 256 * j;
    if (o >= nout) break;
    const int r = o / Q4, d4 = (o % Q4) * 4;
    f4 acc = f4{0.f, 0.f, 0.f, 0.f};
    const float f = rowf[r];
    if (f > 0.f) {
#pragma unroll
      for (int k = 0; k < SMALL_LOADS; ++k) {
        if (k / np == j) {
          const float wp = wgt[r * 64 + k % np];
          if (wp != 0.f) acc = merge_term(acc, wp, v[k]);
        }
      }
    }
    const f4 w = acc * f;
    const int gr = row0 + r, i = gr / a.G, hl = gr % a.G;
    const long ooff = (((long)e.seq * a.QL + i) * a.Hq + e.kvh * a.G + hl) * D + d4;
    uint16_t hv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (a.q_fp16)
        hv[k] = __builtin_bit_cast(uint16_t, (_Float16)w[k]);
      else
        hv[k] = __builtin_bit_cast(uint16_t, (__bf16)w[k]);
    }
    *(u32x2*)((uint16_t*)a.out + ooff) =
        u32x2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
  }
}

// The in-kernel merge of a decode work item that wrote partial slot
// it.slot: every item of the unit counts its arrival on the unit's counter
// (one 128-byte line per unit, indexed by its first slot, zero between
// calls); the last to arrive merges the unit's partials and resets the
// counter.  Partials are released at agent scope before the count and
// acquired with it, so the last arriver reads every other item's stores
// whichever XCD wrote them.  Every thread of the workgroup calls it after
// its own partial stores; lds: merge_lds_bytes<D>() bytes no thread still
// reads.
template <int D>
__device__ __forceinline__ void arrive_and_merge(const MergeArgs& ma, int* counters, const WorkItem& it,
                                                 uint8_t* lds) {
  float* wgt = (float*)lds;
  float* rowf = wgt + merge_wgt_floats<D>();
  int* lastf = (int*)(rowf + 64);
  const int first = it.slot - it.part;
  // Every wave's partial stores have reached the XCD's L2 before the
  // barrier; one release by thread 0 then writes them back (the L2
  // write-back covers the whole workgroup's stores), and the last arriver's
  // acquire invalidates its CU's and XCD's caches for the merge's loads:
  // one write-back per work item and one invalidate per unit.
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    int* ctr = counters + (size_t)first * 32;
    const int before = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const int last = before == it.nparts - 1;
    if (last) {
      // only the merging item invalidates its caches: the others' cached
      // data (a sparse batch's gathered pool) stays
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *lastf = last;
  }
  __syncthreads();
  if (!*lastf) return;  // workgroup-uniform
  const ReduceItem e{it.seq, it.kvh, it.rg, first, it.nparts, 0, 0, 0};
  const int nrows = min(ma.rows_per_group, ma.rows_total - it.rg * kMaxRowsPerItem);
  if (merge_fits_small<D>(nrows, it.nparts)) {
    merge_small<D>(ma, e, wgt, rowf);
    return;
  }
  const int nchunks = (nrows + merge_rows<D>() - 1) / merge_rows<D>();
  for (int ch = 0; ch < nchunks; ++ch) {
    merge_chunk<D, 16>(ma, e, ch, wgt, rowf);
    __syncthreads();  // the chunk's weights read before the next chunk writes them
  }
}

}  // namespace pa
