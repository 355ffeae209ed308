// gfx950 streaming decode kernel for page tables and work items of 17..64
// query rows (multi-token (MTP) verify rows times a GQA group): FP8 caches at
// head dim 128 with one 32-row block (RB = 1) or two (RB = 2) and at head dim
// 256 with one; BF16 caches at head dim 128 with pages of 32 tokens or more
// (BF, at the end of this comment).
//
// Same method as the tile kernel (online softmax per partition, partials
// merged in a fixed order by the reducer or by the unit's last-arriving work
// item: aiter PR #4332 "Add paged-attention Tile kernel" and aiter PR #7079,
// "Launch and reducer latency" and "Partition merges"; scale before mask:
// aiter PR #6617), laid out differently for bandwidth:
//
//  * a workgroup has 4 waves and owns one work item; each 128-token tile of
//    the item is cut into four 32-token steps and wave w takes step w of every
//    tile, for all of the item's query rows;
//  * a wave loads its K, V and per-token scales straight into registers with
//    16-byte global loads (no LDS staging: on this part LDS-DMA streaming
//    tops out well below what register loads reach), three steps ahead of
//    the step it computes (three register buffers, steps taken in groups of
//    three), so the waves never synchronise inside the loop;
//  * QK^T runs on v_mfma_scale_f32_32x32x64_f8f6f4 with K as stored (FP8)
//    against two FP8 terms of the query (hi and a 16x residual, each with
//    its own E8M0 block scale), softmax_scale * log2(e) (and a per-tensor k
//    scale) folded in, so the accumulator holds base-2 logits; per-token k
//    scales multiply them in the FMA that also subtracts the reference
//    maximum;
//  * the QK row of MFMA output register i in lane half h is token 16h + i of
//    the step (the K rows are fed in that order), which is exactly the token
//    order of the lane's slots in the PV operand: probabilities go from the
//    QK accumulator to the PV operand in registers;
//  * probabilities are taken against a per-row reference maximum set at
//    the row's first visible tokens (a score more than TAU_S above it makes
//    the wave redo its share with a larger reference, so the accumulator is
//    only ever written by MFMAs);
//  * PV runs on v_mfma_f32_32x32x16_f16: with per-token scales, the step's
//    largest V scale sets a power of two 2^E; V converts exactly to FP16 as
//    v * 2^E, and each probability times its token's V scale * 2^-E (at most
//    1 unless E hit its clamp) is rounded once to FP16 (11 significant bits);
//    an operand that would reach 2^15 makes the wave restart;
//  * BF16 caches: QK on v_mfma_f32_32x32x16_bf16 with K as stored against
//    the BF16 query (staged once in LDS in the operand's lane order), PV on
//    the same instruction with V as stored against a two-term BF16 split of
//    the probabilities (hi, then the residual), two load buffers per wave.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_merge.h"

namespace pa {

constexpr int SW = 4;  // waves per workgroup
// Scores may exceed a row's reference maximum by this much (base 2) before
// the wave restarts: a probability (times a V scale normalised to below 1)
// then stays below 2^15, inside FP16.
constexpr float TAU_S = 15.0f;
// The V conversion scale 2^E of a step is clamped to [2^-15, 2^6]: every FP8
// value times it is exact in FP16 (the smallest subnormal lands on 2^-24, the
// largest finite value stays below 2^15).
constexpr int VEXP_MIN = -15, VEXP_MAX = 6;

template <int D, int RB>
struct StreamSmem {
  static constexpr int ROWS = 32 * RB;
  static constexpr int OROW = D + 4;  // padded O row, floats
  static constexpr int OBUF = ROWS * OROW * 4;
  static constexpr int MERGE = SW * OBUF;  // one O buffer per wave
  static constexpr int IDS = kStageCap * 4;
  static constexpr int SCALES = SW * 64 * 4;  // per wave: 32 k scales, 32 v scales of its step
  static constexpr int STATS = (SW * ROWS * 2 + SW + ROWS * 4) * 4;
  static constexpr int TOTAL = MERGE + IDS + SCALES + STATS;
  // Requested at launch: more than half of a CU's 160 KB, so that the
  // dispatcher places one workgroup per CU (the plan's budget) also for one
  // row block, whose own footprint would let two share a CU.
  static constexpr int LAUNCH = TOTAL > 81 * 1024 ? TOTAL : 81 * 1024;
};

// Step data of one wave, loaded NB - 1 steps ahead.
//   FP8:  k[ks] (64 dims): K chunks 4ks + 2h, 4ks + 2h + 1 (dims 64ks + 32h
//         .. +31) of token kt; v[db]: V dim 32db + c32, tokens 16h .. 16h+15;
//   BF16: k[ks] (16 dims): K chunk 2ks + h (dims 16ks + 8h .. +7) of token
//         kt; v[2db + kb]: V dim 32db + c32, tokens 16h + 8kb .. +7.
template <int D, bool BF>
struct StepData {
  typename std::conditional<BF, u32x4, i32x8>::type k[BF ? D / 16 : D / 64];
  u32x4 v[BF ? D / 16 : D / 32];
  float sc;  // lanes 0-31: k scale of token c32; lanes 32-63: v scale of token c32
};


__device__ __forceinline__ i32x8 load32(const uint8_t* p0, const uint8_t* p1) {
  const u32x4 lo = *(const u32x4*)p0, hi = *(const u32x4*)p1;
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// BIG: page size >= 32 (the 32 tokens of a step share one page).
// BF: BF16 caches (head dim 128, pages of 32 tokens or more, no scales): QK
// on v_mfma_f32_32x32x16_bf16 with the BF16 query and K as stored, PV on the
// same instruction with V as stored against a two-term BF16 split of P.
template <int D, int RB, bool PT, bool BIG, bool BF = false>
__global__ __launch_bounds__(256) void pa_stream_kernel(KernelArgs a) {
  constexpr int TT = kTileTokens;
  using S = StreamSmem<D, RB>;
  constexpr int NKS = BF ? D / 16 : D / 64;  // QK k-steps (64 dims each; BF16: 16)
  constexpr int NDB = D / 32;                // 32-dim blocks of V and O
  // Load buffers per wave: three at head dim 128 (FP8); two at 256 and for
  // BF16 caches, whose steps are twice the bytes (the same bytes in flight)
  // and, at 256, whose O accumulator is twice the registers.
  constexpr int NB = (D == 128 && !BF) ? 3 : 2;
  static_assert(D == 128 || (D == 256 && RB == 1), "head dim 256 takes one 32-row block");
  static_assert(!BF || (D == 128 && !PT && BIG), "BF16: head dim 128, no scales, pages of 32 tokens or more");
  using SD = StepData<D, BF>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* obuf = (float*)smem;
  static_assert(merge_lds_bytes<D>() <= S::MERGE, "the in-kernel merge reuses the O buffers");
  int32_t* ids = (int32_t*)(smem + S::MERGE);
  float* sbuf = (float*)(smem + S::MERGE + S::IDS);
  float* stats = (float*)(smem + S::MERGE + S::IDS + S::SCALES);

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);  // the same, known wave-uniform
  const int lane = tid & 63;
  const int c32 = lane & 31;
  const int h = lane >> 5;

  const WorkItem it = a.items[blockIdx.x];
  const MetaHeader mh = *a.meta;
  if (!meta_ok(mh, a.tag_lo, a.tag_hi)) return;  // not this plan's list: touch nothing
  if (it.seq < 0) return;  // an unused item of a refreshable plan
  const int s = it.seq, kvh = it.kvh, rg = it.rg;
  const int ps = a.page_size;   // tokens per (sub-)page: pages above 128 are sub-pages of 128
  const int pps = a.phys_page;  // physical page size: strides inside a page
  const int psub = a.page_sub;  // sub-pages per page = 2^psub
  const int ps_log2 = 31 - __builtin_clz(ps);
  const long cap = (long)a.table_stride * pps;
  const int L = (int)min(max((long)a.context_lens[s], 0L), cap);

  // Visible span of the sequence (union over its query rows).
  int lo_u = 0, hi_u = L;
  if (L > 0 && a.window > 0) {
    const int first_pos = a.causal ? L - a.QL : L - 1;
    lo_u = max(0, first_pos - a.window + 1);
  }
  const int t0 = (lo_u >> ps_log2) << ps_log2;
  const int ntiles = hi_u > lo_u ? (hi_u - t0 + TT - 1) / TT : 0;
  const int tb = min(it.tile_begin, ntiles);
  const int te = it.tile_end < 0 ? ntiles : min(it.tile_end, ntiles);

  // Rows: lane holds row 32rb + c32 of the item for rb < RB.
  const int rpg = a.rows_per_group;
  const int row0 = rg * kMaxRowsPerItem;
  const int nrows = min(rpg, a.rows_total - row0);
  int lo_r[RB], hi_r[RB];
  bool valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 32 * rb + c32;
    valid[rb] = r < nrows;
    if (valid[rb]) {
      const int i = (row0 + r) / a.G;
      const int pos = a.causal ? L - a.QL + i : L - 1;
      hi_r[rb] = min(pos, L - 1);
      lo_r[rb] = a.window > 0 ? max(0, pos - a.window + 1) : 0;
    } else {
      lo_r[rb] = 1;
      hi_r[rb] = 0;
    }
  }
  // A tile inside [lo_max, hi_min] is visible to every row of the item.
  int lo_max, hi_min;
  {
    const int i_first = row0 / a.G, i_last = (row0 + nrows - 1) / a.G;
    const int pos_first = a.causal ? L - a.QL + i_first : L - 1;
    const int pos_last = a.causal ? L - a.QL + i_last : L - 1;
    hi_min = min(pos_first, L - 1);
    lo_max = a.window > 0 ? max(0, pos_last - a.window + 1) : 0;
  }

  // ---- the item's page-id range ----
  const int ppt = TT >> ps_log2;  // pages per tile
  const long id0 = ((long)t0 >> ps_log2) + (long)tb * ppt;
  const long id_end = ((long)hi_u + ps - 1) >> ps_log2;  // one past the last page with visible tokens
  const int nstaged = (int)max(0L, min((long)a.stage_limit, min((long)(te - tb) * ppt, id_end - id0)));
  const int32_t* bt_row = a.block_tables + (long)s * a.table_stride;

  // ---- the query rows' raw bits (issued first: their wait does not cover the K/V loads) ----
  constexpr int QP = D / 32;                    // threads per row, 32 dims each
  const int q_r = tid / QP, q_qq = tid % QP;    // 256 / QP rows (64 or 32)
  const bool q_valid = q_r < nrows && q_r < S::ROWS;
  u32x4 qraw[4];
  {
    const int gr = row0 + (q_valid ? q_r : 0);
    const int i = gr / a.G, hl = gr % a.G;
    const long qoff = (((long)s * a.QL + i) * a.Hq + (long)kvh * a.G + hl) * D + 32 * q_qq;
    const uint16_t* qrow = (const uint16_t*)a.q + qoff;
#pragma unroll
    for (int part = 0; part < 4; ++part) qraw[part] = *(const u32x4*)(qrow + 8 * part);  // padding rows read row 0
  }

  // ---- the item's page ids, read before the K/V loads (their wait does not
  // cover those), staged in LDS once the query is prepared ----
  static_assert(kStageCap == 4 * 256, "four ids per thread");
  int32_t idr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const long k = min((long)(tid + 256 * j), (long)max(nstaged - 1, 0));
    const long jj = min(max(id0 + k, 0L), ((long)a.table_stride << psub) - 1);  // in the row whatever the item
    idr[j] = (bt_row[jj >> psub] << psub) | (int)(jj & ((1 << psub) - 1));
  }

  // ---- the first three steps' loads ----
  // Issued before the query is prepared, with page ids read straight from
  // the block table, so that their latency overlaps the query work.
  const uint8_t* kbase = a.k_cache + (long long)kvh * a.head_stride;
  const uint8_t* vbase = a.v_cache + (long long)kvh * a.head_stride;
  // ---- loads of one step ----
  // QK A-operand row c32 is token kt of the step: MFMA output register i of
  // lane half h is then token 16h + i, and lane (c32, h) loads V of dim
  // 32db + c32 for exactly those 16 tokens (into both halves of its operand).
  const int kt = ((c32 >> 2) & 1) * 16 + (c32 >> 3) * 4 + (c32 & 3);
  auto page_ok = [&](long j) {  // id index j (relative to id0) holds visible tokens
    const long tok0 = (long)t0 + ((j + (long)tb * ppt) << ps_log2);
    return tok0 < hi_u && tok0 + ps > lo_u;
  };
  // Lane-constant parts of the addresses (page >= 32: a step lies in one page)
  const int slot_k = (32 * w + kt) & (ps - 1);
  // the lane's first K chunk: 2h (FP8: chunks 2h, 2h+1 of every 64 dims), h (BF16: chunk h of every 16 dims)
  const uint32_t koff = (uint32_t)(((BF ? 1 : 2) * h * pps + slot_k) * 16);
  const uint32_t kcs = (uint32_t)pps * 16;  // K chunk stride
  const int slot_v = (32 * w + 16 * h) & (ps - 1);
  // V: the lane's 16 tokens of dim 32db + c32 (BF16: two 16-byte halves,
  // vkb apart)
  constexpr int X = BF ? 8 : 16;  // tokens per 16-byte unit of transposed V
  uint32_t voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dd = 32 * db + c32;
    voff[db] = a.v_transposed ? (uint32_t)(((slot_v / X) * D + dd) * 16)
                              : (uint32_t)((dd * pps + slot_v) * (BF ? 2 : 1));
  }
  const uint32_t vkb = a.v_transposed ? (uint32_t)D * 16 : 16u;
  const uint32_t soff = (uint32_t)((kvh * pps + ((32 * w + c32) & (ps - 1))) * 4);
  // A (sub-)page id's place in the caches and scales: its page's block plus
  // the sub-page's offset (K: tokens in every chunk; plain V: columns of
  // every row; transposed V: its 16-token blocks; scales: tokens).
  const long msk = (1L << psub) - 1;
  const long vsub_bytes = a.v_transposed ? (long)(ps / X) * D * 16 : (long)ps * (BF ? 2 : 1);
  auto kpage = [&](long id) { return (id >> psub) * a.page_stride + (id & msk) * ps * 16; };
  auto vpage = [&](long id) { return (id >> psub) * a.page_stride + (id & msk) * vsub_bytes; };
  const float* sbase = h ? a.v_scale : a.k_scale;

  // Page ids of a step, wave-uniform: the step's page (page >= 32), or its
  // two pages (page 16: tokens 0-15 and 16-31 of the step).
  struct StepPages {
    long a, b;
  };
  auto load_k = [&](SD& d, StepPages id) {
    if constexpr (BF) {
      const uint8_t* kp = kbase + kpage(id.a);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) d.k[ks] = *(const u32x4*)(kp + koff + 2 * ks * kcs);
    } else if constexpr (BIG) {
      const uint8_t* kp = kbase + kpage(id.a);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) d.k[ks] = load32(kp + koff + 4 * ks * kcs, kp + koff + (4 * ks + 1) * kcs);
      if constexpr (PT)
        d.sc = *(const float*)((const uint8_t*)(sbase + (id.a >> psub) * a.Hkv * pps + (id.a & msk) * ps) + soff);
    } else {
      // page 16: token kt of the step is slot kt & 15 of its first or second page
      const long idk = kt >= 16 ? id.b : id.a;
      const uint8_t* src = kbase + idk * a.page_stride + (long)(kt & 15) * 16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) d.k[ks] = load32(src + (2 * h + 4 * ks) * kcs, src + (2 * h + 4 * ks + 1) * kcs);
      if constexpr (PT) {
        const long ids_ = c32 >= 16 ? id.b : id.a;
        d.sc = sbase[(ids_ * a.Hkv + kvh) * ps + (c32 & 15)];
      }
    }
    if constexpr (!PT) d.sc = 0.f;
  };
  auto load_v = [&](SD& d, StepPages id) {
    if constexpr (BF) {
      const uint8_t* vp = vbase + vpage(id.a);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) d.v[2 * db + kb] = *(const u32x4*)(vp + voff[db] + kb * vkb);
    } else if constexpr (BIG) {
      const uint8_t* vp = vbase + vpage(id.a);
#pragma unroll
      for (int db = 0; db < NDB; ++db) d.v[db] = *(const u32x4*)(vp + voff[db]);
    } else {
      const uint8_t* pg = vbase + (h ? id.b : id.a) * a.page_stride;  // the lane's 16 tokens: one page
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint8_t* src = pg + (long)(32 * db + c32) * 16;  // page 16: both V layouts put a dim's 16 bytes here
        d.v[db] = *(const u32x4*)src;
      }
    }
  };

  const __attribute__((address_space(4))) int32_t* btc =
      (const __attribute__((address_space(4))) int32_t*)bt_row;
  auto step_pages_direct = [&](int k) -> StepPages {  // step k's page ids from the block table
    const long j = (long)((k - tb) * TT + 32 * wu) >> ps_log2;
    StepPages r{0, 0};
    if (page_ok(j)) r.a = ((long)btc[(id0 + j) >> psub] << psub) | ((id0 + j) & msk);
    if (!BIG && page_ok(j + 1)) r.b = btc[id0 + j + 1];  // page 16: no sub-pages
    return r;
  };
  // Unconditional, so that the compiler's wait counts stay exact: an empty
  // item (tb >= te) reads page 0 of its head, which exists (the host routes
  // caches without pages elsewhere), and never uses the data.
  SD ba, bb, bc;  // bc: three buffers only
  {
    const int k1 = min(tb + 1, te - 1), k2 = min(tb + 2, te - 1);
    const StepPages p0 = step_pages_direct(tb);
    const StepPages p1 = step_pages_direct(k1);
    load_k(ba, p0);
    load_v(ba, p0);
    load_k(bb, p1);
    load_v(bb, p1);
    if constexpr (NB == 3) {
      const StepPages p2 = step_pages_direct(k2);
      load_k(bc, p2);
      load_v(bc, p2);
    }
  }

  // ---- query operand: two FP8 terms per row with a power-of-two scale ----
  // Row r is scaled by c = softmax_scale*log2(e) (* k_scale for per-tensor
  // scales) and by 2^-e, e chosen so that |c q / 2^e| <= 448; the terms
  // hi = fp8(c q / 2^e) and lo = fp8(16 (c q / 2^e - hi)) carry the row to
  // within 2^-8 of each element (RNE: half an FP8 ulp of the residual) and
  // enter the MFMA with the E8M0 block scales 2^e and 2^(e-4), so the
  // accumulator holds base-2 logits in FP32 with K taken exactly as stored.
  // The workgroup splits the rows once into LDS (thread = row tid/4, dims
  // 32*(tid%4) ..+31), laid out as the reading lanes want them: lane half h
  // of k-step ks holds dims 64ks + 32h .. +31, the same dims as its K
  // operand; every wave then keeps all of the item's fragments in
  // accumulator registers.
  // BF16 caches: the BF16 query as given, laid out alike in LDS ([RB][NKS
  // ks][64 lanes][16 B]: lane half h of k-step ks holds dims 16ks + 8h ..
  // +7, the same dims as its K operand); softmax_scale * log2(e) multiplies
  // the accumulator.
  uint8_t* qlds = smem;  // [RB][NKS ks][2 terms][64 lanes][32 B]; the merge buffers reuse it after the loop
  int* qexp = (int*)(smem + RB * NKS * 2 * 64 * 32);  // [ROWS] E8M0 of the hi term
  if constexpr (BF) {
    const int r = q_r, qq = q_qq;
    if (r < S::ROWS) {
      const int rb = r >> 5;
#pragma unroll
      for (int part = 0; part < 4; ++part) {
        const int ks = 2 * qq + (part >> 1), hh = part & 1;
        *(u32x4*)(qlds + ((size_t)(rb * NKS + ks) * 64 + 32 * hh + (r & 31)) * 16) =
            q_valid ? qraw[part] : u32x4{0, 0, 0, 0};
      }
    }
  } else {
    const float cbase = a.scale_log2 * (PT ? 1.0f : a.k_scale[0]);
    const int r = q_r, qq = q_qq;
    float qv[32];
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      const u32x4 raw = q_valid ? qraw[part] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const uint16_t bits = (uint16_t)(raw[p >> 1] >> (16 * (p & 1)));
        qv[8 * part + p] =
            a.q_fp16 ? (float)__builtin_bit_cast(_Float16, bits) : __uint_as_float((uint32_t)bits << 16);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(qv[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));  // the row's QP parts are adjacent lanes
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    if constexpr (QP == 8) amax = fmaxf(amax, __shfl_xor(amax, 4));
    const float cq = amax * cbase;
    int e = 0;
    float mul = 0.f;
    if (cq > 0.f && cq < INFINITY) {
      int ex;
      (void)frexpf(cq * (1.0f / FP8_MAX), &ex);  // cq/448 < 2^ex
      e = min(max(ex, -119), 127);
      mul = ldexpf(cbase, -e);
    }
    if (qq == 0 && r < S::ROWS) qexp[r] = 127 + e;
    const int rb = r >> 5, ks = qq >> 1, hh = qq & 1;
    uint8_t* dst = qlds + ((size_t)((rb * NKS + ks) * 2) * 64 + 32 * hh + (r & 31)) * 32;
    if (r < S::ROWS) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 t0v, t1v;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          int w0 = 0, w1 = 0;
          float r1[4], r2[4];
#pragma unroll
          for (int x = 0; x < 4; ++x)
            r1[x] = fminf(fmaxf(qv[16 * half + 4 * j4 + x] * mul, -FP8_MAX), FP8_MAX);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r1[0], r1[1], w0, false);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r1[2], r1[3], w0, true);
          {
            const float hv[4] = {__builtin_amdgcn_cvt_f32_fp8(w0, 0), __builtin_amdgcn_cvt_f32_fp8(w0, 1),
                                 __builtin_amdgcn_cvt_f32_fp8(w0, 2), __builtin_amdgcn_cvt_f32_fp8(w0, 3)};
#pragma unroll
            for (int x = 0; x < 4; ++x) r2[x] = (r1[x] - hv[x]) * 16.0f;
          }
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r2[0], r2[1], w1, false);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r2[2], r2[3], w1, true);
          t0v[j4] = (uint32_t)w0;
          t1v[j4] = (uint32_t)w1;
        }
        *(u32x4*)(dst + 16 * half) = t0v;
        *(u32x4*)(dst + 64 * 32 + 16 * half) = t1v;
      }
    }
  }
  __syncthreads();
  int qsc[RB];
  i32x8 qf[RB][BF ? 1 : NKS][2];
  u32x4 qfb[RB][BF ? NKS : 1];  // BF16 query fragments
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (BF) {
      qsc[rb] = 0;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        qfb[rb][ks] = *(const u32x4*)(qlds + ((size_t)(rb * NKS + ks) * 64 + lane) * 16);
        asm volatile("" : "+a"(qfb[rb][ks]));  // kept in accumulator registers for the whole loop
      }
    } else {
      qsc[rb] = qexp[32 * rb + c32];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const uint8_t* src = qlds + ((size_t)((rb * NKS + ks) * 2 + t) * 64 + lane) * 32;
          const u32x4 lo = *(const u32x4*)src, hi = *(const u32x4*)(src + 16);
          qf[rb][ks][t] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          asm volatile("" : "+a"(qf[rb][ks][t]));  // kept in accumulator registers for the whole loop
        }
    }
  }

  // ---- page ids of the item into LDS (the loop needs them from its fourth
  // step on) ----
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (tid + 256 * j < nstaged) ids[tid + 256 * j] = idr[j];

  // ---- softmax state ----
  // Rows that are padding start with a finite reference so that no path has
  // to special-case them; they are never written out.  O holds
  // sum_t p_t * v_scale(t) * v_t for per-token scales and sum_t p_t v_t for a
  // per-tensor scale (applied at the end).
  float m_ref[RB], m_hi[RB], l_acc[RB];
  f32x16 o[RB][NDB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_ref[rb] = valid[rb] ? -INFINITY : 0.f;
    m_hi[rb] = -INFINITY;
  }
  const float vs_out = (PT || BF) ? 1.0f : a.v_scale[0];
  const float cbf = a.scale_log2;  // BF16: the score scale, applied to the accumulator

  float* ssl = sbuf + w * 64;  // this wave's scale slot

  __syncthreads();  // staged ids visible

  // The loads of step k are issued in two parts: K and the scales once the
  // QK MFMAs of the step before have consumed its K registers, V once its PV
  // MFMAs have consumed its V registers; each part then has a whole step to
  // arrive and lands in the registers it replaces.
  const int idv = lane < nstaged ? ids[lane] : 0;  // the first 64 staged ids, one per lane
  auto page_uniform = [&](long j) -> long {  // id of page j, wave-uniform
    // each source is read and made uniform in its own branch, so waiting for
    // the rare block-table read never waits for the K/V loads in flight
    if (!page_ok(j)) return 0;
    if (j < 64 && j < nstaged) return __builtin_amdgcn_readlane(idv, (int)j);  // no memory access
    if (j < nstaged) return __builtin_amdgcn_readfirstlane(ids[j]);
    // past the staged bound: a scalar read of the block table (the table is
    // constant for the kernel's lifetime), counted apart from the K/V loads
    return ((long)btc[(id0 + j) >> psub] << psub) | ((id0 + j) & msk);
  };
  auto step_page = [&](int k) -> StepPages {  // page ids of step k
    const long j = (long)((k - tb) * TT + 32 * wu) >> ps_log2;
    return StepPages{page_uniform(j), BIG ? 0L : page_uniform(j + 1)};
  };

  // Tiles [ti0, ti1) are visible to every row; their steps skip the masks
  // once every row has a reference maximum.
  int ti0, ti1;
  {
    const int first = lo_max > t0 ? (lo_max - t0 + TT - 1) / TT : 0;
    const int last = hi_min - t0 - (TT - 1) >= 0 ? (hi_min - t0 - (TT - 1)) / TT + 1 : 0;
    ti0 = min(max(first, tb), te);
    ti1 = max(min(last, te), ti0);
  }

  // ---- one step ----
  // `gen` (wave-uniform): a boundary step, with masks and reference updates.
  // The step's registers in `cur` are refilled with step k+2 (two steps of
  // loads in flight per wave); steps past the item reload its last step's
  // cached pages, so the loads are unconditional and the compiler's wait
  // counts stay exact.  A step k >= te (padding an odd count) masks every
  // token.
  // Returns false when the wave has to restart with a larger reference.
  bool ovf = false;
  // Scan pass (wave-uniform): a restart that does not stop at an overflow and
  // records, per row, a reference bound over the whole share (see below).
  bool scan = false;
  // V conversion scale of the next step: with per-token scales, 2^E comes
  // from the step's largest V scale (lanes 32-63 hold its 32 V scales), and
  // the scales go to LDS with the V scales divided by 2^E (and the k scales
  // times the query's 2^e).  E is clamped so that every V value is exact in
  // FP16; above the clamp the normalised V scales exceed 1, and vsmax (their
  // largest) enters the overflow check of the probabilities.  Done at the
  // end of the step before, under its last MFMAs.
  float vconv = 1.0f, vsmax = 1.0f;
  // V scales of tokens outside the visible span (their bytes may be
  // anything) count as 0, in the maximum and in LDS.
  auto prep = [&](const SD& nb, int kk) {
    if constexpr (PT) {
      const int t = t0 + kk * TT + 32 * w + c32;
      const float vsc = (kk < te && t >= lo_u && t < hi_u) ? nb.sc : 0.f;
      float x = fmax_swap32(h ? vsc : 0.f);  // every lane: v scale of token c32
      x = fmaxf(x, dpp_f<0xB1>(x));            // quad: lanes ^1
      x = fmaxf(x, dpp_f<0x4E>(x));            // quad: lanes ^2
      x = fmaxf(x, dpp_f<0x141>(x));           // half-row mirror
      x = fmaxf(x, dpp_f<0x140>(x));           // row mirror
      x = fmax_swap16(x);                      // both 16-lane rows: the step's 32 tokens
      const int e = min(max(__builtin_amdgcn_frexp_expf(x), VEXP_MIN), VEXP_MAX);
      const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
      vconv = __uint_as_float((uint32_t)(127 + e) << 23);
      vsmax = x * inv;
      ssl[lane] = h ? vsc * inv : nb.sc;
    }
  };

  auto step = [&](auto GENc, SD& cur, const SD& nxt, int k) __attribute__((always_inline)) -> bool {
    constexpr bool gen = decltype(GENc)::value;
    if (k >= te) return true;  // padding of the last group of NB: nothing to do
    const int tsa = t0 + k * TT + 32 * w;  // first token of the step
    const int tl = tsa + 16 * h;           // first of the lane's 16 tokens
    const int span_lo = lo_u, span_hi = hi_u;  // tokens whose V may be used
    const int kn = min(k + NB, te - 1);
    const StepPages nid = step_page(kn);

    // V of the step; tokens outside the visible span get zero V (their bytes
    // may be anything, and 0 * NaN would reach O)
    constexpr int NVU = BF ? 2 * NDB : NDB;  // 16-byte V units of the lane
    u32x4 vv[NVU];
#pragma unroll
    for (int u = 0; u < NVU; ++u) vv[u] = cur.v[u];
    if constexpr (gen) {
      const int va = min(max(span_lo - tl, 0), 16), vb = min(max(span_hi - tl, 0), 16);
      if constexpr (BF) {
        // unit 2db + kb, word q: tokens 8kb + 2q (low half) and 8kb + 2q + 1
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int t = 8 * kb + 2 * q;
            const uint32_t m = ((t >= va && t < vb) ? 0xFFFFu : 0u) | ((t + 1 >= va && t + 1 < vb) ? 0xFFFF0000u : 0u);
#pragma unroll
            for (int db = 0; db < NDB; ++db) vv[2 * db + kb][q] &= m;
          }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t m = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int t = 4 * q + b;
            if (t >= va && t < vb) m |= 0xFFu << (8 * b);
          }
#pragma unroll
          for (int db = 0; db < NDB; ++db) vv[db][q] &= m;
        }
      }
    }

    // S^T = K Q^T for one 32-row block: K as stored against the two query
    // terms, each k-step with its own E8M0 scale
    auto qk = [&](int rb) {
      f32x16 acc = {};
      if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur.k[ks]),
                                                        __builtin_bit_cast(bf16x8, qfb[rb][ks]), acc, 0, 0, 0);
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks)
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.k[ks], qf[rb][ks][t], acc, 0, 0, 0, 127, 0,
                                                                  qsc[rb] - 4 * t);
      }
      return acc;
    };
    // V in FP16 (times 2^E): k-block kb of dim 32db + c32 = tokens 16h + 8kb .. +7
    half8 vb[NDB][2];
    auto vcvt = [&]() {
      if constexpr (BF) return;  // BF16 V enters the MFMA as stored
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t d0 = vv[db][2 * kb], d1 = vv[db][2 * kb + 1];
          const h2 x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, vconv, false);
          const h2 x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d0, vconv, true);
          const h2 x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, vconv, false);
          const h2 x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(d1, vconv, true);
          vb[db][kb] = half8{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
        }
    };
    // per-token scales of the lane's 16 tokens (per-tensor: folded into the
    // query and applied at the end)
    float ks16[16], vs16[16];
    auto scales = [&]() {
      if constexpr (PT) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f4 kq = *(const f4*)(ssl + 16 * h + 4 * q);
          const f4 vq = *(const f4*)(ssl + 32 + 16 * h + 4 * q);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            ks16[4 * q + x] = kq[x];
            vs16[4 * q + x] = vq[x];
          }
        }
      }
    };

    // probabilities of one row block -> PV operand (FP16); branch-free so
    // that the MFMAs of the other row block can be interleaved with it
    // PV operand: FP16 P (FP8 caches), or the two BF16 terms of P, hi in
    // [0, 2) and lo in [2, 4) (BF16 caches)
    using PF = typename std::conditional<BF, bf16x8, half8>::type;
    constexpr int NPF = BF ? 4 : 2;
    auto probs = [&](int rb, const f32x16& sa, PF (&pb)[NPF]) {
      float y[16];
      if constexpr (gen) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = BF ? sa[i] * cbf : PT ? sa[i] * ks16[i] : sa[i];
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = tl + i;
          y[i] = (t >= lo_r[rb] && t <= hi_r[rb]) ? y[i] : -INFINITY;
          mx = fmaxf(mx, y[i]);
        }
        mx = fmax_swap32(mx);  // the partner lane holds the row's other 16 tokens
        // the row's first visible tokens set its reference (its O is still zero)
        const bool first = m_ref[rb] == -INFINITY;
        const bool over = !first && mx > m_ref[rb] + TAU_S;
        ovf |= over;
        if (scan) {
          // a reference no logit of the step exceeds and under which the
          // lane's probability sum (at most 16 * 2^(mx - ref)) times the
          // largest normalised V scale stays at most 2^14
          const float need = mx + fmaxf(0.f, __builtin_amdgcn_logf(vsmax) - 10.0f);
          m_hi[rb] = fmaxf(m_hi[rb], need);
        } else {
          m_hi[rb] = over ? fmaxf(m_hi[rb], mx) : m_hi[rb];
        }
        m_ref[rb] = first ? mx : m_ref[rb];
      }
      const float nm = m_ref[rb] == -INFINITY ? 0.f : -m_ref[rb];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (gen) y[i] = y[i] + nm;
        else y[i] = BF ? __builtin_fmaf(sa[i], cbf, nm) : PT ? __builtin_fmaf(sa[i], ks16[i], nm) : sa[i] + nm;
        y[i] = __builtin_amdgcn_exp2f(y[i]);  // exp2(-inf) = 0
      }
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = y[2 * i] + y[2 * i + 1];
      const float ls = ((t8[0] + t8[1]) + (t8[2] + t8[3])) + ((t8[4] + t8[5]) + (t8[6] + t8[7]));
      l_acc[rb] += ls;
      // a PV operand p * (normalised V scale) of 2^15 or more shows in the
      // lane's sum times the largest normalised V scale; a reference raised
      // by log2 of that product brings every operand to at most 1.  A sum
      // that overflowed to infinity raises it by 127 (a finite reference:
      // the restart's masked steps then find the exact maximum if it is
      // still too low).
      const float bnd = ls * vsmax;
      const bool big = bnd > 0x1p15f;
      ovf |= big;
      if (!(gen && scan))
        m_hi[rb] = big ? fmaxf(m_hi[rb], m_ref[rb] + __builtin_amdgcn_logf(fminf(bnd, 0x1p127f))) : m_hi[rb];
      if constexpr (PT) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] *= vs16[i];
      }
      if constexpr (BF) {
        // P = hi + lo, each rounded to BF16 (about 16 significant bits)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int x = 0; x < 8; ++x) {
            const __bf16 hi = (__bf16)y[8 * kb + x];
            pb[kb][x] = hi;
            pb[2 + kb][x] = (__bf16)(y[8 * kb + x] - (float)hi);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          h2 c[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) c[x] = __builtin_convertvector(f2{y[8 * kb + 2 * x], y[8 * kb + 2 * x + 1]}, h2);
          pb[kb] = half8{c[0][0], c[0][1], c[1][0], c[1][1], c[2][0], c[2][1], c[3][0], c[3][1]};
        }
      }
    };
    auto pv = [&](int rb, const PF (&pb)[NPF]) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if constexpr (BF) {
            const bf16x8 vf = __builtin_bit_cast(bf16x8, vv[2 * db + kb]);
            o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kb], o[rb][db], 0, 0, 0);
            o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[2 + kb], o[rb][db], 0, 0, 0);
          } else {
            o[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb[db][kb], pb[kb], o[rb][db], 0, 0, 0);
          }
        }
    };

    // Schedule (one wave per SIMD, so the overlap has to come from within
    // the wave), in parts fenced by scheduling barriers.  Two row blocks: QK
    // of row block 0 with the V conversion; QK of row block 1 with the
    // probabilities of block 0; PV of block 0 with the probabilities of
    // block 1; PV of block 1 with the next step's scales.  One row block: QK
    // with the V conversion, the probabilities on their own, PV with the
    // next step's scales.  V is reloaded (three steps ahead) once converted,
    // K once every row block's QK MFMAs have read it.  Inside a part the
    // compiler interleaves the MFMAs with the VALU work (an interleave pinned
    // by hand, one MFMA per 8-16 VALU, measured 2 % slower).
    static_assert(RB == 1 || RB == 2, "one or two row blocks");
    PF p0[NPF];
    const f32x16 s0 = qk(0);
    vcvt();
    __builtin_amdgcn_sched_barrier(0);
    load_v(cur, nid);  // this step's V is converted (BF16: copied to vv)
    if constexpr (RB == 2) {
      PF p1[NPF];
      const f32x16 s1 = qk(1);
      scales();
      probs(0, s0, p0);
      __builtin_amdgcn_sched_barrier(0);
      load_k(cur, nid);  // both row blocks' QK have read this step's K
      pv(0, p0);
      probs(1, s1, p1);
      __builtin_amdgcn_sched_barrier(0);
      pv(1, p1);
    } else {
      load_k(cur, nid);  // the QK MFMAs have read this step's K
      scales();
      probs(0, s0, p0);
      __builtin_amdgcn_sched_barrier(0);
      pv(0, p0);
    }
    prep(nxt, k + 1);
    __builtin_amdgcn_sched_barrier(0);
    return !__builtin_amdgcn_ballot_w64(ovf);
  };

  // One pass of this wave over the item, NB steps per iteration with one
  // load buffer each (a count that is not a multiple of NB ends with steps
  // that return at once).  An overflow stops it at the top of
  // the next group (a single latch keeps each O accumulator in place across
  // iterations), except in the scan pass, which runs to the end.
  auto attempt = [&](bool first) __attribute__((always_inline)) -> bool {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l_acc[rb] = 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[rb][db] = f32x16{};
    }
    if (tb >= te) return true;
    if (!first) {  // a restart: the first NB steps' loads again
      const StepPages p0 = step_page(tb);
      load_k(ba, p0);
      load_v(ba, p0);
      const int k1 = min(tb + 1, te - 1);
      const StepPages p1 = step_page(k1);
      load_k(bb, p1);
      load_v(bb, p1);
      if constexpr (NB == 3) {
        const int k2 = min(tb + 2, te - 1);
        const StepPages p2 = step_page(k2);
        load_k(bc, p2);
        load_v(bc, p2);
      }
    }
    prep(ba, tb);
    // Groups of NB steps: boundary groups (masks, reference updates) until
    // the interior tiles are reached with every row's reference set, interior
    // groups, then boundary groups again.  Each loop is entered with nothing
    // in flight beyond its NB buffers' loads, which keeps the compiler's wait
    // counts exact inside it.
    bool go = true;  // wave-uniform
    int k = tb;
    auto triple = [&](auto GENc) __attribute__((always_inline)) {
      go = step(GENc, ba, bb, k);
      __builtin_amdgcn_sched_barrier(0);  // the steps do not interleave (registers)
      if constexpr (NB == 3) {
        go = step(GENc, bb, bc, k + 1) && go;
        __builtin_amdgcn_sched_barrier(0);
        go = step(GENc, bc, ba, k + 2) && go;
      } else {
        go = step(GENc, bb, ba, k + 1) && go;
      }
      __builtin_amdgcn_sched_barrier(0);
      go = go || scan;
      k += NB;
    };
    if (first) {
      for (; k < te && go;) {
        bool need_ref = false;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) need_ref |= m_ref[rb] == -INFINITY;
        if (k >= ti0 && k + NB - 1 < ti1 && !__builtin_amdgcn_ballot_w64(need_ref)) break;
        triple(std::true_type{});
      }
      for (; k + NB - 1 < ti1 && go;) triple(std::false_type{});
    }
    for (; k < te && go;) triple(std::true_type{});  // a restart runs every step with the masks
    return !__builtin_amdgcn_ballot_w64(ovf);
  };
  // Restarts.  The first attempt raises a row's reference only to the
  // maxima it saw before it stopped, so logits that keep climbing could
  // stop every later attempt too.  Instead the first restart is a scan pass
  // over the wave's whole share: if it meets no overflow its result stands;
  // otherwise it has recorded, per row, a reference no logit exceeds and
  // under which no PV operand reaches 2^15, and one last pass with that
  // reference cannot overflow for any finite input.  At most three passes.
  // The first attempt is its own copy of the loop, entered straight from the
  // early loads (no join with the restart path, whose different load history
  // would make the compiler wait for all three steps before the first).
  if (!attempt(true)) {
    for (int pass = 0; pass < 2; ++pass) {
      wait_vmcnt<0>();  // loads issued past the stop
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mh = fmax_swap32(m_hi[rb]);
        // after the first attempt: at least the maxima seen; after the scan:
        // the bound over the whole share (rows without visible tokens keep
        // their reference)
        if (pass == 0 ? mh > m_ref[rb] : mh > -INFINITY) m_ref[rb] = mh;
        m_hi[rb] = -INFINITY;
      }
      ovf = false;
      scan = pass == 0;
      if (attempt(false)) break;
    }
    scan = false;
  }

  // ---- merge the four waves' states ----
  // Each wave writes its (max, sum) per row and its unscaled O to LDS; one
  // wave then turns the (max, sum) pairs into per-wave weights
  // 2^(m_w - M) (the per-tensor V scale folded in) and the row's (M, L,
  // output factor); every thread finally sums the four weighted O buffers.
  constexpr int NR = S::ROWS;
  float* wm = stats;                          // [SW][NR] reference maxima, then weights
  float* wl = stats + SW * NR;                // [SW][NR] sums
  float* rowinfo = stats + 2 * SW * NR + SW;  // [NR][4]: M, L, direct-output factor
  {
    float lrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lrow[rb] = fadd_swap32(l_acc[rb]);
    if (h == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        wm[w * NR + 32 * rb + c32] = m_ref[rb];
        wl[w * NR + 32 * rb + c32] = lrow[rb];
      }
    }
    float* ob = obuf + w * (S::OBUF / 4);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = 32 * rb + c32;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(f4*)(ob + r * S::OROW + 32 * db + 8 * q + 4 * h) =
              f4{o[rb][db][4 * q], o[rb][db][4 * q + 1], o[rb][db][4 * q + 2], o[rb][db][4 * q + 3]};
    }
  }
  __syncthreads();
  if (tid < NR) {
    const int r = tid;
    float mv[SW], lv[SW];
#pragma unroll
    for (int x = 0; x < SW; ++x) {
      mv[x] = wm[x * NR + r];
      lv[x] = wl[x * NR + r];
    }
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < SW; ++x) M = lv[x] > 0.f ? fmaxf(M, mv[x]) : M;
    float Lt = 0.f;
#pragma unroll
    for (int x = 0; x < SW; ++x) {
      const float fx = lv[x] > 0.f ? __builtin_amdgcn_exp2f(mv[x] - M) : 0.f;
      Lt += lv[x] * fx;
      wm[x * NR + r] = fx * vs_out;
    }
    float factor = 0.f;
    if (Lt > 0.f) {
      if (a.has_sinks) {
        const int gr = row0 + (r < nrows ? r : 0);
        const int hh = kvh * a.G + gr % a.G;
        const float sk = a.sinks[hh] * LOG2E;
        const float M2 = fmaxf(M, sk);
        const float sc = __builtin_amdgcn_exp2f(M - M2);
        factor = sc / (Lt * sc + __builtin_amdgcn_exp2f(sk - M2));
      } else {
        factor = 1.0f / Lt;
      }
    }
    rowinfo[r * 4 + 0] = M;
    rowinfo[r * 4 + 1] = Lt;
    rowinfo[r * 4 + 2] = factor;
  }
  __syncthreads();

  // ---- write: partial state or final rows ----
  auto osum = [&](int r, int d4) {
    f4 acc = *(const f4*)(obuf + r * S::OROW + d4) * wm[r];
#pragma unroll
    for (int x = 1; x < SW; ++x) acc += *(const f4*)(obuf + x * (S::OBUF / 4) + r * S::OROW + d4) * wm[x * NR + r];
    return acc;
  };
  if (it.slot >= 0) {
    float* sp = a.workspace + (size_t)it.slot * rpg * (2 + D);
    if (tid < nrows) {
      sp[tid] = rowinfo[tid * 4 + 0];
      sp[rpg + tid] = rowinfo[tid * 4 + 1];
    }
    float* po = sp + 2 * rpg;
    for (int e = tid; e < nrows * (D / 4); e += 256) {
      const int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
      *(f4*)(po + (size_t)r * D + d4) = osum(r, d4);
    }
    if (a.merge_ctr) {
      __syncthreads();  // the O buffers read: their LDS is the merge's
      const MergeArgs ma{a.out, a.workspace, a.sinks, a.QL, a.Hq, a.G, a.rows_total, a.rows_per_group, a.q_fp16,
                         a.has_sinks};
      arrive_and_merge<D>(ma, a.merge_ctr, it, (uint8_t*)obuf);
    }
  } else {
    for (int e = tid; e < nrows * (D / 4); e += 256) {
      const int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
      const f4 v = osum(r, d4) * rowinfo[r * 4 + 2];
      const int gr = row0 + r, i = gr / a.G, hl = gr % a.G;
      const long ooff = (((long)s * a.QL + i) * a.Hq + (long)kvh * a.G + hl) * D + d4;
      uint16_t hv[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        hv[x] = a.q_fp16 ? __builtin_bit_cast(uint16_t, (_Float16)v[x]) : __builtin_bit_cast(uint16_t, (__bf16)v[x]);
      *(u32x2*)((uint16_t*)a.out + ooff) =
          u32x2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
    }
  }
}

template <int D, int RB, bool PT, bool BIG, bool BF = false>
static pa_status launch_stream_t(const KernelArgs& args, int nblocks, hipStream_t stream) {
  constexpr int bytes = StreamSmem<D, RB>::LAUNCH;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static bool configured = false;
  if (!configured) {
    if (hipFuncSetAttribute((const void*)pa_stream_kernel<D, RB, PT, BIG, BF>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            bytes) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "hipFuncSetAttribute failed");
    }
    configured = true;
  }
  hipLaunchKernelGGL((pa_stream_kernel<D, RB, PT, BIG, BF>), dim3(nblocks), dim3(256), bytes, stream, args);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("decode launch failed: ") + hipGetErrorString(err));
  return PA_OK;
}

bool stream_kernel_applies(const Plan& P) {
  const pa_problem& p = P.prob;
  if (p.token_table || P.rows_per_group <= 16 || p.num_pages <= 0) return false;
  if (p.kv_dtype == PA_BF16) return p.head_dim == 128 && p.page_size >= 32;
  return p.kv_dtype == PA_FP8_E4M3FN && (p.head_dim == 128 || (p.head_dim == 256 && P.rows_per_group <= 32));
}

template <int D, int RB>
static pa_status launch_stream_rb(const Plan& P, const KernelArgs& args, int nblocks, hipStream_t stream) {
  if constexpr (D == 128) {
    if (P.prob.kv_dtype == PA_BF16) return launch_stream_t<D, RB, false, true, true>(args, nblocks, stream);
  }
  const bool pt = P.prob.scale_mode == PA_SCALE_PER_TOKEN;
  if (P.prob.page_size >= 32)
    return pt ? launch_stream_t<D, RB, true, true>(args, nblocks, stream)
              : launch_stream_t<D, RB, false, true>(args, nblocks, stream);
  return pt ? launch_stream_t<D, RB, true, false>(args, nblocks, stream)
            : launch_stream_t<D, RB, false, false>(args, nblocks, stream);
}

pa_status launch_stream(const Plan& P, const KernelArgs& args, int nblocks, hipStream_t stream) {
  if (P.prob.head_dim == 256) return launch_stream_rb<256, 1>(P, args, nblocks, stream);
  return P.rows_per_group > 32 ? launch_stream_rb<128, 2>(P, args, nblocks, stream)
                               : launch_stream_rb<128, 1>(P, args, nblocks, stream);
}

}  // namespace pa
