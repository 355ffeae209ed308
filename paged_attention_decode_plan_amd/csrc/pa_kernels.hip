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
//  * a workgroup owns one work item = (sequence, KV head, row group of up to
//    64 query rows, a contiguous range of 128-token tiles); every wave owns
//    one 16-row tile of the item's rows and a share of each tile's tokens
//    (Waves / Roles below);
//  * dense caches: K/V pages of a tile go straight from HBM into LDS stages
//    (global_load_lds, 16 bytes per lane, coalesced page-head blocks), two to
//    four tiles deep, so later tiles stream in while one tile computes;
//    token-table (sparse) caches gather the same way with per-token slots;
//  * QK^T is computed as S^T = K Q^T: FP8 caches run
//    v_mfma_scale_f32_16x16x128_f8f6f4 with K as stored against three FP8
//    terms of the query (hi, then two residuals, each with its own E8M0 block
//    scale; two terms at head dim 512), BF16 caches run
//    v_mfma_f32_16x16x32_bf16 with the BF16 query, MXFP4 caches the scaled
//    MFMA with FP4 K and each lane's block scale as the A scale (the query
//    permuted to the FP4 operand's lane order);
//  * PV is computed as O^T = V^T P^T: FP8 V converts exactly to FP16 in
//    registers (v_cvt_scalef32_pk_f16_fp8) against FP16 probabilities on
//    v_mfma_f32_16x16x32_f16 (MXFP4: FP4 V converts exactly as well, its
//    block scales folded into the probabilities per 32-dim block as exponent
//    adds against per-block references); BF16 V runs against a two-term BF16 split of
//    the probabilities; probabilities go from the QK accumulator to the PV
//    operand in registers (the QK rows are read in the token order PV
//    contracts);
//  * row max/sum across the 4 lane groups of a row use v_permlane16/32_swap;
//  * probabilities are taken against a per-row reference maximum set at the
//    row's first visible tokens: a base-2 score more than TAU above it (or a
//    per-token V scale more than VS_BAND above its reference) makes the
//    workgroup redo the item with larger references, after at most one scan
//    pass that records every row's true bound, so the accumulator is only
//    ever written by MFMAs.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_merge.h"

namespace pa {

constexpr int TT = kTileTokens;  // 128 tokens per tile
// Waves per workgroup: 16-row items use 4 waves (and two workgroups share a
// CU); 32- and 64-row items of head dim 128 use 8 waves so that each SIMD
// runs two waves of one workgroup.  Head dim 256 keeps 4 waves (one per
// SIMD, up to 512 registers each: two waves of 256 registers spill there).
// Every wave owns one 16-row tile of the item.
template <int NRT, int D>
struct Waves {
  static constexpr int NW = (NRT >= 2 && D <= 128) ? 8 : 4;
  static constexpr int NT = 64 * NW;
};
// MX: MXFP4 caches (FP4 codes, two per byte, and a scale byte per 32-dim
// block; FP8 is set as well, the query and probability paths being FP8's).
template <int D, bool FP8, int NT, bool MX = false>
struct Tile {
  static constexpr int E = FP8 ? 1 : 2;      // bytes per KV element (MX: half a byte)
  static constexpr int X = MX ? 32 : 16 / E;  // elements per 16-byte chunk
  static constexpr int KBYTES = MX ? D * TT / 2 : D * TT * E;  // K tile: [D/X chunks][TT tokens][16 B]
  static constexpr int VROW = MX ? TT / 2 : TT * E;             // V tile: [D rows][TT tokens]
  static constexpr int VBYTES = D * VROW;
  static constexpr int VUPR = VROW / 16;     // 16-byte units per V row
  // per-token k and v scales (FP32), or (MX) the blocks' scale bytes: D/32
  // per token, which is 4 bytes at head dim 128, laid out alike
  static constexpr int SBYTES = MX ? 2 * TT * (D / 32) : FP8 ? 2 * TT * 4 : 0;
  static constexpr int STAGE = KBYTES + VBYTES + SBYTES;
  static constexpr int KPT = KBYTES / 16 / NT;  // 16-byte K units per thread per tile
  static constexpr int VPT = VBYTES / 16 / NT;
  static constexpr int NM = D / 32;  // MFMA k-steps over the head dim
  static constexpr int NDT = D / 16; // 16-wide d tiles of O
};

// Wave roles: a workgroup's NW waves split an item's row tiles into WR
// groups (one 16-row tile per wave: NRW = 1) and each tile's 128 tokens into
// WT groups (WR * WT = NW), so that one wave's O accumulator is one 16-row
// tile of the head dim (D / 4 registers).
template <int D, int NRT>
struct Roles {
  static constexpr int NW = Waves<NRT, D>::NW;
  static constexpr int NRW = 1;         // row tiles per wave
  static constexpr int WR = NRT;        // row groups
  static constexpr int WT = NW / WR;    // token groups
  static constexpr int STEPS = 4 / WT;  // 32-token steps per wave per tile
  static_assert(WR * WT == NW && WT <= 4 && NRW * WR == NRT, "wave roles");
};

template <int D, bool FP8, int NRT, bool SPARSE, bool MX = false>
struct Smem {
  using R = Roles<D, NRT>;
  // head dim 512: one 128-token FP8 stage is 129 KB, so a single stage (the
  // tile's loads, then its compute, no overlap inside the workgroup)
  static constexpr int STAGES = D >= 512 ? 1 : (!SPARSE && FP8 && D == 128 && NRT >= 2) ? 4 : 2;
  static constexpr int STAGE = Tile<D, FP8, Waves<NRT, D>::NT, MX>::STAGE;
  static constexpr int MERGE = NRT * 16 * (D + 4) * 4;  // one O buffer with padded rows
  static constexpr int MAIN = (STAGES * STAGE > MERGE) ? STAGES * STAGE : MERGE;
  static constexpr int IDS = kStageCap * 4;
  static constexpr int STATS = (R::WT * NRT * 16 * 2 + R::NW + NRT * 16 * 4 + 4) * 4;
  static constexpr int TOTAL = MAIN + IDS + STATS;
};

// Register staging of one tile (token-table path).
template <int D, bool FP8, int NT>
struct Staged {
  u32x4 k[Tile<D, FP8, NT>::KPT];
  u32x4 v[Tile<D, FP8, NT>::VPT];
  u32x4 s;
};

template <int D, bool FP8, int NRT, bool SPARSE, bool MX = false>
__global__ __launch_bounds__((Waves<NRT, D>::NT)) void pa_decode_kernel(KernelArgs a) {
  static_assert(!MX || (FP8 && D == 128 && !SPARSE), "MXFP4: head dim 128, page tables");
  static_assert(!MX || Roles<D, NRT>::NRW == 1, "MXFP4: one row tile per wave (per-step scale references)");
  constexpr int NTHREADS = Waves<NRT, D>::NT;
  constexpr int NWAVES = Waves<NRT, D>::NW;
  using T = Tile<D, FP8, NTHREADS, MX>;
  using S = Smem<D, FP8, NRT, SPARSE, MX>;
  using R = Roles<D, NRT>;
  constexpr int NST = S::STAGES;
  constexpr int NRW = R::NRW;
  constexpr int NM = T::NM;
  constexpr int NDT = T::NDT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* stage_base = smem;
  int32_t* ids = (int32_t*)(smem + S::MAIN);
  float* stats = (float*)(smem + S::MAIN + S::IDS);
  static_assert(merge_lds_bytes<D>() <= S::MAIN, "the in-kernel merge reuses the stage LDS");

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int c = lane & 15;
  const int g = lane >> 4;
  const int wr = w % R::WR;  // this wave's row group
  const int wt = w / R::WR;  // this wave's token group

  const WorkItem it = a.items[blockIdx.x];
  const MetaHeader mh = *a.meta;
  if (!meta_ok(mh, a.tag_lo, a.tag_hi)) return;  // not this plan's list: touch nothing
  if (it.seq < 0) return;  // an unused item of a refreshable plan
  const int s = it.seq, kvh = it.kvh, rg = it.rg;
  const int ps = a.page_size;    // tokens per (sub-)page the item is indexed by
  const int pps = a.phys_page;   // physical page size: strides inside a page
  const int psub = a.page_sub;   // sub-pages per page = 2^psub (0 up to 128 tokens)
  const int ps_log2 = 31 - __builtin_clz(ps);
  // sparse rows: the row's slots (or, two-level, its top-k positions) count
  const long cap = SPARSE ? (long)(a.topk ? a.index_stride : a.table_stride) : (long)a.table_stride * pps;
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

  // Rows of this item; the wave owns row tiles wr*NRW .. wr*NRW+NRW-1.
  const int rpg = a.rows_per_group;
  const int row0 = rg * kMaxRowsPerItem;
  const int nrows = min(rpg, a.rows_total - row0);
  int lo_r[NRW], hi_r[NRW];
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    int r = (wr * NRW + rt) * 16 + c;
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
  // Bounds shared by all rows of the item: a tile inside [lo_max, hi_min]
  // needs no mask at all.
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
  // Id j of the row from memory: a page id (dense), a physical token slot
  // (sparse), or a top-k logical position resolved through the block table
  // (two-level sparse: clamped to the table's extent, so the page id read
  // stays in the row).
  const int32_t* tk_row = (SPARSE && a.topk) ? a.topk + (long)s * a.index_stride : nullptr;
  // (sub-)page id j of a dense row: its page's entry and the sub-page
  auto sub_id = [&](long j) -> long { return ((long)bt_row[j >> psub] << psub) | (j & ((1L << psub) - 1)); };
  auto raw_id = [&](long j) -> long {
    if (SPARSE && tk_row) {
      const long P = min(max((long)tk_row[j], 0L), (long)a.table_stride * ps - 1);
      return ((long)bt_row[P >> ps_log2] << ps_log2) + (P & (ps - 1));
    }
    return SPARSE ? (long)bt_row[j] : sub_id(j);
  };
  const long id_rowlen = (SPARSE && tk_row) ? (long)a.index_stride : (long)a.table_stride << (SPARSE ? 0 : psub);
  // ---- the item's first reads, issued before the query is prepared ----
  // The page ids (staged in LDS after the query split), the query rows'
  // raw bits and then the first tiles' DMA with page ids read straight from
  // the block table: the DMA latency overlaps the query split.
  constexpr int IDR = kStageCap / NTHREADS;
  int32_t idr[IDR];
#pragma unroll
  for (int j = 0; j < IDR; ++j) {
    const long k = min((long)(tid + NTHREADS * j), (long)max(nstaged - 1, 0));
    idr[j] = (int32_t)raw_id(min(max(id0 + k, 0L), id_rowlen - 1));  // in the row whatever the item
  }
  constexpr int NQR = FP8 ? ((D + 127) / 128) * 4 : D / 32;  // 16-byte query loads per row tile
  u32x4 qraw[NRW][NQR];
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int r = (wr * NRW + rt) * 16 + c;
    const int gr = row0 + (r < nrows ? r : 0);  // padding rows read row 0 (zeroed at use)
    const int i = gr / a.G, hl = gr % a.G;
    const uint16_t* qrow = (const uint16_t*)a.q + (((long)s * a.QL + i) * a.Hq + (long)kvh * a.G + hl) * D;
#pragma unroll
    for (int x = 0; x < NQR; ++x)
      // MX: the FP4 form of the QK MFMA pairs nibble j of A lane group g
      // (dim 32g + j of its scale block) with B element 64(g&1) + 16(g>>1) +
      // 32(j>>4) + (j&15), so B lane group g holds dims 16g .. 16g+15, then
      // 64+16g .. 64+16g+15
      qraw[rt][x] = MX    ? *(const u32x4*)(qrow + 64 * (x / 2) + 16 * g + 8 * (x % 2))
                    : FP8 ? (32 * g < D ? *(const u32x4*)(qrow + 128 * (x / 4) + 32 * g + 8 * (x % 4))
                                      : u32x4{0, 0, 0, 0})  // head dim 64: lane groups 2, 3 hold no dims
                        : *(const u32x4*)(qrow + 32 * x + 8 * g);
  }
  // MX block scales take the per-token path (scales staged with each tile,
  // V scales folded into P against a reference)
  const bool per_token = FP8 && (MX || a.scale_mode == PA_SCALE_PER_TOKEN);
  const float kscale0 = (FP8 && !per_token) ? a.k_scale[0] : 1.0f;  // per-tensor scales
  const float vscale0 = (FP8 && !per_token) ? a.v_scale[0] : 1.0f;
  const uint8_t* kbase = a.k_cache + (long long)kvh * a.head_stride;
  const uint8_t* vbase = a.v_cache + (long long)kvh * a.head_stride;
  // ---- dense: DMA of one tile into an LDS stage ----
  // K unit u = tid + k*NTHREADS holds chunk tid/TT + 2k of token kswz(tid%TT);
  // V unit u holds 16 bytes of row tid/VUPR + k*(NTHREADS/VUPR) at position
  // tid%VUPR.  So each thread's K units share one page (likewise V), and its
  // k-th unit sits a constant stride after the first.  Every thread issues
  // the same number of loads per tile (a page outside the visible span is
  // replaced by page 0 of the head: those LDS bytes are masked), so a
  // constant vmcnt tracks the tiles in flight.
  constexpr int KCH = NTHREADS / TT;       // chunks covered per k step
  constexpr int VRS = NTHREADS / T::VUPR;  // V rows covered per k step
  const int k_tok = kswz(tid % TT);
  const int k_pg = k_tok / ps;
  const long k_off = ((long)(tid / TT) * pps + k_tok % ps) * 16;
  const long k_step = (long)KCH * pps * 16;
  const int v_row = tid / T::VUPR;
  const int v_tok = ((tid % T::VUPR) ^ (v_row & (T::VUPR - 1))) * T::X;  // first token of the unit
  const int v_pg = v_tok / ps;
  const int v_sx = (v_tok % ps) / T::X;
  const long vrow_bytes = MX ? (long)pps / 2 : (long)pps * T::E;  // a V row of one page
  const long v_off = a.v_transposed ? ((long)v_sx * D + v_row) * 16 : (long)v_row * vrow_bytes + v_sx * 16;
  const long v_step = a.v_transposed ? (long)VRS * 16 : (long)VRS * vrow_bytes;
  // Byte offsets of a (sub-)page id inside its cache / scale array: the
  // page's block plus the sub-page's place in it (K: token offset in every
  // chunk; plain V: column offset in every row; transposed V: its 16-token
  // blocks; scales: token offset).
  const long vsub_bytes = a.v_transposed ? (long)(ps / T::X) * D * 16 : MX ? (long)ps / 2 : (long)ps * T::E;
  const long msk = (1L << psub) - 1;
  auto kpage = [&](long id) { return (id >> psub) * a.page_stride + (id & msk) * ps * 16; };
  auto vpage = [&](long id) { return (id >> psub) * a.page_stride + (id & msk) * vsub_bytes; };
  auto spage = [&](long id) { return ((id >> psub) * a.Hkv + kvh) * pps + (id & msk) * ps; };
  const int s_tok = (lane & 31) * 4;  // scales: wave 0, lanes 0-31 K, 32-63 V
  const int s_pg = s_tok / ps;
  const float* s_src0 = (lane >> 5) ? a.v_scale : a.k_scale;

  // The page ids a thread's DMA of one tile uses (K, V, scales); a page
  // without visible tokens gets -1 and is replaced by page 0 of the head
  // (its LDS bytes are masked).
  auto tile_ids = [&](int tile, auto get_id, long (&id)[3]) {
    const int ts = t0 + tile * TT;
    const long jt = (long)(tile - tb) * ppt;
    auto page_ok = [&](int j) {
      int tok0 = ts + j * ps;
      return tok0 < hi_u && tok0 + ps > lo_u;
    };
    id[0] = page_ok(k_pg) ? get_id(jt + k_pg) : -1;
    id[1] = page_ok(v_pg) ? get_id(jt + v_pg) : -1;
    id[2] = (FP8 && per_token && w == 0 && page_ok(s_pg)) ? get_id(jt + s_pg) : -1;
  };
  // The block-table entries of those pages, read unconditionally (an index
  // kept inside the row) so that all of them go out together.
  auto tile_entries = [&](int tile, long (&e)[3]) {
    const long jt = (long)(tile - tb) * ppt;
    auto entry = [&](long j) -> long { return sub_id(min(max(id0 + j, 0L), ((long)a.table_stride << psub) - 1)); };
    e[0] = entry(jt + k_pg);
    e[1] = entry(jt + v_pg);
    e[2] = entry(jt + s_pg);
  };
  auto tile_ids_from = [&](int tile, const long (&e)[3], long (&id)[3]) {
    const int ts = t0 + tile * TT;
    auto page_ok = [&](int j) {
      int tok0 = ts + j * ps;
      return tok0 < hi_u && tok0 + ps > lo_u;
    };
    id[0] = page_ok(k_pg) ? e[0] : -1;
    id[1] = page_ok(v_pg) ? e[1] : -1;
    id[2] = (FP8 && per_token && w == 0 && page_ok(s_pg)) ? e[2] : -1;
  };
  auto issue_tile_at = [&](uint8_t* stg, const long (&id)[3]) {
    const uint8_t* ksrc = kbase + k_off + (id[0] >= 0 ? kpage(id[0]) : 0);
    uint8_t* kdst = stg + (tid - lane) * 16;
#pragma unroll
    for (int k = 0; k < T::KPT; ++k)
      __builtin_amdgcn_global_load_lds((const void*)(ksrc + k * k_step), (lds_void*)(kdst + k * NTHREADS * 16), 16,
                                       0, 0);
    const uint8_t* vsrc = vbase + v_off + (id[1] >= 0 ? vpage(id[1]) : 0);
    uint8_t* vdst = stg + T::KBYTES + (tid - lane) * 16;
#pragma unroll
    for (int k = 0; k < T::VPT; ++k)
      __builtin_amdgcn_global_load_lds((const void*)(vsrc + k * v_step), (lds_void*)(vdst + k * NTHREADS * 16), 16,
                                       0, 0);
    if (FP8 && per_token && w == 0) {
      const float* src = s_src0 + (id[2] >= 0 ? spage(id[2]) + s_tok % ps : 0);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(stg + T::KBYTES + T::VBYTES), 16, 0, 0);
    }
  };
  auto issue_tile_ids = [&](int tile, uint8_t* stg, auto get_id) {
    long id[3];
    tile_ids(tile, get_id, id);
    issue_tile_at(stg, id);
  };
  if constexpr (!SPARSE) {
    // The first tiles' page ids straight from the block table, read with the
    // query rows and the staged ids; one wait covers them all (the empty
    // statement makes the compiler take it here), so that the DMA issue and
    // the query split after it wait for nothing else.
    long pe[NST > 1 ? NST - 1 : 1][3];
#pragma unroll
    for (int k = 0; k < NST - 1; ++k) tile_entries(tb + k, pe[k]);
    asm volatile("" ::"v"(kscale0), "v"(vscale0));
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt)
#pragma unroll
      for (int x = 0; x < NQR; ++x) asm volatile("" ::"v"(qraw[rt][x]));
#pragma unroll
    for (int j = 0; j < IDR; ++j) asm volatile("" ::"v"(idr[j]));
#pragma unroll
    for (int k = 0; k < NST - 1; ++k) asm volatile("" ::"v"(pe[k][0]), "v"(pe[k][1]), "v"(pe[k][2]));
#pragma unroll
    for (int k = 0; k < NST - 1; ++k)
      if (tb + k < te) {
        long id[3];
        tile_ids_from(tb + k, pe[k], id);
        issue_tile_at(stage_base + k * T::STAGE, id);
      }
  }


  // ---- query fragments of the wave's rows ----
  // FP8 caches: QK runs on the FP8 matrix cores with K as stored.  The query
  // row is scaled by qs = amax/448 and split into three FP8 terms,
  // q/qs = hi + mid/16 + lo/256 (about 12 significant bits), that enter the
  // MFMA with block scales 1, 2^-4 and 2^-8.  Lane group g of MFMA k-step kk
  // holds d = 128kk + 32g .. +31 (K chunks 8kk+2g and 8kk+2g+1).
  // BF16 caches: BF16 MFMA with q as given; d of step m, lane group g, slot p
  // is 32m + 8g + p.
  constexpr int NQ = FP8 ? (D + 127) / 128 : NM;  // QK k-steps (head dim 64: one, half of it zero)
  using QFrag = typename std::conditional<FP8, i32x8, bf16x8>::type;
  // query terms: three (about 12 significant bits), two at head dim 512
  // (about 8: hi + mid/16), whose fragments and O accumulator would not fit
  // the registers with three
  constexpr int NQT = FP8 ? (D >= 512 ? 2 : 3) : 1;
  QFrag qf[NRW][NQ][NQT];
  float crow[NRW];  // log2-domain score scale of the row (incl. the query scale)
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int r = (wr * NRW + rt) * 16 + c;
    const bool valid = r < nrows;
    const int gr = row0 + (valid ? r : 0);
    const int i = gr / a.G, hl = gr % a.G;
    const long qoff = (((long)s * a.QL + i) * a.Hq + (long)kvh * a.G + hl) * D;
    const uint16_t* qrow = (const uint16_t*)a.q + qoff;
    if constexpr (FP8) {
      float qv[NQ][32];
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const u32x4 raw = valid ? qraw[rt][4 * kk + h] : u32x4{0, 0, 0, 0};
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            const uint16_t bits = (uint16_t)(raw[p >> 1] >> (16 * (p & 1)));
            qv[kk][8 * h + p] = a.q_fp16 ? (float)__builtin_bit_cast(_Float16, bits) : __uint_as_float((uint32_t)bits << 16);
          }
        }
      }
      float amax = 0.f;
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk)
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(qv[kk][j]));
      amax = group_max(amax);
      const float qs = (amax > 0.f && amax < INFINITY) ? amax * (1.0f / FP8_MAX) : 1.0f;
      const float inv_qs = 1.0f / qs;
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) {
#pragma unroll
        for (int j4 = 0; j4 < 8; ++j4) {  // 4 values per 32-bit word
          int w0 = 0, w1 = 0, w2 = 0;
          float r1[4], r2[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) r1[e] = fminf(fmaxf(qv[kk][4 * j4 + e] * inv_qs, -FP8_MAX), FP8_MAX);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r1[0], r1[1], w0, false);
          w0 = __builtin_amdgcn_cvt_pk_fp8_f32(r1[2], r1[3], w0, true);
          {
            const float h[4] = {__builtin_amdgcn_cvt_f32_fp8(w0, 0), __builtin_amdgcn_cvt_f32_fp8(w0, 1),
                                __builtin_amdgcn_cvt_f32_fp8(w0, 2), __builtin_amdgcn_cvt_f32_fp8(w0, 3)};
#pragma unroll
            for (int e = 0; e < 4; ++e) r2[e] = (r1[e] - h[e]) * 16.0f;
          }
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r2[0], r2[1], w1, false);
          w1 = __builtin_amdgcn_cvt_pk_fp8_f32(r2[2], r2[3], w1, true);
          {
            const float h[4] = {__builtin_amdgcn_cvt_f32_fp8(w1, 0), __builtin_amdgcn_cvt_f32_fp8(w1, 1),
                                __builtin_amdgcn_cvt_f32_fp8(w1, 2), __builtin_amdgcn_cvt_f32_fp8(w1, 3)};
#pragma unroll
            for (int e = 0; e < 4; ++e) r1[e] = (r2[e] - h[e]) * 16.0f;
          }
          w2 = __builtin_amdgcn_cvt_pk_fp8_f32(r1[0], r1[1], w2, false);
          w2 = __builtin_amdgcn_cvt_pk_fp8_f32(r1[2], r1[3], w2, true);
          qf[rt][kk][0][j4] = w0;
          qf[rt][kk][1][j4] = w1;
          if constexpr (NQT > 2) qf[rt][kk][2][j4] = w2;
        }
      }
      crow[rt] = a.scale_log2 * qs;
    } else {
#pragma unroll
      for (int m = 0; m < NM; ++m)
        qf[rt][m][0] = valid ? __builtin_bit_cast(bf16x8, qraw[rt][m])
                             : __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
      crow[rt] = a.scale_log2;
    }
  }
  float vs_ref = 1.0f;  // O holds sum p*v / vs_ref
  if (FP8 && !per_token) {
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) crow[rt] *= kscale0;
    vs_ref = vscale0;
  }
  if (per_token) vs_ref = 0.f;
  float inv_ref = per_token ? 0.f : 1.0f;
  // MX: one V-scale reference exponent per 32-dim block (blocks of one token
  // may lie binades apart; a shared reference would push the FP16 products
  // of the smaller blocks into subnormals); O of block b holds
  // sum p * v * 2^(e - erb[b]); -1: no visible token yet
  constexpr int NVB = MX ? D / 32 : 1;
  int erb[NVB], ehb[NVB];
#pragma unroll
  for (int b4 = 0; b4 < NVB; ++b4) erb[b4] = ehb[b4] = -1;
  if (MX) vs_ref = inv_ref = 1.0f;

  // ---- online softmax state (lane holds row (wr*NRW+rt)*16+c) ----
  // Probabilities are exp2(score - m_ref) with m_ref a reference maximum set
  // at a row's first visible token and V scales are taken relative to vs_ref,
  // so the FP16 PV operand stays <= 2^12 * 8.  A later score more than TAU
  // above m_ref (or a V scale more than VS_BAND above vs_ref) marks the
  // attempt as overflowed: the workgroup restarts the item with the larger
  // references.  O is therefore only ever written by MFMAs in the loop.
  float m_ref[NRW], m_hi[NRW], l_part[NRW];
  f4 o[NRW][NDT];
  float vs_hi = 0.f;
  bool ovf = false;
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    m_ref[rt] = -INFINITY;
    m_hi[rt] = -INFINITY;
  }
  int* restart_flag = (int*)(stats + S::STATS / 4 - 4);
  if (tid == 0) *restart_flag = 0;


  // ---- page ids of the item into LDS ----
#pragma unroll
  for (int j = 0; j < IDR; ++j)
    if (tid + NTHREADS * j < nstaged) ids[tid + NTHREADS * j] = idr[j];

  // Staged ids (and the cleared restart flag) visible to every wave: a bare
  // barrier after this wave's LDS writes, since a full __syncthreads would
  // also wait for the first tiles' DMA issued above.
  wait_lgkm0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // Page id (dense) or token slot (sparse) number j of the item: from the LDS
  // list, or past the staged bound from the block table.  The two readers are
  // kept apart so the LDS-only path never emits a generic (flat) load, which
  // would make every DMA issue wait for all outstanding loads.
  auto staged_id = [&](long j) -> long { return (long)ids[j]; };
  auto item_id = [&](long j) -> long { return j < nstaged ? (long)ids[j] : raw_id(id0 + j); };

  auto issue_tile = [&](int tile, uint8_t* stg) {
    if (min((long)(tile - tb + 1) * ppt, id_end - id0) <= (long)nstaged)
      issue_tile_ids(tile, stg, staged_id);  // every id the tile needs is in LDS
    else
      issue_tile_ids(tile, stg, item_id);
  };

  // ---- sparse: gather one tile into registers, then store it to LDS ----
  auto load_sparse = [&](int tile, Staged<D, FP8, NTHREADS>& st) {
    const int ts = t0 + tile * TT;
    const long jt = (long)(tile - tb) * ppt;
    // K unit k of this thread: token kswz(tid % TT) (the same for every k,
    // NTHREADS being a multiple of TT), chunk tid / TT + k * (NTHREADS / TT)
    {
      static_assert(NTHREADS % TT == 0, "one K token per thread");
      const int t = kswz(tid % TT);
      const bool vis = ts + t < hi_u;
      const long Sl = vis ? item_id(jt + t) : 0;
      const long pid = Sl >> ps_log2;  // page sizes are powers of two
      const int slot = (int)Sl & (ps - 1);
      const uint8_t* kt = kbase + pid * a.page_stride + ((long)(tid / TT) * ps + slot) * 16;
#pragma unroll
      for (int k = 0; k < T::KPT; ++k)
        st.k[k] = vis ? *(const u32x4*)(kt + (long)k * (NTHREADS / TT) * ps * 16) : u32x4{0, 0, 0, 0};
    }
    // V unit k of this thread: dim d = d0 + k * (NTHREADS / VUPR), tokens
    // tfirst .. tfirst + X - 1 of the tile, where tfirst is the same for
    // every k: the tokens' slots and page addresses are worked out once per
    // tile.  Consecutive lanes take consecutive dims of the same tokens
    // (DL dims x VUPR token groups per wave), so that neighbouring lanes of
    // one load read the same cache line of a token's V rows (dims sit 16
    // bytes apart at page 16).  With the token groups on neighbouring lanes
    // instead, every lane of a load hit a different page: the sparse batch
    // took 44.5 us per decode launch, 36.3 us this way.
    static_assert((NTHREADS / T::VUPR) % T::VUPR == 0, "one token group per thread");
    constexpr int DL = 64 / T::VUPR;  // consecutive dims per token group in a wave
    const int tgrp = lane / DL;
    const int d0 = lane % DL + DL * w;
    const int tfirst = tgrp * T::X;
    const long dstride = a.v_transposed ? 16 : (long)ps * T::E;  // bytes between dims of one token
    const uint8_t* tok[T::X];
    bool tvis[T::X];
#pragma unroll
    for (int e = 0; e < T::X; ++e) {
      const int t = tfirst + e;
      tvis[e] = ts + t < hi_u;
      const long Sl = tvis[e] ? item_id(jt + t) : 0;
      const long pid = Sl >> ps_log2;
      const int slot = (int)Sl & (ps - 1);
      const long off = a.v_transposed ? (long)(slot / T::X) * D * 16 + (slot % T::X) * T::E : (long)slot * T::E;
      tok[e] = vbase + pid * a.page_stride + off + (long)d0 * dstride;
    }
#pragma unroll
    for (int k = 0; k < T::VPT; ++k) {
      const long dk = (long)k * (NTHREADS / T::VUPR) * dstride;
      uint8_t bytes[16];
#pragma unroll
      for (int e = 0; e < T::X; ++e) {
        if (tvis[e]) {
          const uint8_t* src = tok[e] + dk;
#pragma unroll
          for (int b = 0; b < T::E; ++b) bytes[e * T::E + b] = src[b];
        } else {
#pragma unroll
          for (int b = 0; b < T::E; ++b) bytes[e * T::E + b] = 0;
        }
      }
      std::memcpy(&st.v[k], bytes, 16);
    }
    if (FP8 && per_token && w == 0) {
      const float* sc = s_src0;
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = 0.f;
        if (ts + s_tok + e < hi_u) {
          long Sl = item_id(jt + s_tok + e);
          long pid = Sl >> ps_log2;
          int slot = (int)Sl & (ps - 1);
          f[e] = sc[(pid * a.Hkv + kvh) * ps + slot];
        }
      }
      st.s = u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
    }
  };
  auto store_sparse = [&](const Staged<D, FP8, NTHREADS>& st, uint8_t* stg) {
#pragma unroll
    for (int k = 0; k < T::KPT; ++k) *(u32x4*)(stg + (tid + k * NTHREADS) * 16) = st.k[k];
    {
      // V unit k (dim d, token group tgrp) goes to the LDS slot the compute
      // reads it from: d * VUPR + (tgrp ^ (d mod VUPR))
      const int lane_ = tid & 63;
      const int tgrp = lane_ / (64 / T::VUPR);
      const int d0 = lane_ % (64 / T::VUPR) + (64 / T::VUPR) * (tid >> 6);
#pragma unroll
      for (int k = 0; k < T::VPT; ++k) {
        const int d = d0 + k * (NTHREADS / T::VUPR);
        const int u = d * T::VUPR + (tgrp ^ (d & (T::VUPR - 1)));
        *(u32x4*)(stg + T::KBYTES + u * 16) = st.v[k];
      }
    }
    if (FP8 && per_token && w == 0) *(u32x4*)(stg + T::KBYTES + T::VBYTES + lane * 16) = st.s;
  };

  // ---- one 32-token step of one wave on a staged tile ----
  // Token group tg covers tile tokens 32tg .. 32tg+31.  PT: per-token scales;
  // IN: an interior tile (every token visible to every row: no masks).
  auto step = [&](auto PTc, auto INc, int ts, int tg, const uint8_t* stg) {
    constexpr bool PT = decltype(PTc)::value;
    constexpr bool IN = decltype(INc)::value;
    // lane-derived LDS offsets are recomputed per step rather than kept live
    // across the loop (registers are the scarce resource here)
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const int c = lane & 15;
    const int g = lane >> 4;
    const int wt0 = ts + 32 * tg;  // first token of the step
    if constexpr (!IN) {
      if (!(wt0 < hi_u && wt0 + 32 > lo_u)) return;
    }
    const uint8_t* kl = stg;
    const uint8_t* vl = stg + T::KBYTES;
    const float* sl = (const float*)(stg + T::KBYTES + T::VBYTES);

    // --- S^T = K Q^T: block b, row i <-> token 8(i/4)+4b+(i%4) of the step
    f4 sacc[NRW][2];
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) sacc[rt][0] = sacc[rt][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      // keep the K fragments of one block live at a time (register pressure)
      __builtin_amdgcn_sched_barrier(0);
      const int tok = 32 * tg + 8 * (c >> 2) + 4 * b + (c & 3);
      const uint8_t* krow = kl + kswz(tok) * 16;
      if constexpr (MX) {
        // K as FP4 (A operand, the low four registers): lane group g holds
        // block g (dims 32g .. 32g+31) of token tok, which the MFMA scales
        // by the block's E8M0 byte
        const u32x4 k4 = *(const u32x4*)(krow + g * TT * 16);
        const i32x8 kf = i32x8{(int)k4[0], (int)k4[1], (int)k4[2], (int)k4[3], 0, 0, 0, 0};
        const int kse = (int)((*(const uint32_t*)((const uint8_t*)sl + tok * 4) >> (8 * g)) & 0xFF);
#pragma unroll
        for (int rt = 0; rt < NRW; ++rt) {
          sacc[rt][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[rt][0][0], sacc[rt][b], 4, 0, 0, kse,
                                                                         0, 127);
          sacc[rt][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[rt][0][1], sacc[rt][b], 4, 0, 0, kse,
                                                                         0, 123);
          sacc[rt][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[rt][0][2], sacc[rt][b], 4, 0, 0, kse,
                                                                         0, 119);
        }
      } else if constexpr (FP8) {
#pragma unroll
        for (int kk = 0; kk < NQ; ++kk) {
          // head dim 64: lane groups 2, 3 would read past the K tile; their
          // operand dims are zero (as are the query's)
          const bool kin = D >= 128 || 32 * g < D;
          const u32x4 k0 = kin ? *(const u32x4*)(krow + (8 * kk + 2 * g) * TT * 16) : u32x4{0, 0, 0, 0};
          const u32x4 k1 = kin ? *(const u32x4*)(krow + (8 * kk + 2 * g + 1) * TT * 16) : u32x4{0, 0, 0, 0};
          const i32x8 kf = i32x8{(int)k0[0], (int)k0[1], (int)k0[2], (int)k0[3],
                                 (int)k1[0], (int)k1[1], (int)k1[2], (int)k1[3]};
#pragma unroll
          for (int rt = 0; rt < NRW; ++rt) {
            sacc[rt][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[rt][kk][0], sacc[rt][b], 0, 0, 0,
                                                                           127, 0, 127);
            sacc[rt][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[rt][kk][1], sacc[rt][b], 0, 0, 0,
                                                                           127, 0, 123);
            if constexpr (NQT > 2)
              sacc[rt][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[rt][kk][NQT - 1], sacc[rt][b], 0,
                                                                             0, 0, 127, 0, 119);
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          u32x4 raw = *(const u32x4*)(krow + (4 * m + g) * TT * 16);
          bf16x8 kf = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
          for (int rt = 0; rt < NRW; ++rt)
            sacc[rt][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[rt][m][0], sacc[rt][b], 0, 0, 0);
        }
      }
    }

    // --- the lane's 8 tokens: slot p = 4b + r <-> token 8g + p of the step
    const int tl = 32 * tg + 8 * g;  // tile-relative
    const int tv = ts + tl;          // absolute
    int va = 0, vb = 8;              // slots [va, vb) lie in the visible span
    if constexpr (!IN) {
      va = min(max(lo_u - tv, 0), 8);
      vb = min(max(hi_u - tv, 0), 8);
    }
    float ks[8], vsr[8];
    u32x4 vsw[2];  // MX: the V scale bytes of the lane's tokens tl .. tl+7 (one word per token at D128)
    if constexpr (MX) {
      const uint8_t* vsb = (const uint8_t*)(sl + TT) + tl * 4;
      vsw[0] = *(const u32x4*)vsb;
      vsw[1] = *(const u32x4*)(vsb + 16);
    } else if constexpr (PT) {
      f4 k0 = *(const f4*)(sl + tl), k1 = *(const f4*)(sl + tl + 4);
      f4 v0 = *(const f4*)(sl + TT + tl), v1 = *(const f4*)(sl + TT + tl + 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ks[r] = k0[r];
        ks[4 + r] = k1[r];
        vsr[r] = v0[r];
        vsr[4 + r] = v1[r];
      }
      if constexpr (!IN) {
#pragma unroll
        for (int p = 0; p < 8; ++p) vsr[p] = (p >= va && p < vb) ? vsr[p] : 0.f;  // garbage outside the span
      }
      float vmax = 0.f;
#pragma unroll
      for (int p = 0; p < 8; ++p) vmax = fmaxf(vmax, vsr[p]);
      vmax = group_max(vmax);  // wave-uniform: the 4 lane groups hold the step's 32 tokens
      if (vs_ref == 0.f) {
        if (vmax > 0.f) {  // first visible scales: O is still zero
          vs_ref = vmax;
          inv_ref = __builtin_amdgcn_rcpf(vmax);
        }
      } else if (vmax > vs_ref * VS_BAND) {
        ovf = true;
        vs_hi = fmaxf(vs_hi, vmax);
      }
#pragma unroll
      for (int p = 0; p < 8; ++p) vsr[p] *= inv_ref;
    }

    // --- y = raw score (* k scale), masked -> -inf; row max.  The positive
    // row scale crow is applied in the exponent: max(crow*y) = crow*max(y).
    float y[NRW][8];
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        float v = sacc[rt][p >> 2][p & 3];
        if constexpr (PT && !MX) v *= ks[p];  // MX: the K scales are inside the MFMA
        if constexpr (!IN) {
          const int t = tv + p;
          v = (t >= lo_r[rt] && t <= hi_r[rt]) ? v : -INFINITY;
        }
        y[rt][p] = v;
      }
      float my = y[rt][0];
#pragma unroll
      for (int p = 1; p < 8; ++p) my = fmaxf(my, y[rt][p]);
      const float mx = group_max(my) * crow[rt];  // -inf stays -inf (crow > 0)
      if (m_ref[rt] == -INFINITY) {
        m_ref[rt] = mx;  // first visible tokens of the row: its O is still zero
      } else if (mx > m_ref[rt] + TAU) {
        ovf = true;
        m_hi[rt] = fmaxf(m_hi[rt], mx);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // --- probabilities -> PV operand, in registers
    using PFrag = typename std::conditional<FP8, half8, bf16x8>::type;
    PFrag pf[NRW];
    PFrag pl[NRW];  // BF16 caches: low part of a two-term split of P
    half8 pfx[MX ? D / 32 : 1][NRW];  // MX: P times each V block's relative scale
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const float nm = m_ref[rt] == -INFINITY ? 0.f : -m_ref[rt];
      float pr[8];
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        pr[p] = __builtin_amdgcn_exp2f(__builtin_fmaf(y[rt][p], crow[rt], nm));  // exp2(-inf) = 0
        l_part[rt] += pr[p];
        if constexpr (PT && !MX) pr[p] *= vsr[p];
      }
      if constexpr (MX) {
        // per block: the lane's largest visible scale exponent checks the
        // block's reference (2^3 band; above it the lane marks a restart and
        // records the exponent), and each token's factor 2^(e - erb) goes
        // into P as an exponent add (exact).  The reference is wave-uniform:
        // set from the whole wave's step at its first visible tokens.
#pragma unroll
        for (int b4 = 0; b4 < D / 32; ++b4) {
          int ev[8];
          int emx = -1;
#pragma unroll
          for (int p = 0; p < 8; ++p) {
            ev[p] = (int)((vsw[p >> 2][p & 3] >> (8 * b4)) & 0xFF);
            if constexpr (!IN) ev[p] = (p >= va && p < vb) ? ev[p] : -1;  // scales outside the span are not read
            emx = max(emx, ev[p]);
          }
          if (erb[b4] < 0) {
            erb[b4] = (int)group_max((float)emx);
          } else if (emx > erb[b4] + 3) {
            ovf = true;
            ehb[b4] = max(ehb[b4], emx);
          }
#pragma unroll
          for (int p = 0; p < 8; p += 2) {
            const float p0 = __builtin_amdgcn_ldexpf(pr[p], ev[p] - erb[b4]);  // pr = 0 for masked tokens
            const float p1 = __builtin_amdgcn_ldexpf(pr[p + 1], ev[p + 1] - erb[b4]);
            h2 hp = __builtin_convertvector(f2{p0, p1}, h2);
            pfx[b4][rt][p] = hp[0];
            pfx[b4][rt][p + 1] = hp[1];
          }
        }
      } else if constexpr (FP8) {
#pragma unroll
        for (int p = 0; p < 8; p += 2) {
          h2 hp = __builtin_convertvector(f2{pr[p], pr[p + 1]}, h2);
          pf[rt][p] = hp[0];
          pf[rt][p + 1] = hp[1];
        }
      } else {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          __bf16 hi = (__bf16)pr[p];
          pf[rt][p] = hi;
          pl[rt][p] = (__bf16)(pr[p] - (float)hi);
        }
      }
    }
    // --- O^T += V^T P^T: V row d = 16dt + c, tokens 8g..8g+7 of the step
    bool vmask = false;
    uint64_t keep8 = ~0ull;  // FP8: byte mask of visible tokens
    if constexpr (!IN) {
      vmask = va > 0 || vb < 8;
      // bytes [va, vb) hold visible tokens; no shift by 64 (va or vb may be 8)
      const uint64_t below_vb = vb >= 8 ? ~0ull : ((1ull << (8 * vb)) - 1);
      const uint64_t below_va = va >= 8 ? ~0ull : ((1ull << (8 * va)) - 1);
      keep8 = below_vb & ~below_va;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      // V fragments are read and consumed a quarter of the head dim at a time
      if (dt % (NDT / 4) == 0) __builtin_amdgcn_sched_barrier(0);
      const int d = 16 * dt + c;
      const uint8_t* vrow = vl + d * T::VROW;
      if constexpr (MX) {
        // row d of the tile: 32-token units with the unit index swizzled by
        // d mod 4; the lane's tokens 8g .. 8g+7 of step tg are 4 bytes of
        // unit tg.  FP4 has no NaN: masked tokens need no V mask (their P is
        // 0 and their scale factor 0).
        const uint32_t raw = *(const uint32_t*)(vrow + ((tg ^ (d & (T::VUPR - 1))) * 16) + 4 * g);
        const h2 h0 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 0));
        const h2 h1 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 1));
        const h2 h2_ = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 2));
        const h2 h3 = __builtin_bit_cast(h2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(raw, 1.0f, 3));
        const half8 vf = half8{h0[0], h0[1], h1[0], h1[1], h2_[0], h2_[1], h3[0], h3[1]};
#pragma unroll
        for (int rt = 0; rt < NRW; ++rt)
          o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pfx[dt / 2][rt], o[rt][dt], 0, 0, 0);
      } else if constexpr (FP8) {
        const int q = (2 * tg + (g >> 1)) ^ (d & 7);
        u32x2 raw = *(const u32x2*)(vrow + q * 16 + (g & 1) * 8);
        if constexpr (!IN) {
          if (vmask) {
            raw[0] &= (uint32_t)keep8;
            raw[1] &= (uint32_t)(keep8 >> 32);
          }
        }
        const half8 vf = fp8x8_to_half8(raw);
#pragma unroll
        for (int rt = 0; rt < NRW; ++rt)
          o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[rt], o[rt][dt], 0, 0, 0);
      } else {
        const int q = (4 * tg + g) ^ (d & 15);
        u32x4 raw = *(const u32x4*)(vrow + q * 16);
        if constexpr (!IN) {
          if (vmask) {
#pragma unroll
            for (int q2 = 0; q2 < 4; ++q2) {
              uint32_t keep = 0;
              if (2 * q2 >= va && 2 * q2 < vb) keep |= 0xFFFFu;
              if (2 * q2 + 1 >= va && 2 * q2 + 1 < vb) keep |= 0xFFFF0000u;
              raw[q2] &= keep;
            }
          }
        }
        const bf16x8 vf = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int rt = 0; rt < NRW; ++rt) {
          o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[rt], o[rt][dt], 0, 0, 0);
          o[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[rt], o[rt][dt], 0, 0, 0);
        }
      }
    }
  };
  // The steps of a tile run as a real (not unrolled) loop with an opaque trip
  // count: with the PV MFMAs of several steps in one block the compiler unties
  // their accumulators and shuffles O between registers every iteration.
  auto compute_tile = [&](auto PTc, auto INc, int tile, const uint8_t* stg) {
    const int ts = t0 + tile * TT;
    int nst = R::STEPS;
    asm volatile("" : "+s"(nst));
#pragma unroll 1
    for (int st = 0; st < nst; ++st) step(PTc, INc, ts, wt * R::STEPS + st, stg);
    // publish an overflow of this wave so the whole workgroup restarts
    if (__builtin_amdgcn_ballot_w64(ovf) && lane == 0) *restart_flag = 1;
  };

  // Tiles [ti0, ti1) are interior (no masks); the others are boundary tiles.
  // Leading boundary, interior and trailing boundary tiles run in three
  // separate loops so that each loop body is one straight code path.
  int ti0 = tb, ti1 = tb;  // interior range within [tb, te)
  {
    // interior iff ts >= lo_max and ts + TT - 1 <= hi_min, ts = t0 + TT*tile
    const int first = lo_max > t0 ? (lo_max - t0 + TT - 1) / TT : 0;
    const int last = hi_min - t0 - (TT - 1) >= 0 ? (hi_min - t0 - (TT - 1)) / TT + 1 : 0;  // exclusive
    ti0 = min(max(first, tb), te);
    ti1 = max(min(last, te), ti0);
  }

  // ---- main loop: one attempt over the item's tiles ----
  bool first_attempt = true;
  bool scan = false;  // the scan pass: an attempt that does not stop at an overflow
  auto attempt = [&](auto PTc) {
    if constexpr (!SPARSE) {
      // NST-deep ring: tiles tb .. tb+NST-2 in flight before the first compute
      // (the first attempt's were issued before the query split).
      if (!first_attempt) {
#pragma unroll
        for (int k = 0; k < NST - 1; ++k)
          if (tb + k < te) issue_tile(tb + k, stage_base + k * T::STAGE);
      }
      // returns false if an overflow stopped the attempt
      auto tiles = [&](auto INc, int from, int to) -> bool {
        if constexpr (NST == 1) {
          // one stage: issue the tile, wait for every wave's loads, compute,
          // and let every wave finish reading before the next issue
          for (int tile = from; tile < to; ++tile) {
            issue_tile(tile, stage_base);
            wait_vmcnt<0>();
            wait_lgkm0();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            if (!scan && *(volatile int*)restart_flag) return false;  // an overflow: stop this attempt
            compute_tile(PTc, INc, tile, stage_base);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
          }
          return true;
        }
        for (int tile = from; tile < to; ++tile) {
          const int cur = (tile - tb) % NST;
          // wait for this tile's loads; the later tiles' loads stay in flight
          const int ahead = min(te - 1 - tile, NST - 2);  // tiles issued after this one
          constexpr int PER = T::KPT + T::VPT;
          const bool extra = FP8 && decltype(PTc)::value && w == 0;  // wave 0 also loads scales
          if (ahead <= 0) {
            wait_vmcnt<0>();
          } else if (ahead == 1) {
            if (extra) wait_vmcnt<(PER + 1) % 64>();
            else wait_vmcnt<PER % 64>();
          } else {
            if (extra) wait_vmcnt<(2 * (PER + 1)) % 64>();  // (the modulus only for one-stage kernels, which never get here)
            else wait_vmcnt<(2 * PER) % 64>();
          }
          wait_lgkm0();  // this wave's LDS writes (restart flag) are done
          // all waves' loads of this tile landed and tile-1 compute is done; the
          // empty asm statements keep the compiler from moving LDS accesses across
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_barrier();
          asm volatile("" ::: "memory");
          if (!scan && *(volatile int*)restart_flag) return false;  // an overflow: stop this attempt
          if (tile + NST - 1 < te)
            issue_tile(tile + NST - 1, stage_base + ((tile - tb + NST - 1) % NST) * T::STAGE);
          compute_tile(PTc, INc, tile, stage_base + cur * T::STAGE);
        }
        return true;
      };
      if (tiles(std::false_type{}, tb, ti0))
        if (tiles(std::true_type{}, ti0, ti1)) tiles(std::false_type{}, ti1, te);
      wait_vmcnt<0>();  // drain the ring (loads issued past a stop)
    } else {
      Staged<D, FP8, NTHREADS> st;
      if (tb < te) {
        load_sparse(tb, st);
        store_sparse(st, stage_base);
      }
      // The gather's issue is bound by the vector memory unit's address
      // processing (a tile's byte gathers take several times its compute),
      // and a wave issuing loads cannot compute meanwhile.  Half the waves
      // issue their share of the next tile before computing this one, the
      // other half after, so the unit is kept busy through the compute.
      const bool early = w >= NWAVES / 2;
      for (int tile = tb; tile < te; ++tile) {
        __syncthreads();
        if (!scan && *(volatile int*)restart_flag) break;
        const int cur = (tile - tb) & 1;
        const bool more = tile + 1 < te;
        if (more && early) load_sparse(tile + 1, st);
        if (tile >= ti0 && tile < ti1)
          compute_tile(PTc, std::true_type{}, tile, stage_base + cur * T::STAGE);
        else
          compute_tile(PTc, std::false_type{}, tile, stage_base + cur * T::STAGE);
        if (more && !early) load_sparse(tile + 1, st);
        if (more) store_sparse(st, stage_base + (cur ^ 1) * T::STAGE);
      }
    }
  };
  // Restarts.  An attempt that overflowed raises the references only to the
  // maxima it saw before it stopped, so logits that keep climbing could stop
  // every later attempt as well.  The first restart is therefore a scan pass
  // that runs through the whole item: without an overflow its result stands;
  // with one, the maxima it recorded (every score above its reference + TAU,
  // every V-scale maximum above its band) raise each reference to at least
  // the largest value of the item, and the last pass cannot overflow for any
  // finite input.  At most three passes.
  auto run = [&](auto PTc) {
    for (int pass = 0;; ++pass, first_attempt = false) {
#pragma unroll
      for (int rt = 0; rt < NRW; ++rt) {
        l_part[rt] = 0.f;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[rt][dt] = f4{0.f, 0.f, 0.f, 0.f};
      }
      scan = pass == 1;
      attempt(PTc);
      __syncthreads();
      const bool again = *(volatile int*)restart_flag != 0;
      if (!again || pass == 2) break;
      // restart with the larger references
      __syncthreads();
      if (tid == 0) *restart_flag = 0;
#pragma unroll
      for (int rt = 0; rt < NRW; ++rt) m_ref[rt] = fmaxf(m_ref[rt], m_hi[rt]);
      if (vs_hi > vs_ref) {
        vs_ref = vs_hi;
        inv_ref = 1.0f / vs_ref;
      }
#pragma unroll
      for (int b4 = 0; b4 < NVB; ++b4) erb[b4] = (int)group_max((float)max(erb[b4], ehb[b4]));  // wave-uniform
      ovf = false;
      __syncthreads();
    }
  };
  if constexpr (MX) {
    run(std::true_type{});
  } else if constexpr (FP8) {
    if (per_token)
      run(std::true_type{});
    else
      run(std::false_type{});
  } else {
    run(std::false_type{});
  }

  // ---- merge the token groups' states of each row ----
  constexpr int NR = NRT * 16;  // rows of the item (padded)
  float l_row[NRW];
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) l_row[rt] = group_sum(l_part[rt]);
  __syncthreads();  // all waves done with the stages (the merge buffer aliases them)
  float* wm = stats;                          // [WT][NR] m_ref
  float* wl = stats + R::WT * NR;             // [WT][NR] l
  float* wref = stats + 2 * R::WT * NR;       // [NWAVES] v-scale reference
  float* rowinfo = wref + NWAVES;             // [NR][4]: M, Ltot, out factor
  if (g == 0) {
#pragma unroll
    for (int rt = 0; rt < NRW; ++rt) {
      const int r = (wr * NRW + rt) * 16 + c;
      wm[wt * NR + r] = m_ref[rt];
      wl[wt * NR + r] = l_row[rt];
    }
  }
  if (lane == 0) wref[w] = vs_ref;
  __syncthreads();
  // weight of this wave's O for each of its rows
  float fw[NRW];
#pragma unroll
  for (int rt = 0; rt < NRW; ++rt) {
    const int r = (wr * NRW + rt) * 16 + c;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < R::WT; ++k)
      if (wl[k * NR + r] > 0.f) M = fmaxf(M, wm[k * NR + r]);
    fw[rt] = (l_row[rt] > 0.f) ? __builtin_amdgcn_exp2f(m_ref[rt] - M) * vs_ref : 0.f;
  }
  if (tid < NR) {
    const int r = tid;
    float M = -INFINITY, Lt = 0.f;
#pragma unroll
    for (int k = 0; k < R::WT; ++k)
      if (wl[k * NR + r] > 0.f) M = fmaxf(M, wm[k * NR + r]);
#pragma unroll
    for (int k = 0; k < R::WT; ++k) {
      const float lw = wl[k * NR + r];
      if (lw > 0.f) Lt += lw * __builtin_amdgcn_exp2f(wm[k * NR + r] - M);
    }
    float factor = 0.f;  // direct output: out = O * factor
    if (Lt > 0.f) {
      if (a.has_sinks) {
        const int gr = row0 + (r < nrows ? r : 0);
        const int h = kvh * a.G + gr % a.G;
        const float sk = a.sinks[h] * LOG2E;
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
  // O buffer [NR][D+4]: token group 0 writes its rows, the others add in turn
  constexpr int OROW = D + 4;
  float* obuf = (float*)stage_base;
#pragma unroll
  for (int k = 0; k < R::WT; ++k) {
    if (wt == k) {
#pragma unroll
      for (int rt = 0; rt < NRW; ++rt)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          f4* dst = (f4*)(obuf + ((wr * NRW + rt) * 16 + c) * OROW + 16 * dt + 4 * g);
          const f4 v = o[rt][dt] * (MX ? fw[rt] * __builtin_amdgcn_ldexpf(1.0f, erb[dt / 2] - 127) : fw[rt]);
          *dst = (k == 0) ? v : *dst + v;
        }
    }
    __syncthreads();
  }

  // ---- write: partial state or final rows ----
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
      const int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
      *(f4*)(po + (size_t)r * D + d4) = *(const f4*)(obuf + r * OROW + d4);
    }
    if (a.merge_ctr) {
      __syncthreads();  // the O buffer read: its LDS is the merge's
      const MergeArgs ma{a.out, a.workspace, a.sinks, a.QL, a.Hq, a.G, a.rows_total, a.rows_per_group, a.q_fp16,
                         a.has_sinks};
      arrive_and_merge<D>(ma, a.merge_ctr, it, stage_base);
    }
  } else {
    for (int e = tid; e < nrows * (D / 4); e += NTHREADS) {
      const int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
      const f4 v = *(const f4*)(obuf + r * OROW + d4) * rowinfo[r * 4 + 2];
      const int gr = row0 + r, i = gr / a.G, hl = gr % a.G;
      const long ooff = (((long)s * a.QL + i) * a.Hq + (long)kvh * a.G + hl) * D + d4;
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
}

// ---------------------------------------------------------------------------
// Partition reducer: out = sum_p w_p O_p / (sum_p w_p l_p + [sink]), with
// w_p = 2^(m_p - M), M = max(m_p over parts with l_p > 0, sink), partitions
// added in order (deterministic).  One workgroup per (entry, 1024/D rows:
// one output of 4 dims per thread); the partition weights of its rows are
// computed once into LDS.
// ---------------------------------------------------------------------------
struct ReduceArgs {
  void* out;
  const float* workspace;
  const float* sinks;
  const ReduceItem* entries;
  const MetaHeader* meta;
  uint32_t tag_lo, tag_hi;
  int QL, Hq, G, D, rows_total, rows_per_group, q_fp16, has_sinks, chunks_per_entry;
};

template <int D>
__global__ __launch_bounds__(256) void pa_reduce_kernel(ReduceArgs a) {
  constexpr int RR = merge_rows<D>();
  __shared__ float wgt[RR * kMaxPartitions];
  __shared__ float rowf[RR];
  const ReduceItem e = a.entries[blockIdx.x / a.chunks_per_entry];
  const MetaHeader mh = *a.meta;
  if (!meta_ok(mh, a.tag_lo, a.tag_hi)) return;  // not this plan's list: touch nothing
  if (e.nparts < 2) return;  // a unit with one partition wrote its rows itself
  const MergeArgs ma{a.out, a.workspace, a.sinks, a.QL, a.Hq, a.G, a.rows_total, a.rows_per_group, a.q_fp16,
                     a.has_sinks};
  merge_chunk_any<D>(ma, e, blockIdx.x % a.chunks_per_entry, wgt, rowf);
}

// ---------------------------------------------------------------------------
// Device-side re-partition of a refreshable plan (one workgroup).  The rule
// is the host planner's: per unit (sequence, KV head, row group) of T
// visible 128-token tiles, p = ceil(T / M) partitions (at most maxp and T;
// one for an empty unit, which clears its rows), M the smallest length whose
// partitions fit the item and slot budget; each unit's tiles are split
// evenly, the first T % p partitions taking one extra tile.
// ---------------------------------------------------------------------------
struct RefreshArgs {
  const int32_t* context_lens;
  int index_stride;
  MetaHeader* meta;
  MetaHeader header;  // the plan's header, written with the new list
  WorkItem* items;
  ReduceItem* reduce;
  int num_seqs, QL, window, causal, page_size, phys_page, table_stride, token_table, Hkv, row_groups;
  int maxp, n_items, n_slots;
};

constexpr int REF_T = 1024;  // threads of the refresh workgroup

__device__ int refresh_tiles(const RefreshArgs& a, int s) {
  const long cap = a.token_table == 2 ? (long)a.index_stride
                   : a.token_table    ? (long)a.table_stride
                                      : (long)a.table_stride * a.phys_page;
  const long L = min(max((long)a.context_lens[s], 0L), cap);
  long lo = 0;
  if (!a.token_table && L > 0 && a.window > 0) {
    const long first_pos = a.causal ? L - a.QL : L - 1;
    lo = max(0L, first_pos - a.window + 1);
  }
  const long t0 = a.token_table ? 0 : (lo / a.page_size) * a.page_size;
  return L > lo ? (int)((L - t0 + kTileTokens - 1) / kTileTokens) : 0;
}

__device__ __forceinline__ int refresh_parts(int T, int M, int maxp) {
  return T == 0 ? 1 : min(min((T + M - 1) / M, maxp), T);
}

// block-wide sum of one long per thread
__device__ long refresh_sum(long v, long* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int o = REF_T / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const long r = red[0];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(REF_T) void pa_refresh_kernel(RefreshArgs a) {
  __shared__ long red[REF_T];
  __shared__ long scan_i[REF_T], scan_s[REF_T];
  const int tid = threadIdx.x;
  const int U = a.Hkv * a.row_groups;
  // longest unit
  int tmax = 0;
  for (int s = tid; s < a.num_seqs; s += REF_T) tmax = max(tmax, refresh_tiles(a, s));
  red[tid] = tmax;
  __syncthreads();
  for (int o = REF_T / 2; o > 0; o >>= 1) {
    if (tid < o) red[tid] = max(red[tid], red[tid + o]);
    __syncthreads();
  }
  tmax = (int)red[0];
  __syncthreads();
  // smallest feasible M in [1, max(tmax, 1)] (M = tmax gives one partition per unit)
  int lo = 1, hi = max(tmax, 1);
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    long ni = 0, ns = 0;
    for (int s = tid; s < a.num_seqs; s += REF_T) {
      const int p = refresh_parts(refresh_tiles(a, s), mid, a.maxp);
      ni += p;
      ns += p > 1 ? p : 0;
    }
    ni = refresh_sum(ni, red) * U;
    ns = refresh_sum(ns, red) * U;
    if (ni <= a.n_items && ns <= a.n_slots)
      hi = mid;
    else
      lo = mid + 1;
  }
  const int M = lo;
  // emit, REF_T sequences at a time: exclusive scans of items and slots
  long item_base = 0, slot_base = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += REF_T) {
    const int s = c0 + tid;
    const int T = s < a.num_seqs ? refresh_tiles(a, s) : 0;
    const int p = s < a.num_seqs ? refresh_parts(T, M, a.maxp) : 0;
    scan_i[tid] = (long)p * U;
    scan_s[tid] = p > 1 ? (long)p * U : 0;
    __syncthreads();
    for (int o = 1; o < REF_T; o <<= 1) {  // inclusive Hillis-Steele scans
      const long vi = tid >= o ? scan_i[tid - o] : 0, vs = tid >= o ? scan_s[tid - o] : 0;
      __syncthreads();
      scan_i[tid] += vi;
      scan_s[tid] += vs;
      __syncthreads();
    }
    const long ib = item_base + scan_i[tid] - (long)p * U, sb = slot_base + scan_s[tid] - (p > 1 ? (long)p * U : 0);
    if (s < a.num_seqs) {
      for (int g = 0; g < a.Hkv; ++g)
        for (int rg = 0; rg < a.row_groups; ++rg) {
          const int u = g * a.row_groups + rg;
          const long first = sb + (long)u * p;
          a.reduce[(long)s * U + u] = ReduceItem{s, g, rg, p > 1 ? (int)first : 0, p > 1 ? p : 0, 0, 0, 0};
          const int base = T / p, extra = T % p;
          for (int part = 0; part < p; ++part) {
            const int b = part * base + min(part, extra);
            const int e = b + base + (part < extra ? 1 : 0);
            a.items[ib + (long)u * p + part] =
                WorkItem{s, g, rg, b, part == p - 1 ? -1 : e, p > 1 ? (int)(first + part) : -1, part, p};
          }
        }
    }
    item_base += scan_i[REF_T - 1];
    slot_base += scan_s[REF_T - 1];
    __syncthreads();
  }
  for (long i = item_base + tid; i < a.n_items; i += REF_T) a.items[i] = WorkItem{-1, 0, 0, 0, 0, -1, 0, 1};
  if (tid == 0) *a.meta = a.header;  // the buffer now holds this plan's list
}

// ---------------------------------------------------------------------------
// Launch selection
// ---------------------------------------------------------------------------
template <int D, bool FP8, int NRT, bool SPARSE, bool MX = false>
static pa_status launch_one(const KernelArgs& args, int nblocks, hipStream_t stream) {
  constexpr int bytes = Smem<D, FP8, NRT, SPARSE, MX>::TOTAL;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static bool configured = false;
  if (!configured) {
    if (hipFuncSetAttribute((const void*)pa_decode_kernel<D, FP8, NRT, SPARSE, MX>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "hipFuncSetAttribute failed");
    }
    configured = true;
  }
  hipLaunchKernelGGL((pa_decode_kernel<D, FP8, NRT, SPARSE, MX>), dim3(nblocks), dim3((Waves<NRT, D>::NT)), bytes, stream,
                     args);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("decode launch failed: ") + hipGetErrorString(err));
  return PA_OK;
}

template <int D, bool FP8, int NRT>
static pa_status launch_sp(bool sparse, const KernelArgs& args, int n, hipStream_t st) {
  if constexpr (D >= 512) return launch_one<D, FP8, NRT, false>(args, n, st);  // dense caches only (validated)
  else return sparse ? launch_one<D, FP8, NRT, true>(args, n, st) : launch_one<D, FP8, NRT, false>(args, n, st);
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

// pa_decode and pa_decode_sparse (topk: the top-k index table of a
// token_table = 2 problem, else NULL; context_lens: its counts).
static pa_status decode_impl(const pa_plan_t* plan, void* out, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables, const int32_t* topk,
                             const int32_t* context_lens, const float* k_scale, const float* v_scale,
                             const float* sinks, void* meta_dev, void* workspace_dev, void* stream) {
  const Plan& P = plan->plan;
  const pa_problem& p = P.prob;
  if (P.items.empty()) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || (p.token_table == 2 && !topk))
    return set_error(PA_ERR_INVALID, "a required device pointer is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return set_error(PA_ERR_INVALID, "q, out, k_cache and v_cache must be 16-byte aligned");
  if (p.kv_dtype == PA_FP8_E4M3FN || p.kv_dtype == PA_MXFP4) {
    if (!k_scale || !v_scale) return set_error(PA_ERR_INVALID, "FP8 and MXFP4 caches need k_scale and v_scale");
    if (p.scale_mode != PA_SCALE_PER_TENSOR && (!aligned16(k_scale) || !aligned16(v_scale)))
      return set_error(PA_ERR_INVALID, "per-token and block scales must be 16-byte aligned");
  }
  if (p.has_sinks && !sinks) return set_error(PA_ERR_INVALID, "has_sinks set but sinks is NULL");
  if (!meta_dev) return set_error(PA_ERR_WORKSPACE, "meta_dev is NULL");
  if (!meta_registry_holds(meta_dev, P.serial))
    return set_error(PA_ERR_WORKSPACE, "meta_dev does not hold this plan's metadata: call pa_plan_upload first");
  if (P.num_slots > 0 && !workspace_dev) return set_error(PA_ERR_WORKSPACE, "workspace_dev is NULL");
  hipStream_t st = (hipStream_t)stream;
  // bytes of head_dim * page_size elements of one KV head's page
  const long long head_bytes = (long long)p.head_dim * p.page_size *
                               (p.kv_dtype == PA_BF16 ? 2 : 1) / (p.kv_dtype == PA_MXFP4 ? 2 : 1);
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
  args.topk = p.token_table == 2 ? topk : nullptr;
  args.index_stride = p.index_stride;
  args.items = (const WorkItem*)((const uint8_t*)meta_dev + Plan::items_offset());
  args.meta = (const MetaHeader*)meta_dev;
  args.tag_lo = (uint32_t)P.serial;
  args.tag_hi = (uint32_t)(P.serial >> 32);
  args.workspace = (float*)workspace_dev;
  args.merge_ctr = P.in_kernel_merge ? (int*)((uint8_t*)meta_dev + P.counters_offset()) : nullptr;
  args.head_stride = head_bytes;
  args.page_stride = args.head_stride * p.num_kv_heads;
  args.QL = p.query_len;
  args.Hq = p.num_q_heads;
  args.Hkv = p.num_kv_heads;
  args.G = p.num_q_heads / p.num_kv_heads;
  // dense caches index tokens by sub-pages of at most 128 (the tile), token
  // tables by the physical page
  args.page_size = (p.token_table || p.page_size <= kTileTokens) ? p.page_size : kTileTokens;
  args.page_sub = 31 - __builtin_clz((unsigned)(p.page_size / args.page_size));
  args.phys_page = p.page_size;
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
  if (stream_kernel_applies(P)) return launch_stream(P, args, n, st);
  if (p.kv_dtype == PA_MXFP4) {  // head dim 128, page tables (validated)
    if (P.nrt == 1) return launch_one<128, true, 1, false, true>(args, n, st);
    if (P.nrt == 2) return launch_one<128, true, 2, false, true>(args, n, st);
    return launch_one<128, true, 4, false, true>(args, n, st);
  }
  if (p.kv_dtype == PA_FP8_E4M3FN) {
    if (p.head_dim == 64) return launch_nrt<64, true>(P.nrt, sparse, args, n, st);
    if (p.head_dim == 128) return launch_nrt<128, true>(P.nrt, sparse, args, n, st);
    if (p.head_dim == 512) return launch_nrt<512, true>(P.nrt, sparse, args, n, st);
    return launch_nrt<256, true>(P.nrt, sparse, args, n, st);
  }
  if (p.head_dim == 64) return launch_nrt<64, false>(P.nrt, sparse, args, n, st);
  return launch_nrt<128, false>(P.nrt, sparse, args, n, st);
}

extern "C" pa_status pa_decode(const pa_plan_t* plan, void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                               const float* k_scale, const float* v_scale, const float* sinks, void* meta_dev,
                               void* workspace_dev, void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  if (plan->plan.prob.token_table == 2)
    return set_error(PA_ERR_INVALID, "a plan for top-k index tables needs pa_decode_sparse");
  return decode_impl(plan, out, q, k_cache, v_cache, block_tables, nullptr, context_lens, k_scale, v_scale, sinks,
                     meta_dev, workspace_dev, stream);
}

extern "C" pa_status pa_decode_sparse(const pa_plan_t* plan, void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables, const int32_t* topk_indices,
                                      const int32_t* topk_counts, const float* k_scale, const float* v_scale,
                                      const float* sinks, void* meta_dev, void* workspace_dev, void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  if (plan->plan.prob.token_table != 2)
    return set_error(PA_ERR_INVALID, "pa_decode_sparse needs a plan for top-k index tables (token_table 2)");
  return decode_impl(plan, out, q, k_cache, v_cache, block_tables, topk_indices, topk_counts, k_scale, v_scale, sinks,
                     meta_dev, workspace_dev, stream);
}

extern "C" pa_status pa_plan_refresh(const pa_plan_t* plan, const int32_t* context_lens, void* meta_dev,
                                     void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  const Plan& P = plan->plan;
  if (P.budget_items <= 0) return set_error(PA_ERR_INVALID, "the plan was made without refreshable");
  if (!meta_dev || (P.prob.num_seqs > 0 && !context_lens))
    return set_error(PA_ERR_INVALID, "meta_dev or context_lens is NULL");
  RefreshArgs ra;
  ra.context_lens = context_lens;
  ra.meta = (MetaHeader*)meta_dev;
  std::memcpy(&ra.header, P.meta_host.data(), sizeof(MetaHeader));
  ra.items = (WorkItem*)((uint8_t*)meta_dev + Plan::items_offset());
  ra.reduce = (ReduceItem*)((uint8_t*)meta_dev + P.reduce_offset());
  ra.num_seqs = P.prob.num_seqs;
  ra.QL = P.prob.query_len;
  ra.window = P.prob.sliding_window;
  ra.causal = P.prob.causal;
  ra.page_size = std::min(P.prob.page_size, kTileTokens);  // the kernels' tile origin (sub-pages above 128)
  ra.phys_page = P.prob.page_size;
  ra.table_stride = P.prob.table_stride;
  ra.token_table = P.prob.token_table;
  ra.index_stride = P.prob.index_stride;
  ra.Hkv = P.prob.num_kv_heads;
  ra.row_groups = P.row_groups;
  ra.maxp = P.maxp;
  ra.n_items = (int)P.items.size();
  ra.n_slots = P.num_slots;
  hipLaunchKernelGGL(pa_refresh_kernel, dim3(1), dim3(REF_T), 0, (hipStream_t)stream, ra);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("refresh launch failed: ") + hipGetErrorString(err));
  meta_registry_set(meta_dev, P.serial);  // the device list is now this plan's
  return PA_OK;
}

extern "C" pa_status pa_reduce(const pa_plan_t* plan, void* out, const float* sinks, void* meta_dev,
                               void* workspace_dev, void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  const Plan& P = plan->plan;
  if (P.reduce.empty() || P.in_kernel_merge) return PA_OK;  // nothing to merge, or merged by pa_decode
  if (!out) return set_error(PA_ERR_INVALID, "out is NULL");
  if (!aligned16(out)) return set_error(PA_ERR_INVALID, "out must be 16-byte aligned");
  if (P.prob.has_sinks && !sinks) return set_error(PA_ERR_INVALID, "has_sinks set but sinks is NULL");
  if (!meta_dev || !workspace_dev) return set_error(PA_ERR_WORKSPACE, "meta_dev or workspace_dev is NULL");
  if (!meta_registry_holds(meta_dev, P.serial))
    return set_error(PA_ERR_WORKSPACE, "meta_dev does not hold this plan's metadata: call pa_plan_upload first");
  ReduceArgs ra;
  ra.out = out;
  ra.workspace = (const float*)workspace_dev;
  ra.sinks = sinks;
  ra.entries = (const ReduceItem*)((const uint8_t*)meta_dev + P.reduce_offset());
  ra.meta = (const MetaHeader*)meta_dev;
  ra.tag_lo = (uint32_t)P.serial;
  ra.tag_hi = (uint32_t)(P.serial >> 32);
  ra.QL = P.prob.query_len;
  ra.Hq = P.prob.num_q_heads;
  ra.G = P.prob.num_q_heads / P.prob.num_kv_heads;
  ra.D = P.prob.head_dim;
  ra.rows_total = P.rows_total;
  ra.rows_per_group = P.rows_per_group;
  ra.q_fp16 = P.prob.q_dtype == PA_FP16;
  ra.has_sinks = P.prob.has_sinks;
  const int D = P.prob.head_dim;
  const int rr = D == 512 ? merge_rows<512>() : D == 256 ? merge_rows<256>() : D == 64 ? merge_rows<64>() : merge_rows<128>();
  ra.chunks_per_entry = (P.rows_per_group + rr - 1) / rr;
  const unsigned grid = (unsigned)(P.reduce.size() * ra.chunks_per_entry);
  if (D == 512)
    hipLaunchKernelGGL(pa_reduce_kernel<512>, dim3(grid), dim3(256), 0, (hipStream_t)stream, ra);
  else if (P.prob.head_dim == 256)
    hipLaunchKernelGGL(pa_reduce_kernel<256>, dim3(grid), dim3(256), 0, (hipStream_t)stream, ra);
  else if (P.prob.head_dim == 64)
    hipLaunchKernelGGL(pa_reduce_kernel<64>, dim3(grid), dim3(256), 0, (hipStream_t)stream, ra);
  else
    hipLaunchKernelGGL(pa_reduce_kernel<128>, dim3(grid), dim3(256), 0, (hipStream_t)stream, ra);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return set_error(PA_ERR_DEVICE, std::string("reduce launch failed: ") + hipGetErrorString(err));
  return PA_OK;
}
