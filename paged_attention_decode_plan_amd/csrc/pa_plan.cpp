// Host work planner and the host-only part of the C ABI.
//
// Split-KV planning follows the FlyDSL decode pages: partitions per
// (sequence, KV head) are bounded by the device compute-unit count and a
// static 256-partition limit (aiter PR #4332, the commit that defaults the
// per-sequence plan limit to the CU count); the partitioned range of a
// sequence is the union of the tiles its query rows can see under a sliding
// window and multi-token (MTP) rows, and the staged page ids cover only that
// union (aiter PR #6617 "Extend packed D256 PA decode pipe", summary); empty
// sequences clear their rows (aiter PR #7079, "Partition merges").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <functional>
#include <mutex>
#include <queue>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_internal.h"

namespace pa {

static thread_local std::string g_last_error;

pa_status set_error(pa_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

static std::atomic<uint64_t> g_next_serial{1};
static std::mutex g_registry_mutex;
static std::unordered_map<const void*, uint64_t> g_registry;

void meta_registry_set(const void* meta_dev, uint64_t serial) {
  std::lock_guard<std::mutex> lock(g_registry_mutex);
  g_registry[meta_dev] = serial;
}

bool meta_registry_holds(const void* meta_dev, uint64_t serial) {
  std::lock_guard<std::mutex> lock(g_registry_mutex);
  auto it = g_registry.find(meta_dev);
  return it != g_registry.end() && it->second == serial;
}

pa_status validate_problem(const pa_problem* p) {
  if (!p) return set_error(PA_ERR_INVALID, "problem is NULL");
  if (p->num_seqs < 0) return set_error(PA_ERR_INVALID, "num_seqs < 0");
  if (p->query_len < 1) return set_error(PA_ERR_INVALID, "query_len < 1");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1) return set_error(PA_ERR_INVALID, "head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return set_error(PA_ERR_INVALID, "num_q_heads must be a multiple of num_kv_heads");
  if (p->head_dim < 1 || p->page_size < 1) return set_error(PA_ERR_INVALID, "head_dim and page_size must be >= 1");
  if (p->num_pages < 0) return set_error(PA_ERR_INVALID, "num_pages < 0");
  if (p->num_seqs > 0 && p->table_stride < 1) return set_error(PA_ERR_INVALID, "table_stride < 1");
  if (p->sliding_window < 0) return set_error(PA_ERR_INVALID, "sliding_window < 0");
  if (p->q_dtype != PA_BF16 && p->q_dtype != PA_FP16) return set_error(PA_ERR_INVALID, "q_dtype must be BF16 or FP16");
  if (p->kv_dtype != PA_FP8_E4M3FN && p->kv_dtype != PA_BF16 && p->kv_dtype != PA_MXFP4)
    return set_error(PA_ERR_INVALID, "kv_dtype must be FP8_E4M3FN, BF16 or MXFP4");
  if (p->v_layout != PA_V_PLAIN && p->v_layout != PA_V_TRANSPOSED) return set_error(PA_ERR_INVALID, "bad v_layout");
  if (p->scale_mode < PA_SCALE_NONE || p->scale_mode > PA_SCALE_MX)
    return set_error(PA_ERR_INVALID, "bad scale_mode");
  if ((p->causal | p->has_sinks) & ~1) return set_error(PA_ERR_INVALID, "flags must be 0 or 1");
  if (p->token_table < 0 || p->token_table > 2) return set_error(PA_ERR_INVALID, "token_table must be 0, 1 or 2");
  if (p->token_table == 2 && p->num_seqs > 0 && p->index_stride < 1)
    return set_error(PA_ERR_INVALID, "top-k index tables need index_stride >= 1");
  double cache_elems = (double)p->num_pages * p->num_kv_heads * p->page_size * p->head_dim;
  if (cache_elems > (double)(1ull << 40)) return set_error(PA_ERR_INVALID, "cache larger than 2^40 elements");
  // Valid but not implemented here.
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256 && p->head_dim != 512)
    return set_error(PA_ERR_UNSUPPORTED, "head_dim must be 64, 128, 256 or 512");
  if (p->head_dim == 512 && (p->kv_dtype != PA_FP8_E4M3FN || p->token_table))
    return set_error(PA_ERR_UNSUPPORTED, "head_dim 512 needs FP8 caches and page tables");
  if (p->page_size < 16 || p->page_size > 1024 || (p->page_size & (p->page_size - 1)))
    return set_error(PA_ERR_UNSUPPORTED, "page_size must be a power of two from 16 to 1024");
  if (p->token_table && p->page_size > kTileTokens)
    return set_error(PA_ERR_UNSUPPORTED, "token tables support pages of at most 128 tokens");
  if (p->kv_dtype == PA_FP8_E4M3FN && p->scale_mode == PA_SCALE_NONE)
    return set_error(PA_ERR_UNSUPPORTED, "FP8 caches need a per-tensor or per-token scale");
  if (p->kv_dtype == PA_BF16 && p->scale_mode != PA_SCALE_NONE)
    return set_error(PA_ERR_UNSUPPORTED, "BF16 caches take no dequant scale");
  if (p->kv_dtype == PA_BF16 && p->head_dim == 256)
    return set_error(PA_ERR_UNSUPPORTED, "BF16 caches support head_dim 64 and 128");
  if (p->kv_dtype == PA_BF16 && p->q_dtype != PA_BF16)
    return set_error(PA_ERR_UNSUPPORTED, "BF16 caches need BF16 queries");
  if (p->token_table && (p->sliding_window > 0 || p->query_len != 1))
    return set_error(PA_ERR_UNSUPPORTED, "token tables need query_len 1 and no sliding window");
  if ((p->kv_dtype == PA_MXFP4) != (p->scale_mode == PA_SCALE_MX))
    return set_error(PA_ERR_UNSUPPORTED, "MXFP4 caches take (only) the MX block scales");
  if (p->kv_dtype == PA_MXFP4 &&
      (p->head_dim != 128 || p->page_size < 32 || p->page_size > kTileTokens || p->token_table ||
       p->v_layout != PA_V_PLAIN))
    return set_error(PA_ERR_UNSUPPORTED,
                     "MXFP4 caches: head_dim 128, page_size 32 to 128, page tables and the plain V layout");
  return PA_OK;
}

// Workgroups of the decode kernel that stay resident on one CU together.
// (16-row items: 4-wave workgroups, two per CU; 17-64-row items: one
// workgroup per CU, the 8-wave tile kernel or the 4-wave streaming kernel;
// head dim 256 and BF16 caches fill the LDS with one.)
static int resident_per_cu(const pa_problem& p, int nrt) {
  if (nrt >= 2 || p.head_dim > 128 || p.kv_dtype == PA_BF16 || p.token_table) return 1;
  return 2;
}

static inline long ceil_div(long a, long b) { return (a + b - 1) / b; }

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_plan(const pa_problem* problem, const int32_t* context_lens_host, const pa_plan_opts* opts,
                             pa_plan_t** out) {
  if (!out) return set_error(PA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  pa_status st = validate_problem(problem);
  if (st != PA_OK) return st;
  if (problem->num_seqs > 0 && !context_lens_host) return set_error(PA_ERR_INVALID, "context_lens_host is NULL");
  pa_plan_opts o{};
  if (opts) o = *opts;
  if (o.merge < 0 || o.merge > 2) return set_error(PA_ERR_INVALID, "merge must be 0, 1 or 2");
  if (o.cu_count < 0 || o.max_partitions < 0 || o.partition_tokens < 0 || o.stage_limit < 0)
    return set_error(PA_ERR_INVALID, "plan options must be >= 0");
  if (o.refreshable & ~1) return set_error(PA_ERR_INVALID, "refreshable must be 0 or 1");
  const pa_problem& p = *problem;
  // MXFP4 caches take 256-token partitions (aiter PR #7079, merge of #7056)
  const bool mx = p.kv_dtype == PA_MXFP4;
  if (mx && (o.refreshable || (o.partition_tokens != 0 && o.partition_tokens != 2 * kTileTokens)))
    return set_error(PA_ERR_UNSUPPORTED, "MXFP4 plans take 256-token partitions and are not refreshable");

  int cu = o.cu_count;
  if (cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "cu_count is 0 and the device CU count could not be queried");
    }
  }

  auto* handle = new pa_plan_s();
  Plan& P = handle->plan;
  P.prob = p;
  if (P.prob.softmax_scale <= 0.f) P.prob.softmax_scale = 1.0f / std::sqrt((float)p.head_dim);
  P.opts = o;
  P.cu_count = cu;
  const int G = p.num_q_heads / p.num_kv_heads;
  P.rows_total = p.query_len * G;
  P.rows_per_group = std::min(P.rows_total, kMaxRowsPerItem);
  P.row_groups = (int)ceil_div(P.rows_total, kMaxRowsPerItem);
  int rt = (int)ceil_div(P.rows_per_group, 16);
  P.nrt = rt <= 1 ? 1 : (rt <= 2 ? 2 : 4);
  P.stage_limit = o.stage_limit > 0 ? std::min(o.stage_limit, kStageCap) : kStageCap;
  P.scale_log2 = P.prob.softmax_scale * 1.4426950408889634f;
  int maxp = o.max_partitions > 0 ? o.max_partitions : cu;
  maxp = std::max(1, std::min(maxp, kMaxPartitions));

  // Tiles of each sequence's visible span (the same for all its KV heads).
  const long cap = p.token_table == 2 ? (long)p.index_stride
                   : p.token_table    ? (long)p.table_stride
                                      : (long)p.table_stride * p.page_size;
  std::vector<int> seq_tiles(p.num_seqs, 0);
  for (int s = 0; s < p.num_seqs; ++s) {
    long L = std::min<long>(std::max<long>(context_lens_host[s], 0), cap);
    long lo = 0, hi = L;
    if (!p.token_table && L > 0 && p.sliding_window > 0) {
      long first_pos = p.causal ? L - p.query_len : L - 1;
      lo = std::max<long>(0, first_pos - p.sliding_window + 1);
    }
    // tiles start at the (sub-)page boundary the kernels index by: pages
    // above 128 tokens are taken as sub-pages of 128
    const long vps = std::min(p.page_size, kTileTokens);
    long t0 = p.token_table ? 0 : (lo / vps) * vps;
    seq_tiles[s] = hi > lo ? (int)ceil_div(hi - t0, kTileTokens) : 0;
  }
  // Partitions are cut at multiples of gran tiles of the span (MXFP4: 256
  // tokens); the choices below count in those units.
  const int gran = mx ? 2 : 1;
  std::vector<int> seq_units(p.num_seqs, 0);
  for (int s = 0; s < p.num_seqs; ++s) seq_units[s] = (int)ceil_div(seq_tiles[s], gran);

  // Units: (sequence, KV head, row group).  Choose partition counts.
  const int units_per_seq = p.num_kv_heads * P.row_groups;
  const long nunits = (long)p.num_seqs * units_per_seq;
  std::vector<int> parts(p.num_seqs, 1);  // identical for every unit of a sequence
  const int occ = resident_per_cu(p, P.nrt);
  const long slots_budget = std::max<long>((long)cu * occ, nunits);
  if (o.partition_tokens > 0) {
    int units_per_part = (int)ceil_div(ceil_div(o.partition_tokens, kTileTokens), gran);
    for (int s = 0; s < p.num_seqs; ++s)
      parts[s] = std::max(1, std::min<int>({(int)ceil_div(seq_units[s], units_per_part), maxp,
                                            std::max(seq_units[s], 1)}));
  } else {
    // Greedy: split the sequence with the longest work item while the shorter
    // makespan outweighs the added partial traffic and the budget allows.
    const double elem = p.kv_dtype == PA_FP8_E4M3FN ? 1.0 : mx ? 0.5 : 2.0;
    const double tile_bytes = gran * kTileTokens * (2.0 * p.head_dim * elem + 8.0);  // of one unit
    const double partial_bytes = P.rows_per_group * (p.head_dim + 2.0) * 4.0;
    const double cost_per_item = 2.0 * partial_bytes / (tile_bytes * cu);  // in tile-times
    // The reducer takes a unit's partitions eight at a time, one memory
    // round trip (about one tile-time) each: an eighth of a tile-time per
    // partition on the merge's critical path, which does not add up over the
    // units it runs for in parallel.
    const double reduce_per_part = 0.125;
    auto greedy = [&](long budget) {
      std::vector<int> pr(p.num_seqs, 1);
      long items = nunits;
      using E = std::pair<long, int>;  // (current longest item tiles, seq)
      std::priority_queue<E> pq;
      for (int s = 0; s < p.num_seqs; ++s)
        if (seq_units[s] > 1) pq.push({seq_units[s], s});
      while (!pq.empty()) {
        auto [len, s] = pq.top();
        pq.pop();
        if (len <= 1) continue;
        // the smallest partition count that shortens this sequence's longest
        // item (one more partition may not, when the tiles do not divide)
        const int np = (int)ceil_div(seq_units[s], len - 1);
        if (np > maxp || np > seq_units[s]) continue;
        const long add = (long)(np - pr[s]) * units_per_seq;
        if (items + add > budget) break;
        long newlen = ceil_div(seq_units[s], np);
        // the first split of a sequence also creates its first partial slots
        double added = cost_per_item * units_per_seq * ((np - pr[s]) + (pr[s] == 1 ? 1 : 0)) +
                       reduce_per_part * (np - pr[s]);
        if ((double)(len - newlen) < added) continue;
        pr[s] = np;
        items += add;
        pq.push({newlen, s});
      }
      return pr;
    };
    parts = greedy(slots_budget);
    if (!o.refreshable) {
      // More items than resident workgroups (the dispatcher starts one as
      // another ends) balance long sequences better when one item per slot
      // leaves some slots with twice the work of others.  Estimated makespan
      // in tile-times: the items, longest first, each on the least loaded of
      // the resident slots, each paying a start of about four tile-times
      // (its first loads and page ids) plus its partial traffic.  A budget of
      // k slots' worth of items is taken when it is at least 3 % shorter.
      const long nslots = (long)cu * occ;
      const double start_tiles = 4.0;
      auto makespan = [&](const std::vector<int>& pr) {
        std::vector<double> len;
        for (int s = 0; s < p.num_seqs; ++s) {
          const int nt = seq_units[s], np = pr[s];
          for (int part = 0; part < np; ++part) {
            const int t = nt / np + (part < nt % np ? 1 : 0);
            for (int u = 0; u < units_per_seq; ++u)
              len.push_back(t + start_tiles + (np > 1 ? cost_per_item : 0.0));
          }
        }
        std::sort(len.begin(), len.end(), std::greater<double>());
        std::priority_queue<double, std::vector<double>, std::greater<double>> load;
        for (long i = 0; i < nslots; ++i) load.push(0.0);
        double worst = 0.0;
        for (double l : len) {
          const double t = load.top() + l;
          load.pop();
          load.push(t);
          worst = std::max(worst, t);
        }
        return worst;
      };
      double best = makespan(parts);
      for (int k = 2; k <= 8; ++k) {
        std::vector<int> pk = greedy(std::max(slots_budget, k * nslots));
        const double m = makespan(pk);
        if (m < 0.97 * best) {
          best = m;
          parts = pk;
        }
      }
    }
  }

  // Emit items: slots are contiguous per unit, in partition order.
  int slot = 0;
  P.max_parts = 1;
  P.total_tiles = 0;
  for (int s = 0; s < p.num_seqs; ++s) {
    int np = parts[s];
    int nt = seq_units[s];
    P.max_parts = std::max(P.max_parts, np);
    for (int g = 0; g < p.num_kv_heads; ++g)
      for (int rg = 0; rg < P.row_groups; ++rg) {
        int first = np > 1 ? slot : -1;
        if (np > 1) {
          P.reduce.push_back(ReduceItem{s, g, rg, slot, np, 0, 0, 0});
          slot += np;
        } else if (o.refreshable) {
          P.reduce.push_back(ReduceItem{s, g, rg, 0, 0, 0, 0, 0});  // one entry per unit: nothing to merge
        }
        for (int part = 0; part < np; ++part) {
          // balanced split: the first (nt % np) parts get one extra tile
          int base = nt / np, extra = nt % np;
          int b = part * base + std::min(part, extra);
          int e = b + base + (part < extra ? 1 : 0);
          b *= gran;
          e = std::min(e * gran, seq_tiles[s]);
          WorkItem w{s, g, rg, b, part == np - 1 ? -1 : e, np > 1 ? first + part : -1, part, np};
          P.items.push_back(w);
          P.total_tiles += e - b;
        }
      }
  }
  P.num_slots = slot;
  // Longest items first; ties keep (sequence, head, part) order.
  std::stable_sort(P.items.begin(), P.items.end(), [&](const WorkItem& a, const WorkItem& b) {
    auto len = [&](const WorkItem& w) {
      int e = w.tile_end >= 0 ? w.tile_end : seq_tiles[w.seq];
      return e - w.tile_begin;
    };
    return len(a) > len(b);
  });
  if (o.refreshable) {
    // A fixed budget that pa_plan_refresh re-partitions on the device: items
    // past the used ones do nothing (seq -1), and each item owns at most
    // one partial slot.
    P.maxp = maxp;
    P.budget_items = (int)std::max<long>(slots_budget, (long)P.items.size());
    P.items.resize(P.budget_items, WorkItem{-1, 0, 0, 0, 0, -1, 0, 1});
    P.num_slots = std::max(P.num_slots, P.budget_items);
  }
  P.serial = g_next_serial.fetch_add(1);
  // 2 (in-kernel merge) where asked; the library's choice is the reducer
  P.in_kernel_merge = o.merge == 2 && P.num_slots > 0;
  P.meta_host.assign(P.in_kernel_merge ? P.counters_offset() + (size_t)P.num_slots * Plan::kCounterBytes
                                       : P.reduce_offset() + P.reduce.size() * sizeof(ReduceItem),
                     0);  // counters start at zero
  const MetaHeader hdr{kMetaMagic, (uint32_t)P.serial, (uint32_t)(P.serial >> 32), (uint32_t)P.items.size(),
                       (uint32_t)P.reduce.size(), 0, 0, 0};
  std::memcpy(P.meta_host.data(), &hdr, sizeof hdr);
  if (!P.items.empty())
    std::memcpy(P.meta_host.data() + P.items_offset(), P.items.data(), P.items.size() * sizeof(WorkItem));
  if (!P.reduce.empty())
    std::memcpy(P.meta_host.data() + P.reduce_offset(), P.reduce.data(), P.reduce.size() * sizeof(ReduceItem));
  *out = handle;
  return PA_OK;
}

extern "C" pa_status pa_plan_sizes(const pa_plan_t* plan, size_t* meta_bytes, size_t* workspace_bytes) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  if (meta_bytes) *meta_bytes = plan->plan.meta_bytes();
  if (workspace_bytes) *workspace_bytes = plan->plan.workspace_bytes();
  return PA_OK;
}

extern "C" pa_status pa_plan_info(const pa_plan_t* plan, pa_plan_info_t* info) {
  if (!plan || !info) return set_error(PA_ERR_INVALID, "plan or info is NULL");
  const Plan& P = plan->plan;
  info->num_items = (int32_t)P.items.size();
  info->num_slots = P.num_slots;
  info->num_reduce = (int32_t)P.reduce.size();
  info->rows_per_group = P.rows_per_group;
  info->row_groups = P.row_groups;
  info->max_parts = P.max_parts;
  info->total_tiles = P.total_tiles;
  info->cu_count = P.cu_count;
  return PA_OK;
}

extern "C" pa_status pa_plan_work(const pa_plan_t* plan, int32_t* out, int32_t n_items_capacity) {
  if (!plan || (!out && n_items_capacity > 0)) return set_error(PA_ERR_INVALID, "plan or out is NULL");
  const Plan& P = plan->plan;
  if (n_items_capacity < (int32_t)P.items.size()) return set_error(PA_ERR_INVALID, "capacity too small");
  if (!P.items.empty()) std::memcpy(out, P.items.data(), P.items.size() * sizeof(WorkItem));
  return PA_OK;
}

extern "C" pa_status pa_plan_upload(const pa_plan_t* plan, void* meta_dev, void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  if (!meta_dev) return set_error(PA_ERR_WORKSPACE, "meta_dev is NULL");
  if (((uintptr_t)meta_dev & 15) != 0) return set_error(PA_ERR_INVALID, "meta_dev must be 16-byte aligned");
  const Plan& P = plan->plan;
  if (!P.meta_pinned) {
    // a pinned source keeps the copy asynchronous (and capturable in a graph)
    void* h = nullptr;
    if (hipHostMalloc(&h, P.meta_host.size(), hipHostMallocDefault) != hipSuccess || !h) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "pinned host buffer for the metadata could not be allocated");
    }
    std::memcpy(h, P.meta_host.data(), P.meta_host.size());
    P.meta_pinned = (uint8_t*)h;
  }
  if (hipMemcpyAsync(meta_dev, P.meta_pinned, P.meta_host.size(), hipMemcpyHostToDevice, (hipStream_t)stream) !=
      hipSuccess) {
    (void)hipGetLastError();
    return set_error(PA_ERR_DEVICE, "metadata upload failed");
  }
  meta_registry_set(meta_dev, P.serial);
  return PA_OK;
}

extern "C" void pa_plan_free(pa_plan_t* plan) {
  if (plan && plan->plan.meta_pinned) (void)hipHostFree(plan->plan.meta_pinned);
  delete plan;
}

extern "C" const char* pa_last_error(void) { return g_last_error.c_str(); }
