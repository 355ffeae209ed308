// Internal plan representation shared by the host planner and the launch code.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "pa_decode.h"

namespace pa {

constexpr int kTileTokens = 128;   // tokens per pipeline tile (a multiple of every page size)
constexpr int kMaxRowsPerItem = 64; // query rows one work item carries (4 row tiles of 16)
constexpr int kStageCap = 1024;     // page / slot ids staged in LDS per work item
constexpr int kMaxPartitions = 256; // static per-(sequence, KV head) bound

// One workgroup's work: 8 int32, uploaded verbatim.
struct WorkItem {
  int32_t seq, kvh, rg;           // sequence, KV head, row group
  int32_t tile_begin, tile_end;   // tiles relative to the page-aligned span start; -1: to the end
  // (seq -1: an unused item of a refreshable plan, which does nothing)
  int32_t slot;                   // partial slot; -1: direct output
  int32_t part, nparts;
};
static_assert(sizeof(WorkItem) == 32, "work item is 32 bytes");

// One multi-partition (sequence, KV head, row group): its partials occupy
// slots [first_slot, first_slot + nparts) in partition order.  nparts < 2:
// nothing to merge (refreshable plans keep one entry per unit).
struct ReduceItem {
  int32_t seq, kvh, rg, first_slot, nparts, pad0, pad1, pad2;
};
static_assert(sizeof(ReduceItem) == 32, "reduce item is 32 bytes");

// First 32 bytes of meta_dev: which plan's list the buffer holds.  Every
// kernel compares it with the plan it was launched for and does nothing on
// a mismatch (a buffer reallocated or overwritten since its upload), so a
// foreign list can never steer its indices.
constexpr uint32_t kMetaMagic = 0x314D4150u;  // "PAM1"
struct MetaHeader {
  uint32_t magic, serial_lo, serial_hi, n_items, n_reduce, pad0, pad1, pad2;
};
static_assert(sizeof(MetaHeader) == 32, "metadata header is 32 bytes");

// Layout of meta_dev: [MetaHeader][WorkItem x num_items][ReduceItem x num_reduce]
// and, for the in-kernel merge, 128-byte aligned arrival counters: one
// 128-byte line per partial slot (a unit's counter sits at its first slot).
struct Plan {
  pa_problem prob;
  pa_plan_opts opts;
  int cu_count = 0;
  int rows_total = 0;      // QL * G
  int rows_per_group = 0;  // min(64, rows_total)
  int row_groups = 0;
  int nrt = 0;             // 16-row tiles per work item (1, 2 or 4)
  int stage_limit = kStageCap;
  int max_parts = 0;
  int total_tiles = 0;
  float scale_log2 = 0.f;  // softmax_scale * log2(e)
  int maxp = 0;            // partition cap per unit (refreshable plans)
  int budget_items = 0;    // fixed item count of a refreshable plan (0: not refreshable)
  std::vector<WorkItem> items;
  std::vector<ReduceItem> reduce;
  int num_slots = 0;
  bool in_kernel_merge = false;     // last-arriver merge in the decode launch (no reducer launch)
  uint64_t serial = 0;              // unique per plan in the process
  std::vector<uint8_t> meta_host;   // serialised metadata (header, items, reduce table)
  mutable uint8_t* meta_pinned = nullptr;  // pinned copy of meta_host, made by the first upload

  size_t meta_bytes() const { return meta_host.size(); }
  static constexpr size_t items_offset() { return sizeof(MetaHeader); }
  size_t reduce_offset() const { return sizeof(MetaHeader) + items.size() * sizeof(WorkItem); }
  size_t counters_offset() const { return (reduce_offset() + reduce.size() * sizeof(ReduceItem) + 127) & ~(size_t)127; }
  static constexpr size_t kCounterBytes = 128;  // one line per counter
  // partial state per slot: m[rows_per_group], l[rows_per_group], o[rows_per_group][D]
  size_t slot_floats() const { return (size_t)rows_per_group * (2 + prob.head_dim); }
  size_t workspace_bytes() const { return (size_t)num_slots * slot_floats() * sizeof(float); }
};

// thread-local error message helper (defined in pa_plan.cpp)
pa_status set_error(pa_status st, const std::string& msg);
pa_status validate_problem(const pa_problem* p);

// Which plan's metadata each device buffer holds (process-wide; set by
// pa_plan_upload and pa_plan_refresh, checked by pa_decode and pa_reduce).
void meta_registry_set(const void* meta_dev, uint64_t serial);
bool meta_registry_holds(const void* meta_dev, uint64_t serial);

}  // namespace pa

struct pa_plan_s {
  pa::Plan plan;
};
