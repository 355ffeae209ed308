// Read-only bandwidth probes for the decode's KV access patterns (a
// measurement tool built into its own library, libpa_ceiling.so; the decode
// library does not contain or call it).
//
// Each probe reads exactly the bytes one decode launch reads for a plan's
// work list (FP8 caches, head dim 128, 128-token pages, plain V, per-token
// scales, no window: one page per tile, so every table index it reads lies
// inside the sequence's extent) and folds them into one word per thread, so
// its time is what the memory system gives for that access pattern with no
// attention arithmetic:
//   mode 0  the streaming decode kernel's pattern: 4 waves, wave w takes the
//           32-token step w of every 128-token tile, 16-byte loads straight
//           into registers, three steps in flight per wave;
//   mode 1  an LDS ring: the workgroup copies each tile (K, V, scales) into
//           one of three LDS stages with global_load_lds_dwordx4, waits for
//           the oldest stage, reads it back from LDS;
//   mode 2  mode 0 with V read as whole 128-byte rows: the same bytes per
//           tile and per wave, but each V load instruction covers 8 full
//           rows of the page instead of a 32-byte piece of 32 rows (in mode 0
//           the four waves each read a quarter of every V row);
// and pa_ceiling_read streams a contiguous buffer (the plain-read rate).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct ProbeArgs {
  const uint8_t* k_cache;
  const uint8_t* v_cache;
  const float* k_scale;
  const float* v_scale;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* items;  // the plan's work list: 8 int32 per item
  uint32_t* out;         // one word per thread of the grid
  long long page_stride, head_stride;
  int Hkv, page_size, table_stride;
};

constexpr int TT = 128;  // tokens per tile

struct Item {
  int seq, kvh, tb, te;
};

__device__ Item item_of(const ProbeArgs& a) {
  const int32_t* it = a.items + 8 * blockIdx.x;
  Item r{it[0], it[1], it[3], it[4]};
  if (r.seq < 0) return Item{-1, 0, 0, 0};
  const long cap = (long)a.table_stride * a.page_size;
  const long L = min(max((long)a.context_lens[r.seq], 0L), cap);
  const int ntiles = (int)((L + TT - 1) / TT);
  r.tb = min(r.tb, ntiles);
  r.te = r.te < 0 ? ntiles : min(r.te, ntiles);
  return r;
}

struct Step {
  u32x4 k[4], v[4];
  float sc;
};

template <bool FULL_ROWS>
__global__ __launch_bounds__(256) void probe_registers(ProbeArgs a) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, c32 = lane & 31, h = lane >> 5;
  const Item it = item_of(a);
  uint32_t acc = 0;
  if (it.seq >= 0 && it.tb < it.te) {
    const int ps = a.page_size, ppt = TT / ps;
    const int32_t* bt = a.block_tables + (long)it.seq * a.table_stride;
    const uint8_t* kb = a.k_cache + (long long)it.kvh * a.head_stride;
    const uint8_t* vb = a.v_cache + (long long)it.kvh * a.head_stride;
    const float* sb = h ? a.v_scale : a.k_scale;
    const int kt = ((c32 >> 2) & 1) * 16 + (c32 >> 3) * 4 + (c32 & 3);
    const uint32_t kcs = (uint32_t)ps * 16;
    auto load = [&](Step& s, int k) {
      k = min(k, it.te - 1);
      const int j = k * ppt + ((32 * w) / ps);  // the step's page (a step lies in one page)
      const long pid = bt[j];
      const int slot = (32 * w) & (ps - 1);
      const uint8_t* kp = kb + pid * a.page_stride + (2 * h * ps + slot + kt) * 16;
      s.k[0] = *(const u32x4*)kp;
      s.k[1] = *(const u32x4*)(kp + kcs);
      s.k[2] = *(const u32x4*)(kp + 4 * kcs);
      s.k[3] = *(const u32x4*)(kp + 5 * kcs);
      const uint8_t* vp = vb + pid * a.page_stride + slot + 16 * h;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        if (FULL_ROWS)  // rows 32w + 8db .. +7 of the page, 16 bytes per lane
          s.v[db] = *(const u32x4*)(vb + pid * a.page_stride + (32 * w + 8 * db + (lane >> 3)) * ps + 16 * (lane & 7));
        else
          s.v[db] = *(const u32x4*)(vp + (32 * db + c32) * ps);
      }
      s.sc = sb[(pid * a.Hkv + it.kvh) * ps + slot + c32];
    };
    auto use = [&](const Step& s) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc ^= s.k[i][0] ^ s.k[i][1] ^ s.k[i][2] ^ s.k[i][3] ^ s.v[i][0] ^ s.v[i][1] ^ s.v[i][2] ^ s.v[i][3];
      acc += __float_as_uint(s.sc);
    };
    Step b0, b1, b2;
    load(b0, it.tb);
    load(b1, it.tb + 1);
    load(b2, it.tb + 2);
    for (int k = it.tb; k < it.te; k += 3) {
      use(b0);
      load(b0, k + 3);
      if (k + 1 < it.te) use(b1);
      load(b1, k + 4);
      if (k + 2 < it.te) use(b2);
      load(b2, k + 5);
    }
  }
  a.out[blockIdx.x * 256 + tid] = acc;
}

// LDS ring: K (16 KB), V (16 KB) and the two scale rows (1 KB) of a tile per
// stage, three stages.
constexpr int KB = TT * 128, VB = TT * 128, SB = 2 * TT * 4;
constexpr int STAGE = KB + VB + SB;
constexpr int NSTAGE = 3;

__device__ __forceinline__ void wait_vm(int n) {
  // vmcnt(n) for n in {0, 9, 18} (the loads of 0, 1 or 2 later tiles in flight)
  if (n >= 18)
    __builtin_amdgcn_s_waitcnt((18 & 0xF) | ((18 >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  else if (n >= 9)
    __builtin_amdgcn_s_waitcnt((9 & 0xF) | ((9 >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  else
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
}

__global__ __launch_bounds__(256) void probe_lds(ProbeArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const Item it = item_of(a);
  uint32_t acc = 0;
  if (it.seq >= 0 && it.tb < it.te) {
    const int ps = a.page_size, ppt = TT / ps;
    const int32_t* bt = a.block_tables + (long)it.seq * a.table_stride;
    const uint8_t* kb = a.k_cache + (long long)it.kvh * a.head_stride;
    const uint8_t* vb = a.v_cache + (long long)it.kvh * a.head_stride;
    // every thread issues 4 K + 4 V units (16 bytes each) and one scale unit
    // per tile: 9 loads, so a constant vmcnt tracks the tiles in flight
    auto issue = [&](int tile, int stage) {
      uint8_t* st = smem + stage * STAGE;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u;          // 16-byte unit of the tile's K (or V) bytes
        const int byte = e * 16;              // offset inside the tile's K block
        const int page_in_tile = byte / (ps * 128);
        const long pid = bt[tile * ppt + page_in_tile];
        const int off = byte % (ps * 128);
        __builtin_amdgcn_global_load_lds((const void*)(kb + pid * a.page_stride + off),
                                         (lds_void*)(st + (tid - lane) * 16 + u * 4096), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(vb + pid * a.page_stride + off),
                                         (lds_void*)(st + KB + (tid - lane) * 16 + u * 4096), 16, 0, 0);
      }
      {
        const int half = tid >> 7;  // threads 0-127: k scales, 128-255: v scales (4 bytes each)
        const int t = tid & 127;
        const int page_in_tile = t / ps;
        const long pid = bt[tile * ppt + page_in_tile];
        const float* src = (half ? a.v_scale : a.k_scale) + (pid * a.Hkv + it.kvh) * ps + t % ps;
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(st + KB + VB + (tid - lane) * 4), 4, 0, 0);
      }
    };
    for (int k = 0; k < NSTAGE - 1; ++k)
      if (it.tb + k < it.te) issue(it.tb + k, k);
    for (int tile = it.tb; tile < it.te; ++tile) {
      const int ahead = min(it.te - 1 - tile, NSTAGE - 2);  // tiles issued after this one
      wait_vm(9 * ahead);
      __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (tile + NSTAGE - 1 < it.te) issue(tile + NSTAGE - 1, (tile - it.tb + NSTAGE - 1) % NSTAGE);
      const uint8_t* st = smem + ((tile - it.tb) % NSTAGE) * STAGE;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const u32x4 x = *(const u32x4*)(st + (tid + 256 * u) * 16);
        acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
      }
      acc += *(const uint32_t*)(st + KB + VB + tid * 4);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();  // the stage is read before it is refilled
      asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
  }
  a.out[blockIdx.x * 256 + tid] = acc;
}

__global__ __launch_bounds__(256) void probe_read(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 x = p[i], y = p[i + stride], z = p[i + 2 * stride], q = p[i + 3 * stride];
    acc ^= x[0] ^ x[3] ^ y[1] ^ y[2] ^ z[0] ^ z[1] ^ q[2] ^ q[3];
  }
  for (; i < n16; i += stride) acc ^= p[i][0];
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// Returns 0 on success, 1 for an unsupported layout, 2 for a launch error.
extern "C" int pa_ceiling_gather(int mode, const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* block_tables, const int32_t* context_lens,
                                 const int32_t* items, int num_items, uint32_t* out, int num_kv_heads, int page_size,
                                 int table_stride, void* stream) {
  if (page_size != TT || num_items <= 0) return 1;
  ProbeArgs a;
  a.k_cache = (const uint8_t*)k_cache;
  a.v_cache = (const uint8_t*)v_cache;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.items = items;
  a.out = out;
  a.head_stride = 128LL * page_size;
  a.page_stride = a.head_stride * num_kv_heads;
  a.Hkv = num_kv_heads;
  a.page_size = page_size;
  a.table_stride = table_stride;
  if (mode == 0) {
    hipLaunchKernelGGL(probe_registers<false>, dim3(num_items), dim3(256), 0, (hipStream_t)stream, a);
  } else if (mode == 2) {
    hipLaunchKernelGGL(probe_registers<true>, dim3(num_items), dim3(256), 0, (hipStream_t)stream, a);
  } else if (mode == 1) {
    static bool configured = false;
    if (!configured) {
      if (hipFuncSetAttribute((const void*)probe_lds, hipFuncAttributeMaxDynamicSharedMemorySize,
                              NSTAGE * STAGE) != hipSuccess)
        return 2;
      configured = true;
    }
    hipLaunchKernelGGL(probe_lds, dim3(num_items), dim3(256), NSTAGE * STAGE, (hipStream_t)stream, a);
  } else {
    return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int pa_ceiling_read(const void* buf, size_t bytes, uint32_t* out, int grid, void* stream) {
  if (grid <= 0 || (bytes & 15)) return 1;
  hipLaunchKernelGGL(probe_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)buf, bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
