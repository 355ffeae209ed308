// Device-side definitions shared by the decode kernels: vector types, launch
// arguments, numeric constants and wave-level helpers for gfx950.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "pa_internal.h"

namespace pa {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float TAU = 12.0f;     // probabilities are taken against a reference max: p <= 2^12
constexpr float VS_BAND = 8.0f;  // per-token V scales against a reference: vs/ref <= 8
constexpr float LOG2E = 1.4426950408889634f;
constexpr float FP8_MAX = 448.0f;  // largest finite e4m3fn value

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
  const int32_t* topk;  // top-k logical positions (two-level sparse rows), else NULL
  const WorkItem* items;
  const MetaHeader* meta;  // header of the metadata buffer (items follow it)
  uint32_t tag_lo, tag_hi;  // the launching plan's serial: the header must hold it
  float* workspace;
  int* merge_ctr;  // arrival counters of the in-kernel merge, else NULL (the reducer merges)
  long long page_stride;  // bytes between physical pages (Hkv * D * page * elem)
  long long head_stride;  // bytes between KV heads of a page (D * page * elem)
  // page_size: the page size the kernels index tokens by.  Pages above 128
  // tokens are taken as 2^page_sub sub-pages of 128 (dense caches): a
  // sub-page id is (block-table entry << page_sub) | sub-page, and strides
  // inside a page use the physical size phys_page.
  int QL, Hq, Hkv, G, page_size, page_sub, phys_page, table_stride, window, causal;
  int v_transposed, scale_mode, q_fp16, has_sinks, rows_total, rows_per_group, stage_limit, index_stride;
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
// x of another lane of the 16-lane row (DPP control CTRL: quad permutes, mirrors)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// max / sum over the whole wave, in registers (butterflies: quad lane ^1 and
// ^2, half-row and row mirrors, then the 16- and 32-lane swaps); every lane
// gets the same result
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return fmax_swap32(fmax_swap16(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return fadd_swap32(fadd_swap16(x));
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
// spreads the QK operand reads of one lane group over more bank quads; it is
// its own inverse.
__device__ __forceinline__ int kswz(int t) { return t ^ (((t >> 3) & 1) << 2); }

// Whether the metadata buffer holds the launching plan's list (its header
// carries the plan's serial); loaded together with the work item.
__device__ __forceinline__ bool meta_ok(const MetaHeader& h, uint32_t lo, uint32_t hi) {
  return h.magic == kMetaMagic && h.serial_lo == lo && h.serial_hi == hi;
}

// s_waitcnt with only the vector-memory count constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// s_waitcnt lgkmcnt(0) with the other counters unconstrained.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Streaming kernel for FP8 caches, head dim 128, page tables and 17..64-row
// work items.
bool stream_kernel_applies(const Plan& P);
pa_status launch_stream(const Plan& P, const KernelArgs& args, int nblocks, hipStream_t stream);

}  // namespace pa
