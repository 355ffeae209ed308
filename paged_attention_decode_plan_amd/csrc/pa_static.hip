// pa_attend_static: pa_decode + pa_reduce with the plan metadata and the
// partial states in a fixed device array of this library, for callers that
// cannot allocate device memory.
//
// The array `scratch` is a file-scope __device__ variable: each GPU the
// library runs on holds its own copy (PA_STATIC_SCRATCH_BYTES) until the
// process ends.  In host code its name is only a stand-in for the symbol, so
// its device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and that pointer is what the kernels receive.
// Every call on one GPU shares the array: calls that overlap on one GPU race.
// Nothing in it needs clearing between calls: the metadata is copied in
// whole whenever the array does not already hold the calling plan's, and
// every partial slot the reducer reads is written by the same call's decode.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "pa_internal.h"

static __device__ __align__(256) uint8_t scratch[PA_STATIC_SCRATCH_BYTES];

namespace pa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up on first use).
pa_status scratch_of_current_device(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return set_error(PA_ERR_DEVICE, "no current HIP device");
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "hipGetSymbolAddress of the static scratch array failed");
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = (uint8_t*)g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status pa_attend_static(const pa_plan_t* plan, void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                      const float* k_scale, const float* v_scale, const float* sinks, void* stream) {
  if (!plan) return set_error(PA_ERR_INVALID, "plan is NULL");
  const Plan& P = plan->plan;
  const size_t meta_span = (P.meta_bytes() + 255) & ~(size_t)255;  // partials start 256-byte aligned
  const size_t need = meta_span + P.workspace_bytes();
  if (need > (size_t)PA_STATIC_SCRATCH_BYTES)
    return set_error(PA_ERR_WORKSPACE, "plan needs " + std::to_string(need) + " bytes of metadata and partials; the "
                                           "static scratch array holds " +
                                           std::to_string((size_t)PA_STATIC_SCRATCH_BYTES));
  uint8_t* base = nullptr;
  pa_status st = scratch_of_current_device(&base);
  if (st != PA_OK) return st;
  uint8_t* meta = base;
  uint8_t* ws = base + meta_span;
  if (!meta_registry_holds(meta, P.serial)) {
    // from the plan's pinned copy if an upload made one, else from its host
    // vector: no allocation either way
    const void* src = P.meta_pinned ? (const void*)P.meta_pinned : (const void*)P.meta_host.data();
    if (hipMemcpyAsync(meta, src, P.meta_bytes(), hipMemcpyHostToDevice, (hipStream_t)stream) != hipSuccess) {
      (void)hipGetLastError();
      return set_error(PA_ERR_DEVICE, "metadata copy into the static scratch array failed");
    }
    meta_registry_set(meta, P.serial);
  }
  st = pa_decode(plan, out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, sinks, meta, ws, stream);
  if (st != PA_OK) return st;
  return pa_reduce(plan, out, sinks, meta, ws, stream);
}
