// kda_noalloc.hip -- kda_fwd for callers that cannot allocate device memory.
//
// The forward's workspace (chunk map, per chunk-head operand blocks, stretch
// buffers of the segment scan) comes from `scratch`, a file-scope device array
// of KDA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the device address is looked up once per device with
// hipGetSymbolAddress and only that pointer is ever handed to kernels.
//
// Nothing in the forward's workspace has to start at zero: every region is
// written before it is read within one call.  Calls on one GPU share the array,
// so calls that overlap on one GPU (different streams or host threads without
// ordering) race on it.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kda.h"
#include "kda_internal.hpp"

namespace {

static __device__ __align__(256) char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// Device address of this device's copy of `scratch` (looked up on first use).
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_fwd_noalloc(const kda_desc* desc, const void* q, const void* k, const void* v,
                                      const void* log_alpha, const void* beta, const float* init_state,
                                      void* out, float* final_state, const int32_t* cu_seqlens, void* stream) {
  kda::set_error("");
  if (desc && (desc->flags & KDA_FLAG_SAVE_FOR_BACKWARD)) return KDA_ERROR_INVALID_VALUE;   // nothing to keep
  void* ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) {
    char msg[160];
    std::snprintf(msg, sizeof msg, "kda_fwd_noalloc: scratch lookup failed: %s", hipGetErrorString(e));
    kda::set_error(msg);
    return KDA_ERROR_LAUNCH;
  }
  size_t need = 0;
  const kda_status s = kda::fwd_checked(desc, q, k, v, log_alpha, beta, init_state, out, final_state, cu_seqlens,
                                        ws, (size_t)KDA_NOALLOC_SCRATCH_BYTES, stream, &need);
  if (s == KDA_ERROR_WORKSPACE_TOO_SMALL) {
    char msg[200];
    std::snprintf(msg, sizeof msg, "kda_fwd_noalloc: the problem needs %zu bytes of scratch, the library holds %zu",
                  need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
    kda::set_error(msg);
  }
  return s;
}
