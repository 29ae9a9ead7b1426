// sage_noalloc.hip -- sage_attn_fwd for callers that cannot allocate device
// memory: the workspace is a fixed array in the library's own device memory.
//
// `scratch` below is a file-scope device array.  Its name in host code is a
// host-side stand-in, not a device address, so the address every device sees
// is taken once per device with hipGetSymbolAddress (on the first call on
// that device, with the device current) and only that pointer is handed to
// the kernels.  Each device holds its own copy for the life of the process.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sage_attn.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // SAGE_NOALLOC_MAX_WORKSPACE
static_assert(kScratchBytes == SAGE_NOALLOC_MAX_WORKSPACE, "header and source agree");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` on each device (null: not yet taken)

// The address of this device's copy of `scratch`, or null on a HIP error.
void* scratch_on(int dev) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" {

int sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H,
                          int N, int d, int causal, int pv_mode, int dtype, void* stream) {
  // The shape and mode, then the fixed size; sage_attn_fwd validates the rest
  // (pointers, flags, dtype) before it enqueues anything.
  if (pv_mode != SAGE_PV_FP16 && pv_mode != SAGE_PV_FP8 && pv_mode != SAGE_PV_INT8)
    return SAGE_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return SAGE_ERR_INVALID_ARG;
  const size_t need = sage_attn_workspace_bytes(B, H, N, d, pv_mode);
  if (need == 0) return SAGE_ERR_UNSUPPORTED;          // d, or N beyond 2^24
  if (need > kScratchBytes) return SAGE_ERR_WORKSPACE;  // beyond the fixed array
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
    (void)hipGetLastError();
    return SAGE_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_UNSUPPORTED;
  void* ws = scratch_on(dev);
  if (!ws) return SAGE_ERR_HIP;
  return sage_attn_fwd(q, k, v, o, B, H, N, d, causal, pv_mode, dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
