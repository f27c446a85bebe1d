// mhc_pre_noalloc: hc_pre for callers that cannot allocate device memory.
// The workspace mhc_pre takes from its caller (packed φ, exchange records,
// ticket counter) lives here in a static device buffer instead, one per GPU
// the library runs on, held until the process ends.  Nothing in it needs
// clearing between calls: the split-K kernels tag their records per call and
// take their tickets modulo the grid, whatever the buffer holds.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "mhc.h"
#include "mhc_internal.h"

namespace {

static_assert(MHC_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch size keeps the 256-byte alignment");
static __device__ __align__(256) unsigned char scratch[MHC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch buffer, looked up once per
// device (with that device current) and kept.  The name `scratch` itself is a
// host-side stand-in and is never passed to a kernel.
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" mhc_status mhc_pre_noalloc(const mhc_desc* d, const void* x, const float* phi, const float* bias,
                                      void* h, float* H_pre, float* H_post, float* H_res, hipStream_t stream) {
  // mhc_pre_workspace_bytes is 0 for an invalid descriptor; mhc_pre reports that
  const size_t need = mhc_pre_workspace_bytes(d);
  if (need > (size_t)MHC_NOALLOC_SCRATCH_BYTES) return MHC_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (scratch_of_current_device(&ws) != hipSuccess) return MHC_ERR_HIP;
  return mhc_pre(d, x, phi, bias, h, H_pre, H_post, H_res, ws, (size_t)MHC_NOALLOC_SCRATCH_BYTES, stream);
}
