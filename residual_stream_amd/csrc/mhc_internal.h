// Host-side launchers behind the C ABI (one per kernel family).  Each returns
// the HIP error of its last launch; arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "mhc.h"

namespace mhc {

// Kernel-level tracing (mhc_trace_kernel_events): per host thread, an array of
// caller-owned event pairs recorded around each launch, with the kernels'
// names.  Off (events == nullptr) unless a caller turns it on.
struct KernelTrace {
  hipEvent_t* events = nullptr;
  const char** names = nullptr;
  int capacity = 0;
  int* count = nullptr;
  int n = 0;
};
extern thread_local KernelTrace g_kernel_trace;

inline void trace_before(hipStream_t s) {
  KernelTrace& t = g_kernel_trace;
  if (t.events != nullptr && t.n < t.capacity) (void)hipEventRecord(t.events[2 * t.n], s);
}
inline void trace_after(hipStream_t s, const char* name) {
  KernelTrace& t = g_kernel_trace;
  if (t.events == nullptr || t.n >= t.capacity) return;
  (void)hipEventRecord(t.events[2 * t.n + 1], s);
  if (t.names != nullptr) t.names[t.n] = name;
  ++t.n;
  if (t.count != nullptr) *t.count = t.n;
}

// Every kernel of the library is launched through this: hipLaunchKernelGGL
// with the tracing hooks around it.  Arguments as for hipLaunchKernelGGL
// (kernel, grid, block, shared bytes, stream, kernel arguments...).
#define MHC_STREAM_OF_(grid, block, shmem, stream, ...) stream
#define MHC_LAUNCH(kernel, ...)                                   \
  do {                                                            \
    ::mhc::trace_before(MHC_STREAM_OF_(__VA_ARGS__));             \
    hipLaunchKernelGGL(kernel, __VA_ARGS__);                      \
    ::mhc::trace_after(MHC_STREAM_OF_(__VA_ARGS__), #kernel);     \
  } while (0)

// Compute units of the current device (cached per device; a property query,
// not mutable state).
int device_cu_count();
int occupancy_per_cu(const void* kernel, int threads, size_t lds);

// Seed of the exchange-record tags of the split-K hc_pre, drawn once per
// process (each call adds a per-device call number on the device).
uint32_t process_tag_seed();

// hc_pre with whole token tiles held on chip, the reduction split over groups
// of four workgroups (bf16, N = 4, D = 5120 or 2560); φ packed into the
// workspace as bf16 high and low parts first.
// n floats set to zero on the stream (a kernel, not a memset).
hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
bool pre_tile_eligible(const mhc_desc& d);
// Test hook behind mhc_test_exchange_fault: workgroup `drop_slice` of every
// group publishes nothing and record waits give up after spin_limit polls
// (drop_slice = -1: off).
void set_exchange_fault(int drop_slice, uint32_t spin_limit);
size_t pre_tile_workspace_bytes(const mhc_desc& d);
hipError_t launch_pre_tile(const mhc_desc& d, const void* x, const float* phi, const float* bias, void* h,
                           float* H_pre, float* H_post, float* H_res, void* ws, hipStream_t s);

size_t pre_workspace_bytes(const mhc_desc& d);
size_t post_pre_workspace_bytes(const mhc_desc& d);
hipError_t launch_pre(const mhc_desc& d, const void* x, const float* phi, const float* bias,
                      void* h, float* H_pre, float* H_post, float* H_res, void* ws,
                      hipStream_t s);

// few-token (decode-sized) hc_pre: k split across the chip, two launches
constexpr int64_t kDecodeMaxT = 64;
bool pre_decode_eligible(const mhc_desc& d);
size_t pre_decode_workspace_bytes(const mhc_desc& d);
hipError_t launch_pre_decode(const mhc_desc& d, const void* x, const float* phi, const float* bias,
                             void* h, float* H_pre, float* H_post, float* H_res, void* ws,
                             hipStream_t s);

// hc_post then hc_pre on its output (the two kernels, one after the other)
hipError_t launch_post_pre(const mhc_desc& d, const void* x, const void* y, const float* H_post_in,
                           const float* H_res_in, void* x_next, const float* phi, const float* bias,
                           void* h, float* H_pre, float* H_post, float* H_res, void* ws, hipStream_t s);
hipError_t launch_post(const mhc_desc& d, const void* x, const void* y, const float* H_post,
                       const float* H_res, void* x_next, hipStream_t s,
                       bool keep_out = false);

hipError_t launch_post_bwd(const mhc_desc& d, const void* dxn, const void* x, const void* y,
                           const float* H_post, const float* H_res, void* dx, void* dy,
                           float* dH_post, float* dH_res, hipStream_t s);

// openPangu's stabilised write-back (sandwich norm of y with weight wy, block
// post-norm of the state with weight wx; a null weight turns its norm off)
bool post_stable_supported(const mhc_desc& d);
size_t post_stable_bwd_workspace_bytes(const mhc_desc& d, bool sw, bool pn);
hipError_t launch_post_stable(const mhc_desc& d, const void* x, const void* y, const float* wy,
                              const float* H_post, const float* H_res, const float* wx, void* x_next,
                              hipStream_t s);
hipError_t launch_post_stable_bwd(const mhc_desc& d, const void* dxn, const void* x, const void* y,
                                  const float* wy, const float* H_post, const float* H_res,
                                  const float* wx, void* dx, void* dy, float* dwy, float* dwx,
                                  float* dH_post, float* dH_res, void* ws, hipStream_t s);

size_t pre_bwd_workspace_bytes(const mhc_desc& d);

// Matrix-core backward of hc_pre (bf16, N = 4, D % 256 == 0); leaves the
// per-token dℓ and dα terms in the workspace for the shared bias/α reduction.
bool pre_bwd_mfma_eligible(const mhc_desc& d);
size_t pre_bwd_mfma_workspace_bytes(const mhc_desc& d);
// With dxn and H_res non-null (bf16 only) the dx pass writes
// dx = H_resᵀ·dx_next + the hc_pre part instead of accumulating into dx.
hipError_t launch_pre_bwd_mfma(const mhc_desc& d, const void* dh, const void* x, const float* phi,
                               const float* bias, const float* dH_post, const float* dH_res,
                               void* dx, float* dphi, float* dbias, float* dalpha, void* ws,
                               hipStream_t s, const void* dxn, const float* H_res);
hipError_t launch_pre_bwd(const mhc_desc& d, const void* dh, const void* x, const float* phi,
                          const float* bias, const float* dH_post, const float* dH_res, void* dx,
                          float* dphi, float* dbias, float* dalpha, void* ws, hipStream_t s);
hipError_t launch_pre_bwd_mix(const mhc_desc& d, const void* dh, const void* x, const float* phi,
                              const float* bias, const float* dH_post, const float* dH_res,
                              const void* dxn, const float* H_res, void* dx, float* dphi, float* dbias,
                              float* dalpha, void* ws, hipStream_t s);

}  // namespace mhc
