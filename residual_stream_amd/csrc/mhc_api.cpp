// C ABI of the mHC hot path (declared in include/mhc.h): argument validation
// and dispatch to the gfx950 kernels.  No allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <limits>
#include <mutex>

#include "mhc.h"
#include "mhc_internal.h"

namespace mhc {

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Resident workgroups per CU of a kernel at a block size and dynamic LDS, from
// the runtime's occupancy query, kept per device in a fixed table (the query
// otherwise costs host time on every call); at least 1.
int occupancy_per_cu(const void* kernel, int threads, size_t lds) {
  struct Entry {
    int dev;
    const void* kernel;
    int threads;
    size_t lds;
    int per_cu;
  };
  constexpr int kSlots = 64;
  static Entry table[kSlots];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (table[i].dev == dev && table[i].kernel == kernel && table[i].threads == threads && table[i].lds == lds)
        return table[i].per_cu;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1) n = 1;
  std::lock_guard<std::mutex> lock(mu);
  if (used < kSlots) table[used++] = Entry{dev, kernel, threads, lds, n};
  return n;
}

thread_local KernelTrace g_kernel_trace;

// Seed of the split-K exchange tags: the device adds each call's number to
// it, and sets the top bit so that zeroed memory never matches.  Drawn from
// the clock once per load of the library, so that a reloaded library (whose
// device counters start again at zero) most likely tags differently.
uint32_t process_tag_seed() {
  static const uint32_t seed =
      (uint32_t)((uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u);
  return seed;
}

}  // namespace mhc

namespace {

constexpr int kMaxIters = 100000;
constexpr int kMaxBwdIters = 64;

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool finite(float v) { return std::isfinite(v); }

// Shape and scalar checks common to every call.
mhc_status check_desc(const mhc_desc* d) {
  if (d == nullptr) return MHC_ERR_INVALID_ARG;
  if (d->T < 0 || d->T > std::numeric_limits<int32_t>::max()) return MHC_ERR_INVALID_ARG;
  if (d->io != MHC_F32 && d->io != MHC_BF16) return MHC_ERR_INVALID_ARG;
  if (d->sinkhorn_iters < 1) return MHC_ERR_INVALID_ARG;
  if (!finite(d->eps) || d->eps < 0.f) return MHC_ERR_INVALID_ARG;
  if (d->alpha == nullptr && (!finite(d->alpha_pre) || !finite(d->alpha_post) || !finite(d->alpha_res)))
    return MHC_ERR_INVALID_ARG;
  if (d->alpha != nullptr && (reinterpret_cast<uintptr_t>(d->alpha) & 3u) != 0) return MHC_ERR_INVALID_ARG;
  if (d->N != 1 && d->N != 2 && d->N != 4 && d->N != 8) return MHC_ERR_UNSUPPORTED;
  if (d->D < 8 || d->D % 8 != 0 || d->D > (1 << 24)) return MHC_ERR_UNSUPPORTED;
  if (d->sinkhorn_iters > kMaxIters) return MHC_ERR_UNSUPPORTED;
  return MHC_OK;
}

size_t io_bytes(const mhc_desc* d) { return d->io == MHC_F32 ? 4 : 2; }

// True if the byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

bool workspace_ok(const void* ws, size_t have, size_t need) {
  if (need == 0) return true;
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return false;
  return have >= need;
}

mhc_status from_hip(hipError_t e) { return e == hipSuccess ? MHC_OK : MHC_ERR_HIP; }

}  // namespace

extern "C" {

int mhc_abi_version(void) { return MHC_ABI_VERSION; }

mhc_status mhc_trace_kernel_events(hipEvent_t* events, const char** names, int capacity, int* count) {
  if (capacity < 0 || (events != nullptr && capacity == 0)) return MHC_ERR_INVALID_ARG;
  mhc::KernelTrace& t = mhc::g_kernel_trace;
  t.events = events;
  t.names = events != nullptr ? names : nullptr;
  t.capacity = events != nullptr ? capacity : 0;
  t.count = events != nullptr ? count : nullptr;
  t.n = 0;
  if (t.count != nullptr) *t.count = 0;
  return MHC_OK;
}

mhc_status mhc_test_exchange_fault(int drop_slice, unsigned spin_limit) {
  if (drop_slice < -1 || (drop_slice >= 0 && spin_limit == 0)) return MHC_ERR_INVALID_ARG;
  mhc::set_exchange_fault(drop_slice, spin_limit);
  return MHC_OK;
}

const char* mhc_status_string(mhc_status s) {
  switch (s) {
    case MHC_OK: return "ok";
    case MHC_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or scalar, workspace too small, aliasing)";
    case MHC_ERR_UNSUPPORTED: return "unsupported shape (N must be 1, 2, 4 or 8; D a multiple of 8; iteration limit)";
    case MHC_ERR_HIP: return "HIP runtime error while launching";
    case MHC_ERR_TOO_LARGE: return "the call needs more scratch than MHC_NOALLOC_SCRATCH_BYTES (use mhc_pre with a workspace)";
  }
  return "unknown status";
}

size_t mhc_pre_workspace_bytes(const mhc_desc* d) {
  if (check_desc(d) != MHC_OK || d->T == 0) return 0;
  return mhc::pre_workspace_bytes(*d);
}

size_t mhc_pre_bwd_workspace_bytes(const mhc_desc* d) {
  if (check_desc(d) != MHC_OK || d->T == 0) return 0;
  return mhc::pre_bwd_workspace_bytes(*d);
}

// An empty batch (T = 0): no token outputs, and the gradients of the
// parameters (sums over the tokens) are zero.  Their pointers must still be
// valid and aligned; the token tensors' pointers are not looked at.
static mhc_status zero_params(float* const* p, const size_t* n, int count, hipStream_t stream) {
  for (int i = 0; i < count; ++i) {
    if (p[i] == nullptr) continue;
    const hipError_t e = mhc::launch_fill_zero(p[i], n[i], stream);
    if (e != hipSuccess) return from_hip(e);
  }
  return MHC_OK;
}

mhc_status mhc_pre(const mhc_desc* d, const void* x, const float* phi, const float* bias, void* h,
                   float* H_pre, float* H_post, float* H_res, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  if (d->T == 0) return MHC_OK;
  if (!aligned16(x) || !aligned16(phi) || !aligned16(bias) || !aligned16(h) || !aligned16(H_pre) ||
      !aligned16(H_post) || !aligned16(H_res))
    return MHC_ERR_INVALID_ARG;
  const size_t T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  if (overlaps(h, T * D * io_bytes(d), x, T * N * D * io_bytes(d))) return MHC_ERR_INVALID_ARG;
  if (!workspace_ok(workspace, workspace_bytes, mhc::pre_workspace_bytes(*d)))
    return MHC_ERR_INVALID_ARG;
  return from_hip(mhc::launch_pre(*d, x, phi, bias, h, H_pre, H_post, H_res, workspace, stream));
}

mhc_status mhc_post(const mhc_desc* d, const void* x, const void* y, const float* H_post,
                    const float* H_res, void* x_next, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  if (d->T == 0) return MHC_OK;
  if (!aligned16(x) || !aligned16(y) || !aligned16(H_post) || !aligned16(H_res) ||
      !aligned16(x_next))
    return MHC_ERR_INVALID_ARG;
  const size_t b = io_bytes(d), T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  if (overlaps(x_next, T * N * D * b, x, T * N * D * b) || overlaps(x_next, T * N * D * b, y, T * D * b))
    return MHC_ERR_INVALID_ARG;
  return from_hip(mhc::launch_post(*d, x, y, H_post, H_res, x_next, stream));
}

mhc_status mhc_post_bwd(const mhc_desc* d, const void* dx_next, const void* x, const void* y,
                        const float* H_post, const float* H_res, void* dx, void* dy,
                        float* dH_post, float* dH_res, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  if (d->T == 0) return MHC_OK;
  // dx may be null: the caller then forms it in mhc_pre_bwd_mix
  if (!aligned16(dx_next) || !aligned16(x) || !aligned16(y) || !aligned16(H_post) ||
      !aligned16(H_res) || (dx != nullptr && !aligned16(dx)) || !aligned16(dy) || !aligned16(dH_post) ||
      !aligned16(dH_res))
    return MHC_ERR_INVALID_ARG;
  const size_t b = io_bytes(d), T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  const size_t big = T * N * D * b, small = T * D * b;
  if (dx != nullptr && (overlaps(dx, big, dx_next, big) || overlaps(dx, big, x, big) ||
                        overlaps(dx, big, y, small) || overlaps(dy, small, dx, big)))
    return MHC_ERR_INVALID_ARG;
  if (overlaps(dy, small, dx_next, big) || overlaps(dy, small, x, big)) return MHC_ERR_INVALID_ARG;
  return from_hip(
      mhc::launch_post_bwd(*d, dx_next, x, y, H_post, H_res, dx, dy, dH_post, dH_res, stream));
}

mhc_status mhc_pre_bwd(const mhc_desc* d, const void* dh, const void* x, const float* phi,
                       const float* bias, const float* dH_post, const float* dH_res, void* dx,
                       float* dphi, float* dbias, float* dalpha, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  if (d->sinkhorn_iters > kMaxBwdIters) return MHC_ERR_UNSUPPORTED;
  if (d->T == 0) {
    if (!aligned16(dphi) || !aligned16(dbias) || (dalpha != nullptr && (reinterpret_cast<uintptr_t>(dalpha) & 3u) != 0))
      return MHC_ERR_INVALID_ARG;
    const size_t C = (size_t)d->N * d->N + 2 * d->N;
    float* const p[3] = {dphi, dbias, dalpha};
    const size_t n[3] = {(size_t)d->N * d->D * C, C, 3};
    return zero_params(p, n, 3, stream);
  }
  if (!aligned16(dh) || !aligned16(x) || !aligned16(phi) || !aligned16(bias) ||
      !aligned16(dH_post) || !aligned16(dH_res) || !aligned16(dx) || !aligned16(dphi) ||
      !aligned16(dbias))
    return MHC_ERR_INVALID_ARG;
  if (dalpha != nullptr && (reinterpret_cast<uintptr_t>(dalpha) & 3u) != 0) return MHC_ERR_INVALID_ARG;
  const size_t b = io_bytes(d), T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  if (overlaps(dx, T * N * D * b, x, T * N * D * b) || overlaps(dx, T * N * D * b, dh, T * D * b))
    return MHC_ERR_INVALID_ARG;
  if (!workspace_ok(workspace, workspace_bytes, mhc::pre_bwd_workspace_bytes(*d)))
    return MHC_ERR_INVALID_ARG;
  return from_hip(mhc::launch_pre_bwd(*d, dh, x, phi, bias, dH_post, dH_res, dx, dphi, dbias,
                                      dalpha, workspace, stream));
}

mhc_status mhc_pre_bwd_mix(const mhc_desc* d, const void* dh, const void* x, const float* phi,
                           const float* bias, const float* dH_post, const float* dH_res,
                           const void* dx_next, const float* H_res, void* dx, float* dphi, float* dbias,
                           float* dalpha, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  if (d->sinkhorn_iters > kMaxBwdIters) return MHC_ERR_UNSUPPORTED;
  if (d->T == 0) {
    if (!aligned16(dphi) || !aligned16(dbias) || (dalpha != nullptr && (reinterpret_cast<uintptr_t>(dalpha) & 3u) != 0))
      return MHC_ERR_INVALID_ARG;
    const size_t C = (size_t)d->N * d->N + 2 * d->N;
    float* const p[3] = {dphi, dbias, dalpha};
    const size_t n[3] = {(size_t)d->N * d->D * C, C, 3};
    return zero_params(p, n, 3, stream);
  }
  if (!aligned16(dh) || !aligned16(x) || !aligned16(phi) || !aligned16(bias) ||
      !aligned16(dH_post) || !aligned16(dH_res) || !aligned16(dx_next) || !aligned16(H_res) ||
      !aligned16(dx) || !aligned16(dphi) || !aligned16(dbias))
    return MHC_ERR_INVALID_ARG;
  if (dalpha != nullptr && (reinterpret_cast<uintptr_t>(dalpha) & 3u) != 0) return MHC_ERR_INVALID_ARG;
  const size_t b = io_bytes(d), T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  const size_t big = T * N * D * b, small = T * D * b;
  // dx may be dx_next itself (updated in place), but not overlap it otherwise
  if (overlaps(dx, big, x, big) || overlaps(dx, big, dh, small) ||
      (dx != dx_next && overlaps(dx, big, dx_next, big)))
    return MHC_ERR_INVALID_ARG;
  if (!workspace_ok(workspace, workspace_bytes, mhc::pre_bwd_workspace_bytes(*d)))
    return MHC_ERR_INVALID_ARG;
  return from_hip(mhc::launch_pre_bwd_mix(*d, dh, x, phi, bias, dH_post, dH_res, dx_next, H_res, dx, dphi,
                                          dbias, dalpha, workspace, stream));
}

size_t mhc_post_pre_workspace_bytes(const mhc_desc* d) {
  if (check_desc(d) != MHC_OK || d->T == 0) return 0;
  return mhc::post_pre_workspace_bytes(*d);
}

mhc_status mhc_post_pre(const mhc_desc* d, const void* x, const void* y, const float* H_post_in,
                        const float* H_res_in, const float* phi, const float* bias, void* x_next,
                        void* h, float* H_pre, float* H_post, float* H_res, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  if (d->T == 0) return MHC_OK;
  if (!aligned16(x) || !aligned16(y) || !aligned16(H_post_in) || !aligned16(H_res_in) ||
      !aligned16(phi) || !aligned16(bias) || !aligned16(x_next) || !aligned16(h) ||
      !aligned16(H_pre) || !aligned16(H_post) || !aligned16(H_res))
    return MHC_ERR_INVALID_ARG;
  const size_t b = io_bytes(d), T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  const size_t big = T * N * D * b, small = T * D * b, cq = T * N * 4, cr = T * N * N * 4;
  if (overlaps(x_next, big, x, big) || overlaps(x_next, big, y, small) || overlaps(h, small, x_next, big) ||
      overlaps(h, small, x, big) || overlaps(h, small, y, small) || overlaps(H_post, cq, H_post_in, cq) ||
      overlaps(H_post, cq, H_res_in, cr) || overlaps(H_res, cr, H_post_in, cq) ||
      overlaps(H_res, cr, H_res_in, cr) || overlaps(H_pre, cq, H_post_in, cq) ||
      overlaps(H_pre, cq, H_res_in, cr))
    return MHC_ERR_INVALID_ARG;
  if (!workspace_ok(workspace, workspace_bytes, mhc::post_pre_workspace_bytes(*d)))
    return MHC_ERR_INVALID_ARG;
  return from_hip(mhc::launch_post_pre(*d, x, y, H_post_in, H_res_in, x_next, phi, bias, h, H_pre,
                                       H_post, H_res, workspace, stream));
}

size_t mhc_post_stable_bwd_workspace_bytes(const mhc_desc* d, int with_y_weight, int with_out_weight) {
  if (check_desc(d) != MHC_OK || d->T == 0) return 0;
  if (!with_y_weight && !with_out_weight) return 0;
  if (!mhc::post_stable_supported(*d)) return 0;
  return mhc::post_stable_bwd_workspace_bytes(*d, with_y_weight != 0, with_out_weight != 0);
}

mhc_status mhc_post_stable(const mhc_desc* d, const void* x, const void* y, const float* y_weight,
                           const float* H_post, const float* H_res, const float* out_weight,
                           void* x_next, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  if ((y_weight != nullptr || out_weight != nullptr) && !mhc::post_stable_supported(*d))
    return MHC_ERR_UNSUPPORTED;
  if (d->T == 0) return MHC_OK;
  if (!aligned16(x) || !aligned16(y) || !aligned16(H_post) || !aligned16(H_res) || !aligned16(x_next))
    return MHC_ERR_INVALID_ARG;
  if ((y_weight != nullptr && !aligned16(y_weight)) || (out_weight != nullptr && !aligned16(out_weight)))
    return MHC_ERR_INVALID_ARG;
  const size_t b = io_bytes(d), T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  const size_t big = T * N * D * b, small = T * D * b;
  if (overlaps(x_next, big, x, big) || overlaps(x_next, big, y, small) ||
      (y_weight != nullptr && overlaps(x_next, big, y_weight, D * 4)) ||
      (out_weight != nullptr && overlaps(x_next, big, out_weight, N * D * 4)))
    return MHC_ERR_INVALID_ARG;
  return from_hip(mhc::launch_post_stable(*d, x, y, y_weight, H_post, H_res, out_weight, x_next, stream));
}

mhc_status mhc_post_stable_bwd(const mhc_desc* d, const void* dx_next, const void* x, const void* y,
                               const float* y_weight, const float* H_post, const float* H_res,
                               const float* out_weight, void* dx, void* dy, float* dy_weight,
                               float* dout_weight, float* dH_post, float* dH_res, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  mhc_status st = check_desc(d);
  if (st != MHC_OK) return st;
  const bool sw = y_weight != nullptr, pn = out_weight != nullptr;
  if ((sw || pn) && !mhc::post_stable_supported(*d)) return MHC_ERR_UNSUPPORTED;
  if (sw != (dy_weight != nullptr) || pn != (dout_weight != nullptr)) return MHC_ERR_INVALID_ARG;
  if (d->T == 0) {
    if ((sw && !aligned16(dy_weight)) || (pn && !aligned16(dout_weight))) return MHC_ERR_INVALID_ARG;
    float* const p[2] = {dy_weight, dout_weight};
    const size_t n[2] = {(size_t)d->D, (size_t)d->N * d->D};
    return zero_params(p, n, 2, stream);
  }
  if (!aligned16(dx_next) || !aligned16(x) || !aligned16(y) || !aligned16(H_post) ||
      !aligned16(H_res) || !aligned16(dx) || !aligned16(dy) || !aligned16(dH_post) ||
      !aligned16(dH_res))
    return MHC_ERR_INVALID_ARG;
  if ((sw && (!aligned16(y_weight) || !aligned16(dy_weight))) ||
      (pn && (!aligned16(out_weight) || !aligned16(dout_weight))))
    return MHC_ERR_INVALID_ARG;
  const size_t b = io_bytes(d), T = (size_t)d->T, N = (size_t)d->N, D = (size_t)d->D;
  const size_t big = T * N * D * b, small = T * D * b;
  if (overlaps(dx, big, dx_next, big) || overlaps(dx, big, x, big) || overlaps(dx, big, y, small) ||
      overlaps(dy, small, dx_next, big) || overlaps(dy, small, x, big) || overlaps(dy, small, dx, big) ||
      overlaps(dy, small, y, small))
    return MHC_ERR_INVALID_ARG;
  const size_t need = mhc_post_stable_bwd_workspace_bytes(d, sw, pn);
  if (!workspace_ok(workspace, workspace_bytes, need)) return MHC_ERR_INVALID_ARG;
  if (need != 0) {
    const size_t part = need;
    if ((sw && overlaps(dy_weight, D * 4, workspace, part)) || (pn && overlaps(dout_weight, N * D * 4, workspace, part)))
      return MHC_ERR_INVALID_ARG;
  }
  return from_hip(mhc::launch_post_stable_bwd(*d, dx_next, x, y, y_weight, H_post, H_res, out_weight, dx,
                                              dy, dy_weight, dout_weight, dH_post, dH_res, workspace,
                                              stream));
}

}  // extern "C"
