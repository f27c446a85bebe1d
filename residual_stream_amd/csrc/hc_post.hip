// hc_post forward: x_next[n] = Σ_m H_res[n,m]·x[m] + H_post[n]·y
// (openPangu 2.0 analysis, §5.3 roles of the maps; Ascend mHC Triton article,
// definition paragraph).  Pure stream: x and y read once, x_next written once.
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {

// At most ten waves a workgroup: a D = 5120 row in one pass, one 8-element
// chunk a thread (measured on MI355X: 62 instead of 66 µs per call at
// T = 4096, N = 4, D = 5120, bf16, against 256 threads and 2.5 passes).
constexpr int kPostMaxThreads = 640;

// One workgroup per token; each thread owns 8 consecutive d of every stream
// (d0, d0 + 8·blockDim, …).  x_next is stored non-temporally, unless KEEP:
// then with the default policy, for a kernel that reads it right after.
template <int N, int IO, bool KEEP>
__global__ __launch_bounds__(kPostMaxThreads) void hc_post_generic(
    const void* __restrict__ x, const void* __restrict__ y, const float* __restrict__ H_post,
    const float* __restrict__ H_res, void* __restrict__ x_next, int D) {
  const int64_t t = blockIdx.x;
  float hr[N][N], hp[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    hp[n] = H_post[t * N + n];
#pragma unroll
    for (int m = 0; m < N; ++m) hr[n][m] = H_res[(t * N + n) * N + m];
  }
  const int64_t xb = t * (int64_t)N * D;
  for (int d0 = threadIdx.x * 8; d0 < D; d0 += (int)blockDim.x * 8) {
    float xv[N][8], yv[8];
    load8_stream<IO>(y, t * D + d0, yv);
#pragma unroll
    for (int m = 0; m < N; ++m) load8_stream<IO>(x, xb + (int64_t)m * D + d0, xv[m]);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // fixed order, explicit fused multiply-adds: H_post·y first, then
        // the streams in order (the order the oracle's tolerance was set for
        // and that every caller of the write-back gets, bit for bit)
        float a = hp[n] * yv[j];
#pragma unroll
        for (int m = 0; m < N; ++m) a = __builtin_fmaf(hr[n][m], xv[m][j], a);
        o[j] = a;
      }
      if constexpr (KEEP)
        store8<IO>(x_next, xb + (int64_t)n * D + d0, o);
      else
        store8_stream<IO>(x_next, xb + (int64_t)n * D + d0, o);
    }
  }
}

hipError_t launch_post(const mhc_desc& d, const void* x, const void* y, const float* H_post,
                       const float* H_res, void* x_next, hipStream_t s, bool keep_out) {
  // a chunk per thread, whole waves, up to the maximum
  const int chunks = (d.D + 7) / 8;
  int nthr = (chunks + kWave - 1) / kWave * kWave;
  if (nthr > kPostMaxThreads) nthr = kPostMaxThreads;
  bool ok = dispatch_n(d.N, [&](auto n_) {
    dispatch_io(d.io, [&](auto io_) {
      constexpr int N = decltype(n_)::value;
      constexpr int IO = decltype(io_)::value;
      if (keep_out)
        MHC_LAUNCH((hc_post_generic<N, IO, true>), dim3((unsigned)d.T), dim3((unsigned)nthr), 0, s,
                   x, y, H_post, H_res, x_next, d.D);
      else
        MHC_LAUNCH((hc_post_generic<N, IO, false>), dim3((unsigned)d.T), dim3((unsigned)nthr), 0, s,
                   x, y, H_post, H_res, x_next, d.D);
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mhc
