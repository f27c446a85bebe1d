// hc_pre forward (openPangu 2.0 analysis, §5.3 "mHC" formula block), generic
// path for the shapes the matrix-core kernel does not cover (N ≠ 4, D not a
// multiple of 32, very wide D).
//
// Kernel: one workgroup per token.  Pass 1 reads the token's N·D
// elements once, accumulating the sum of squares and the C = N²+2N raw
// projections x·φ (φ rows come from L2); a block reduction gives the totals;
// one thread forms the logits, gates and Sinkhorn rounds; pass 2 collapses the
// streams, h = Σ_n H_pre[n]·x[n], re-reading the token (an L2 hit: the same
// workgroup touched it microseconds before).
#include "mhc_coef.h"
#include "mhc_internal.h"

namespace mhc {

constexpr int kPreThreads = 256;

template <int N, int IO>
__global__ __launch_bounds__(kPreThreads) void hc_pre_generic(
    const void* __restrict__ x, const float* __restrict__ phi, const float* __restrict__ bias,
    void* __restrict__ h, float* __restrict__ H_pre, float* __restrict__ H_post,
    float* __restrict__ H_res, int D, int iters, float eps, float a_pre, float a_post,
    float a_res, const float* __restrict__ alpha_dev) {
  if (alpha_dev != nullptr) {  // the gate scalars are held on the device (trained α)
    a_pre = alpha_dev[0];
    a_post = alpha_dev[1];
    a_res = alpha_dev[2];
  }
  constexpr int C = N * N + 2 * N;
  __shared__ float red[(kPreThreads / kWave) * (C + 1)];
  __shared__ float hpre_s[N];

  const int64_t t = blockIdx.x;
  const int K = N * D;
  const int64_t base = t * (int64_t)K;

  float acc[C + 1];
#pragma unroll
  for (int c = 0; c <= C; ++c) acc[c] = 0.f;

  for (int k0 = threadIdx.x * 8; k0 < K; k0 += kPreThreads * 8) {
    float v[8];
    load8<IO>(x, base + k0, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[C] += v[j] * v[j];
      const float* prow = phi + (int64_t)(k0 + j) * C;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] += v[j] * prow[c];
    }
  }
  block_sum<C + 1>(acc, red);

  if (threadIdx.x == 0) {
    float l[C];
    token_logits<N>(acc, acc[C], K, eps, a_pre, a_post, a_res, bias, l);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float hp = sigmoid(l[n]);
      hpre_s[n] = hp;
      H_pre[t * N + n] = hp;
      H_post[t * N + n] = 2.0f * sigmoid(l[N + n]);
    }
    float M[N][N];
    res_exp<N>(l + 2 * N, M);
    for (int it = 0; it < iters; ++it) sinkhorn_round<N>(M, nullptr);
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) H_res[(t * N + i) * N + j] = M[i][j];
  }
  __syncthreads();

  float hp[N];
#pragma unroll
  for (int n = 0; n < N; ++n) hp[n] = hpre_s[n];
  for (int d0 = threadIdx.x * 8; d0 < D; d0 += kPreThreads * 8) {
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float v[8];
      load8<IO>(x, base + (int64_t)n * D + d0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] += hp[n] * v[j];
    }
    store8<IO>(h, t * D + d0, o);
  }
}

hipError_t launch_pre_generic(const mhc_desc& d, const void* x, const float* phi,
                              const float* bias, void* h, float* H_pre, float* H_post,
                              float* H_res, hipStream_t s) {
  bool ok = dispatch_n(d.N, [&](auto n_) {
    dispatch_io(d.io, [&](auto io_) {
      constexpr int N = decltype(n_)::value;
      constexpr int IO = decltype(io_)::value;
      MHC_LAUNCH((hc_pre_generic<N, IO>), dim3((unsigned)d.T), dim3(kPreThreads), 0, s,
                         x, phi, bias, h, H_pre, H_post, H_res, d.D, d.sinkhorn_iters, d.eps,
                         d.alpha_pre, d.alpha_post, d.alpha_res, d.alpha);
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mhc
