// hc_pre forward for few tokens (decode-sized T), any N and D (openPangu 2.0
// analysis, §5.3 "mHC" formula block).
//
// With T ≤ kDecodeMaxT the work is tiny (x is at most T·40 KB at D=5120, N=4)
// and the time is latency: φ alone (N·D × (N²+2N) fp32, 2 MB at D=5120) is
// larger than x.  So the reduction is split over k across the whole chip:
//
//  1. pre_decode_partial: workgroup g owns 64 consecutive k (rows of φ) and
//     every token; it stages its φ rows in LDS, each thread takes one token and
//     8 of the k, and the eight threads of a token meet by lane shuffles.  It
//     writes, per token, the partial projections p[C] and sum of squares over
//     its k range.
//  2. pre_decode_finish: one workgroup per token sums the partials in k
//     order, forms rstd, logits and gates and runs the Sinkhorn rounds on N
//     lanes (one H_res row each; the same reciprocal instructions as the
//     split-K kernel), then collapses h = Σ_n H_pre[n]·x[n].
#include "mhc_coef.h"
#include "mhc_internal.h"

namespace mhc {
namespace decode {

constexpr int kThreads = 256;
constexpr int kRows = 64;                 // k (φ rows) per workgroup of pass 1
constexpr int kChunks = kRows / 8;        // threads per token in pass 1
constexpr int kTokPass = kThreads / kChunks;  // tokens per pass of a pass-1 workgroup

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

// Sum over each aligned group of G lanes (G = 1, 2, 4, 8) by DPP, every lane
// of a group getting the same total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<0xB1>(v);   // quad_perm(1,0,3,2)
  if constexpr (G >= 4) v += dpp<0x4E>(v);   // quad_perm(2,3,0,1)
  if constexpr (G >= 8) v += dpp<0x141>(v);  // row_half_mirror
  return v;
}

template <int N, int IO>
__global__ __launch_bounds__(kThreads) void pre_decode_partial(const void* __restrict__ x,
                                                               const float* __restrict__ phi,
                                                               float* __restrict__ part, int T, int K) {
  constexpr int C = N * N + 2 * N;
  __shared__ float phis[kRows * C];
  const int k0 = blockIdx.x * kRows;
  const int rows = K - k0 < kRows ? K - k0 : kRows;  // a multiple of 8
  for (int i = threadIdx.x; i < rows * C; i += kThreads) phis[i] = phi[(int64_t)k0 * C + i];
  __syncthreads();
  const int chunk = threadIdx.x % kChunks;
  const int kl = 8 * chunk;  // this thread's first row in the slice
  for (int tb = 0; tb < T; tb += kTokPass) {
    const int t = tb + threadIdx.x / kChunks;
    float acc[C + 1];
#pragma unroll
    for (int c = 0; c <= C; ++c) acc[c] = 0.f;
    if (t < T && kl < rows) {
      float v[8];
      load8<IO>(x, (int64_t)t * K + k0 + kl, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[C] += v[j] * v[j];
        const float* prow = phis + (kl + j) * C;
#pragma unroll
        for (int c = 0; c < C; ++c) acc[c] += v[j] * prow[c];
      }
    }
    // the kChunks = 8 threads of a token are lanes 8j..8j+7: sum them with
    // DPP in a fixed order
#pragma unroll
    for (int c = 0; c <= C; ++c) acc[c] = group_sum<kChunks>(acc[c]);
    if (chunk == 0 && t < T) {
      float* dst = part + ((int64_t)blockIdx.x * T + t) * (C + 1);
#pragma unroll
      for (int c = 0; c <= C; ++c) dst[c] = acc[c];
    }
  }
}

template <int N, int IO>
__global__ __launch_bounds__(kThreads) void pre_decode_finish(
    const void* __restrict__ x, const float* __restrict__ part, int G, const float* __restrict__ bias,
    void* __restrict__ h, float* __restrict__ H_pre, float* __restrict__ H_post,
    float* __restrict__ H_res, int T, int D, int iters, float eps, float a_pre, float a_post,
    float a_res, const float* __restrict__ alpha_dev) {
  if (alpha_dev != nullptr) {  // the gate scalars are held on the device (trained α)
    a_pre = alpha_dev[0];
    a_post = alpha_dev[1];
    a_res = alpha_dev[2];
  }
  constexpr int C = N * N + 2 * N;
  constexpr int kParts = kThreads / (C + 1);  // partial sums per column
  constexpr int kChunk = 16;                   // loads of a thread in flight together
  __shared__ float red[C + 1][kParts];
  __shared__ float tot[C + 1];
  __shared__ float hpre_s[N];
  const int64_t t = blockIdx.x;
  const int K = N * D;
  const int64_t base = t * (int64_t)K;
  // thread (q, c) sums column c of workgroups q, q + kParts, … (consecutive
  // threads read consecutive columns), then the parts are added in order
  if (threadIdx.x < (C + 1) * kParts) {
    const int c = threadIdx.x % (C + 1), q = threadIdx.x / (C + 1);
    float s = 0.f;
    for (int g0 = q; g0 < G; g0 += kChunk * kParts) {
      float v[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int g = g0 + u * kParts;
        v[u] = part[((int64_t)(g < G ? g : q) * T + t) * (C + 1) + c];
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (g0 + u * kParts < G) s += v[u];
    }
    red[c][q] = s;
  }
  __syncthreads();
  if (threadIdx.x <= C) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < kParts; ++q) s += red[threadIdx.x][q];
    tot[threadIdx.x] = s;
  }
  __syncthreads();
  // gates and Sinkhorn on N lanes of wave 0, lane i owning row i of H_res
  // (row sums in the lane, column sums across the N lanes)
  if (threadIdx.x < N) {
    const int i = threadIdx.x;
    const float rstd = __builtin_amdgcn_rsqf(tot[C] / (float)K + eps);
    const float hp = __builtin_amdgcn_rcpf(1.0f + expf(-(a_pre * (rstd * tot[i]) + bias[i])));
    hpre_s[i] = hp;
    H_pre[t * N + i] = hp;
    H_post[t * N + i] = 2.0f * __builtin_amdgcn_rcpf(1.0f + expf(-(a_post * (rstd * tot[N + i]) + bias[N + i])));
    float m[N], mx = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < N; ++j) {
      m[j] = a_res * (rstd * tot[2 * N + i * N + j]) + bias[2 * N + i * N + j];
      mx = fmaxf(mx, m[j]);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) m[j] = expf(m[j] - mx);  // a row factor: removed by the first row step
    for (int it = 0; it < iters; ++it) {
      float r = 0.f;
#pragma unroll
      for (int j = 0; j < N; ++j) r += m[j];
      const float rinv = __builtin_amdgcn_rcpf(r);
#pragma unroll
      for (int j = 0; j < N; ++j) m[j] *= rinv;
#pragma unroll
      for (int j = 0; j < N; ++j) {
        m[j] *= __builtin_amdgcn_rcpf(group_sum<N>(m[j]));
      }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) H_res[(t * N + i) * N + j] = m[j];
  }
  __syncthreads();
  float hp[N];
#pragma unroll
  for (int n = 0; n < N; ++n) hp[n] = hpre_s[n];
  for (int d0 = threadIdx.x * 8; d0 < D; d0 += kThreads * 8) {
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

}  // namespace decode

bool pre_decode_eligible(const mhc_desc& d) {
  // few tokens, and a partial-sum workspace of at most a few MB.  Measured on
  // MI355X at N = 4, D = 5120 (kernel time per call, bf16 and fp32): this
  // path takes 18-26 µs from 17 to 64 tokens, the split-K kernel 28-31 µs;
  // from 96 tokens on the split-K kernel is the faster one (this path grows
  // by about 6 µs per 32 tokens)
  return d.T <= kDecodeMaxT && (int64_t)d.N * d.D <= (1 << 20);
}

size_t pre_decode_workspace_bytes(const mhc_desc& d) {
  const int64_t K = (int64_t)d.N * d.D;
  const int64_t G = (K + decode::kRows - 1) / decode::kRows;
  const int C = d.N * d.N + 2 * d.N;
  return (size_t)(G * d.T * (C + 1)) * sizeof(float);
}

hipError_t launch_pre_decode(const mhc_desc& d, const void* x, const float* phi, const float* bias,
                             void* h, float* H_pre, float* H_post, float* H_res, void* ws,
                             hipStream_t s) {
  const int K = d.N * d.D;
  const int G = (K + decode::kRows - 1) / decode::kRows;
  float* part = static_cast<float*>(ws);
  bool ok = dispatch_n(d.N, [&](auto n_) {
    dispatch_io(d.io, [&](auto io_) {
      constexpr int N = decltype(n_)::value;
      constexpr int IO = decltype(io_)::value;
      MHC_LAUNCH((decode::pre_decode_partial<N, IO>), dim3((unsigned)G), dim3(decode::kThreads), 0,
                         s, x, phi, part, (int)d.T, K);
      MHC_LAUNCH((decode::pre_decode_finish<N, IO>), dim3((unsigned)d.T), dim3(decode::kThreads), 0,
                         s, x, part, G, bias, h, H_pre, H_post, H_res, (int)d.T, d.D, d.sinkhorn_iters,
                         d.eps, d.alpha_pre, d.alpha_post, d.alpha_res, d.alpha);
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mhc
