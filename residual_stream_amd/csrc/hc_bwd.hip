// Backward of hc_post and hc_pre (exact derivative of the openPangu 2.0
// analysis §5.3 formulas).  hc_pre's backward recomputes norm, logits and the
// Sinkhorn rounds from x, keeping no forward intermediates (Ascend mHC Triton
// article, intra-layer recompute paragraph).
#include "mhc_coef.h"
#include "mhc_internal.h"

namespace mhc {

// Five waves a token: two 8-element chunks a thread at D = 5120.  Measured on
// MI355X at T = 4096, N = 4, D = 5120, bf16, without dx: 71.0 µs against
// 72.2 µs for 256 threads and 81.0 µs for 640 (with the transposed
// workgroup sums; before them 256 threads measured best).
constexpr int kBwdThreads = 320;

// ------------------------------------------------------------ hc_post bwd ---
// One workgroup per token.  dx[m] = Σ_n H_res[n,m]·g[n], dy = Σ_n H_post[n]·g[n],
// dH_res[n,m] = <g[n], x[m]>, dH_post[n] = <g[n], y>, with g = dx_next; the
// N² + N sums in a fixed order.  WDX = false leaves dx to the caller's hc_pre
// backward (mhc_pre_bwd_mix forms it from dx_next there).
template <int N, int IO, bool WDX>
__global__ __launch_bounds__(kBwdThreads) void hc_post_bwd_generic(
    const void* __restrict__ dxn, const void* __restrict__ x, const void* __restrict__ y,
    const float* __restrict__ H_post, const float* __restrict__ H_res, void* __restrict__ dx,
    void* __restrict__ dy, float* __restrict__ dH_post, float* __restrict__ dH_res, int D) {
  constexpr int R = N * N + N;
  __shared__ float red[(kBwdThreads / kWave) * R];
  const int64_t t = blockIdx.x;
  float hr[N][N], hp[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    hp[n] = H_post[t * N + n];
#pragma unroll
    for (int m = 0; m < N; ++m) hr[n][m] = H_res[(t * N + n) * N + m];
  }
  float acc[R];
#pragma unroll
  for (int i = 0; i < R; ++i) acc[i] = 0.f;

  const int64_t xb = t * (int64_t)N * D;
  for (int d0 = threadIdx.x * 8; d0 < D; d0 += kBwdThreads * 8) {
    float g[N][8], xv[N][8], yv[8];
    load8_stream<IO>(y, t * D + d0, yv);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      load8_stream<IO>(dxn, xb + (int64_t)n * D + d0, g[n]);
      // without dx, the hc_pre backward of the same block reads x next: the
      // default policy leaves it to the caches (measured on MI355X: this
      // kernel's time unchanged, and the hc_pre projection pass 42 instead of
      // 50 µs when it follows directly, at T = 4096, D = 5120, bf16)
      if constexpr (WDX) load8_stream<IO>(x, xb + (int64_t)n * D + d0, xv[n]);
      else load8<IO>(x, xb + (int64_t)n * D + d0, xv[n]);
    }
    if constexpr (WDX) {
#pragma unroll
      for (int m = 0; m < N; ++m) {
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float a = 0.f;
#pragma unroll
          for (int n = 0; n < N; ++n) a += hr[n][m] * g[n][j];
          o[j] = a;
        }
        store8_stream<IO>(dx, xb + (int64_t)m * D + d0, o);
      }
    }
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float a = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) a += hp[n] * g[n][j];
      o[j] = a;
    }
    store8_stream<IO>(dy, t * D + d0, o);
#pragma unroll
    for (int n = 0; n < N; ++n) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int m = 0; m < N; ++m) acc[n * N + m] += g[n][j] * xv[m][j];
        acc[N * N + n] += g[n][j] * yv[j];
      }
    }
  }
  if constexpr (R <= kWave) {
    // DPP wave totals and one LDS exchange; lane i of wave 0 writes total i
    const float tot = wg_sum<R, kBwdThreads / kWave>(acc, red);
    if (threadIdx.x < N * N)
      dH_res[t * N * N + threadIdx.x] = tot;
    else if (threadIdx.x < R)
      dH_post[t * N + threadIdx.x - N * N] = tot;
  } else {
    block_sum<R>(acc, red);
    if (threadIdx.x == 0) {
#pragma unroll
      for (int i = 0; i < N * N; ++i) dH_res[t * N * N + i] = acc[i];
#pragma unroll
      for (int n = 0; n < N; ++n) dH_post[t * N + n] = acc[N * N + n];
    }
  }
}

// Zero fill of n floats (the parameter gradients of an empty batch): a
// kernel, so that a captured graph records no memset node.
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  MHC_LAUNCH(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, (int64_t)n);
  return hipGetLastError();
}

hipError_t launch_post_bwd(const mhc_desc& d, const void* dxn, const void* x, const void* y,
                           const float* H_post, const float* H_res, void* dx, void* dy,
                           float* dH_post, float* dH_res, hipStream_t s) {
  bool ok = dispatch_n(d.N, [&](auto n_) {
    dispatch_io(d.io, [&](auto io_) {
      constexpr int N = decltype(n_)::value;
      constexpr int IO = decltype(io_)::value;
      if (dx != nullptr)
        MHC_LAUNCH((hc_post_bwd_generic<N, IO, true>), dim3((unsigned)d.T), dim3(kBwdThreads), 0,
                           s, dxn, x, y, H_post, H_res, dx, dy, dH_post, dH_res, d.D);
      else
        MHC_LAUNCH((hc_post_bwd_generic<N, IO, false>), dim3((unsigned)d.T), dim3(kBwdThreads),
                           0, s, dxn, x, y, H_post, H_res, dx, dy, dH_post, dH_res, d.D);
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// dx[m] = Σ_n H_res[n,m]·dx_next[n] alone (one workgroup per token), in the
// arithmetic of hc_post_bwd_generic: the hc_post part of the state gradient
// for shapes whose hc_pre backward does not form it itself.
template <int N, int IO>
__global__ __launch_bounds__(kBwdThreads) void res_mix_t_kernel(const void* __restrict__ dxn,
                                                               const float* __restrict__ H_res,
                                                               void* __restrict__ dx, int D) {
  const int64_t t = blockIdx.x;
  float hr[N][N];
#pragma unroll
  for (int n = 0; n < N; ++n)
#pragma unroll
    for (int m = 0; m < N; ++m) hr[n][m] = H_res[(t * N + n) * N + m];
  const int64_t xb = t * (int64_t)N * D;
  for (int d0 = threadIdx.x * 8; d0 < D; d0 += kBwdThreads * 8) {
    float g[N][8];
#pragma unroll
    for (int n = 0; n < N; ++n) load8_stream<IO>(dxn, xb + (int64_t)n * D + d0, g[n]);
#pragma unroll
    for (int m = 0; m < N; ++m) {
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float a = 0.f;
#pragma unroll
        for (int n = 0; n < N; ++n) a += hr[n][m] * g[n][j];
        o[j] = a;
      }
      store8_stream<IO>(dx, xb + (int64_t)m * D + d0, o);
    }
  }
}

static hipError_t launch_res_mix_t(const mhc_desc& d, const void* dxn, const float* H_res, void* dx,
                                   hipStream_t s) {
  bool ok = dispatch_n(d.N, [&](auto n_) {
    dispatch_io(d.io, [&](auto io_) {
      constexpr int N = decltype(n_)::value;
      constexpr int IO = decltype(io_)::value;
      MHC_LAUNCH((res_mix_t_kernel<N, IO>), dim3((unsigned)d.T), dim3(kBwdThreads), 0, s, dxn,
                         H_res, dx, d.D);
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------- hc_pre bwd ---
//
// Workspace (fp32, each region 256-byte aligned):
//   gq[T][C]      rstd·α_g·dℓ   (the per-token factor of dφ = Σ_t x_tᵀ gq_t)
//   dlog[T][C]    dℓ            (summed over t into dbias)
//   dal[T][4]     Σ_{c∈g} dℓ_c·q_c per gate group (summed into dα)
//   part[S][K][C] per-token-split partial sums of dφ

static inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct PreBwdLayout {
  int C, K, S, kpt;
  size_t gq, dlog, dal, part, total;
};

static int dphi_kpt(int N) { return N <= 2 ? 8 : (N == 4 ? 4 : 1); }

static PreBwdLayout pre_bwd_layout(const mhc_desc& d) {
  PreBwdLayout L;
  L.C = d.N * d.N + 2 * d.N;
  L.K = d.N * d.D;
  L.kpt = dphi_kpt(d.N);
  int64_t s = (d.T + 255) / 256;
  L.S = (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
  const size_t T = (size_t)d.T;
  L.gq = 0;
  L.dlog = L.gq + align256(T * L.C * sizeof(float));
  L.dal = L.dlog + align256(T * L.C * sizeof(float));
  L.part = L.dal + align256(T * 4 * sizeof(float));
  L.total = L.part + align256((size_t)L.S * L.K * L.C * sizeof(float));
  return L;
}

size_t pre_bwd_workspace_bytes(const mhc_desc& d) {
  if (pre_bwd_mfma_eligible(d)) return pre_bwd_mfma_workspace_bytes(d);
  return pre_bwd_layout(d).total;
}

// One workgroup per token.  Pass 1: sum of squares, raw projections and
// dH_pre[n] = <dh, x[n]>.  One thread then recomputes the coefficients,
// records the Sinkhorn steps in LDS and walks them backwards.  Pass 2 writes
// dx += Σ_c gq_c·φ[k,c] − β·x_k + H_pre[n]·dh, β = rstd³·(dq·p)/K.
template <int N, int IO>
__global__ __launch_bounds__(kBwdThreads) void hc_pre_bwd_token(
    const void* __restrict__ dh, const void* __restrict__ x, const float* __restrict__ phi,
    const float* __restrict__ bias, const float* __restrict__ dH_post_in,
    const float* __restrict__ dH_res_in, void* __restrict__ dx, float* __restrict__ gq_out,
    float* __restrict__ dlog_out, float* __restrict__ dal_out, int D, int iters, float eps,
    float a_pre, float a_post, float a_res, const float* __restrict__ alpha_dev) {
  if (alpha_dev != nullptr) {  // the gate scalars are held on the device (trained α)
    a_pre = alpha_dev[0];
    a_post = alpha_dev[1];
    a_res = alpha_dev[2];
  }
  constexpr int C = N * N + 2 * N;
  constexpr int A = C + 1 + N;  // raw p[C], ss, dH_pre[N]
  __shared__ float red[(kBwdThreads / kWave) * A];
  __shared__ float gq_s[C];
  __shared__ float misc_s[N + 1];  // H_pre[N], beta
  extern __shared__ float rec[];   // Sinkhorn record: 2·iters·(N²+N)

  const int64_t t = blockIdx.x;
  const int K = N * D;
  const int64_t base = t * (int64_t)K;

  float acc[A];
#pragma unroll
  for (int i = 0; i < A; ++i) acc[i] = 0.f;
#pragma unroll
  for (int n = 0; n < N; ++n) {
    for (int d0 = threadIdx.x * 8; d0 < D; d0 += kBwdThreads * 8) {
      float v[8], g[8];
      load8<IO>(x, base + (int64_t)n * D + d0, v);
      load8<IO>(dh, t * D + d0, g);
      const int k0 = n * D + d0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        acc[C] += v[j] * v[j];
        acc[C + 1 + n] += g[j] * v[j];
        const float* prow = phi + (int64_t)(k0 + j) * C;
#pragma unroll
        for (int c = 0; c < C; ++c) acc[c] += v[j] * prow[c];
      }
    }
  }
  block_sum<A>(acc, red);

  if (threadIdx.x == 0) {
    float l[C];
    const float rstd = token_logits<N>(acc, acc[C], K, eps, a_pre, a_post, a_res, bias, l);
    float dl[C];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float sp = sigmoid(l[n]);
      const float sq = sigmoid(l[N + n]);
      misc_s[n] = sp;
      dl[n] = acc[C + 1 + n] * sp * (1.0f - sp);
      dl[N + n] = dH_post_in[t * N + n] * 2.0f * sq * (1.0f - sq);
    }
    float M0[N][N], M[N][N], G[N][N];
    res_exp<N>(l + 2 * N, M0);
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) {
        M[i][j] = M0[i][j];
        G[i][j] = dH_res_in[(t * N + i) * N + j];
      }
    for (int it = 0; it < iters; ++it) sinkhorn_round<N>(M, rec + (size_t)it * 2 * (N * N + N));
    sinkhorn_backward<N>(G, rec, iters);
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) dl[2 * N + i * N + j] = G[i][j] * M0[i][j];

    float dqp = 0.f, da[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int grp = c < N ? 0 : (c < 2 * N ? 1 : 2);
      const float a = grp == 0 ? a_pre : (grp == 1 ? a_post : a_res);
      const float dq = a * dl[c];
      dqp += dq * acc[c];
      da[grp] += dl[c] * (rstd * acc[c]);
      gq_s[c] = rstd * dq;
      gq_out[t * C + c] = rstd * dq;
      dlog_out[t * C + c] = dl[c];
    }
    misc_s[N] = rstd * rstd * rstd * dqp / (float)K;
    dal_out[t * 4 + 0] = da[0];
    dal_out[t * 4 + 1] = da[1];
    dal_out[t * 4 + 2] = da[2];
    dal_out[t * 4 + 3] = 0.f;
  }
  __syncthreads();

  float g[C];
#pragma unroll
  for (int c = 0; c < C; ++c) g[c] = gq_s[c];
  const float beta = misc_s[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const float hp = misc_s[n];
    for (int d0 = threadIdx.x * 8; d0 < D; d0 += kBwdThreads * 8) {
      float v[8], gh[8], o[8];
      const int64_t i0 = base + (int64_t)n * D + d0;
      load8<IO>(x, i0, v);
      load8<IO>(dh, t * D + d0, gh);
      load8<IO>(dx, i0, o);
      const int k0 = n * D + d0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float* prow = phi + (int64_t)(k0 + j) * C;
        float a = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) a += g[c] * prow[c];
        o[j] += a - beta * v[j] + hp * gh[j];
      }
      store8<IO>(dx, i0, o);
    }
  }
}

template <int IO, int KPT>
__device__ __forceinline__ void load_kpt(const void* base, int64_t i, float (&v)[KPT]) {
  if constexpr (KPT == 8) {
    load8<IO>(base, i, v);
  } else if constexpr (IO == kF32) {
    const float* p = static_cast<const float*>(base) + i;
    if constexpr (KPT == 4) {
      float4 a = *reinterpret_cast<const float4*>(p);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) v[j] = p[j];
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + i;
    if constexpr (KPT == 4) {
      uint2 w = *reinterpret_cast<const uint2*>(p);
      v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j) v[j] = __uint_as_float((uint32_t)p[j] << 16);
    }
  }
}

// Partial dφ over one token split: part[s][k][c] = Σ_{t in split s} x[t,k]·gq[t,c].
// Each thread owns KPT consecutive k; gq rows are staged through LDS.
constexpr int kStageTok = 64;
template <int N, int IO, int KPT>
__global__ __launch_bounds__(kBwdThreads) void dphi_partial(const void* __restrict__ x,
                                                            const float* __restrict__ gq,
                                                            float* __restrict__ part, int64_t T,
                                                            int K, int64_t tok_per_split) {
  constexpr int C = N * N + 2 * N;
  __shared__ float gs[kStageTok * C];
  const int k0 = (blockIdx.x * kBwdThreads + threadIdx.x) * KPT;
  const int64_t t_beg = (int64_t)blockIdx.y * tok_per_split;
  int64_t t_end = t_beg + tok_per_split;
  if (t_end > T) t_end = T;
  float acc[KPT][C];
#pragma unroll
  for (int i = 0; i < KPT; ++i)
#pragma unroll
    for (int c = 0; c < C; ++c) acc[i][c] = 0.f;

  for (int64_t tc = t_beg; tc < t_end; tc += kStageTok) {
    const int nt = (int)((t_end - tc) < kStageTok ? (t_end - tc) : kStageTok);
    __syncthreads();
    for (int i = threadIdx.x; i < nt * C; i += kBwdThreads) gs[i] = gq[tc * C + i];
    __syncthreads();
    if (k0 < K) {
      for (int tt = 0; tt < nt; ++tt) {
        float v[KPT];
        load_kpt<IO, KPT>(x, (tc + tt) * K + k0, v);
#pragma unroll
        for (int i = 0; i < KPT; ++i)
#pragma unroll
          for (int c = 0; c < C; ++c) acc[i][c] += v[i] * gs[tt * C + c];
      }
    }
  }
  if (k0 < K) {
    float* dst = part + ((int64_t)blockIdx.y * K + k0) * C;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
#pragma unroll
      for (int c = 0; c < C; ++c) dst[i * C + c] = acc[i][c];
  }
}

// dφ = Σ_s part[s], in split order.
__global__ __launch_bounds__(kBwdThreads) void dphi_reduce(const float* __restrict__ part,
                                                           float* __restrict__ dphi, int64_t KC,
                                                           int S) {
  const int64_t i = (int64_t)blockIdx.x * kBwdThreads + threadIdx.x;
  if (i >= KC) return;
  float s = 0.f;
  for (int j = 0; j < S; ++j) s += part[(int64_t)j * KC + i];
  dphi[i] = s;
}

// dbias[c] = Σ_t dℓ[t,c]; dα[g] = Σ_t dal[t,g].  One workgroup, fixed order.
template <int N>
__global__ __launch_bounds__(kBwdThreads) void bias_alpha_reduce(const float* __restrict__ dlog,
                                                                 const float* __restrict__ dal,
                                                                 float* __restrict__ dbias,
                                                                 float* __restrict__ dalpha,
                                                                 int64_t T) {
  constexpr int C = N * N + 2 * N;
  __shared__ float red[(kBwdThreads / kWave) * (C + 3)];
  float acc[C + 3];
#pragma unroll
  for (int i = 0; i < C + 3; ++i) acc[i] = 0.f;
  for (int64_t t = threadIdx.x; t < T; t += kBwdThreads) {
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] += dlog[t * C + c];
#pragma unroll
    for (int g = 0; g < 3; ++g) acc[C + g] += dal[t * 4 + g];
  }
  block_sum<C + 3>(acc, red);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int c = 0; c < C; ++c) dbias[c] = acc[c];
    if (dalpha) {
#pragma unroll
      for (int g = 0; g < 3; ++g) dalpha[g] = acc[C + g];
    }
  }
}

hipError_t launch_pre_bwd_mix(const mhc_desc& d, const void* dh, const void* x, const float* phi,
                              const float* bias, const float* dH_post, const float* dH_res,
                              const void* dxn, const float* H_res, void* dx, float* dphi, float* dbias,
                              float* dalpha, void* ws, hipStream_t s) {
  // bf16 on the matrix-core path: the dx pass reads dx_next and mixes it in
  // registers; elsewhere the mix is written first and accumulated into
  if (pre_bwd_mfma_eligible(d) && d.io == kBF16)
    return launch_pre_bwd_mfma(d, dh, x, phi, bias, dH_post, dH_res, dx, dphi, dbias, dalpha, ws, s, dxn,
                               H_res);
  const hipError_t e = launch_res_mix_t(d, dxn, H_res, dx, s);
  if (e != hipSuccess) return e;
  return launch_pre_bwd(d, dh, x, phi, bias, dH_post, dH_res, dx, dphi, dbias, dalpha, ws, s);
}

hipError_t launch_pre_bwd(const mhc_desc& d, const void* dh, const void* x, const float* phi,
                          const float* bias, const float* dH_post, const float* dH_res, void* dx,
                          float* dphi, float* dbias, float* dalpha, void* ws, hipStream_t s) {
  if (pre_bwd_mfma_eligible(d)) {
    return launch_pre_bwd_mfma(d, dh, x, phi, bias, dH_post, dH_res, dx, dphi, dbias, dalpha, ws, s,
                               nullptr, nullptr);
  }
  const PreBwdLayout L = pre_bwd_layout(d);
  char* w = static_cast<char*>(ws);
  float* gq = reinterpret_cast<float*>(w + L.gq);
  float* dlog = reinterpret_cast<float*>(w + L.dlog);
  float* dal = reinterpret_cast<float*>(w + L.dal);
  float* part = reinterpret_cast<float*>(w + L.part);
  const int64_t tok_per_split = (d.T + L.S - 1) / L.S;
  hipError_t err = hipSuccess;
  bool ok = dispatch_n(d.N, [&](auto n_) {
    dispatch_io(d.io, [&](auto io_) {
      constexpr int N = decltype(n_)::value;
      constexpr int IO = decltype(io_)::value;
      constexpr int C = N * N + 2 * N;
      constexpr int KPT = N <= 2 ? 8 : (N == 4 ? 4 : 1);
      const size_t rec_bytes = (size_t)2 * d.sinkhorn_iters * (N * N + N) * sizeof(float);
      MHC_LAUNCH((hc_pre_bwd_token<N, IO>), dim3((unsigned)d.T), dim3(kBwdThreads),
                         rec_bytes, s, dh, x, phi, bias, dH_post, dH_res, dx, gq, dlog, dal, d.D,
                         d.sinkhorn_iters, d.eps, d.alpha_pre, d.alpha_post, d.alpha_res, d.alpha);
      if ((err = hipGetLastError()) != hipSuccess) return;
      const unsigned gx = (unsigned)((L.K + kBwdThreads * KPT - 1) / (kBwdThreads * KPT));
      MHC_LAUNCH((dphi_partial<N, IO, KPT>), dim3(gx, (unsigned)L.S), dim3(kBwdThreads), 0,
                         s, x, gq, part, (int64_t)d.T, L.K, tok_per_split);
      if ((err = hipGetLastError()) != hipSuccess) return;
      const int64_t KC = (int64_t)L.K * C;
      MHC_LAUNCH(dphi_reduce, dim3((unsigned)((KC + kBwdThreads - 1) / kBwdThreads)),
                         dim3(kBwdThreads), 0, s, part, dphi, KC, L.S);
      if ((err = hipGetLastError()) != hipSuccess) return;
      MHC_LAUNCH((bias_alpha_reduce<N>), dim3(1), dim3(kBwdThreads), 0, s, dlog, dal,
                         dbias, dalpha, (int64_t)d.T);
      err = hipGetLastError();
    });
  });
  if (!ok) return hipErrorInvalidValue;
  return err;
}

}  // namespace mhc
