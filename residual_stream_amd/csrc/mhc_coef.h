// Per-token coefficient math of hc_pre, on one thread: gates and Sinkhorn
// (openPangu 2.0 analysis, §5.3 "mHC" formula block), and their derivative.
#pragma once

#include "mhc_device.h"

namespace mhc {

// Logits of one token from its raw projection p = x·φ and sum of squares ss:
// rstd = (ss/K + eps)^(-1/2), ℓ_c = α_g(c)·rstd·p_c + b_c, with the column
// groups [pre N | post N | res N²].
template <int N>
__device__ __forceinline__ float token_logits(const float* p, float ss, int K, float eps,
                                              float a_pre, float a_post, float a_res,
                                              const float* bias, float* l) {
  constexpr int C = N * N + 2 * N;
  const float rstd = 1.0f / sqrtf(ss / (float)K + eps);
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float a = c < N ? a_pre : (c < 2 * N ? a_post : a_res);
    l[c] = a * (rstd * p[c]) + bias[c];
  }
  return rstd;
}

// exp of the res logits with each row's maximum subtracted.  Sinkhorn's first
// step divides every row by its sum, so a per-row factor cancels exactly; the
// shift only keeps exp in range.
template <int N>
__device__ __forceinline__ void res_exp(const float* l_res, float M[N][N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float mx = l_res[i * N];
#pragma unroll
    for (int j = 1; j < N; ++j) mx = fmaxf(mx, l_res[i * N + j]);
#pragma unroll
    for (int j = 0; j < N; ++j) M[i][j] = expf(l_res[i * N + j] - mx);
  }
}

// One Sinkhorn–Knopp round: divide each row by its sum, then each column by
// its sum.  If `rec` is given, store both step outputs and their divisors:
// rec = [Y_row (N²), r (N), Y_col (N²), c (N)].
template <int N>
__device__ __forceinline__ void sinkhorn_round(float M[N][N], float* rec) {
  float s[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float r = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) r += M[i][j];
    s[i] = r;
    const float inv = 1.0f / r;
#pragma unroll
    for (int j = 0; j < N; ++j) M[i][j] *= inv;
  }
  if (rec) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int j = 0; j < N; ++j) rec[i * N + j] = M[i][j];
      rec[N * N + i] = s[i];
    }
    rec += N * N + N;
  }
#pragma unroll
  for (int j = 0; j < N; ++j) {
    float c = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) c += M[i][j];
    s[j] = c;
    const float inv = 1.0f / c;
#pragma unroll
    for (int i = 0; i < N; ++i) M[i][j] *= inv;
  }
  if (rec) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
#pragma unroll
      for (int j = 0; j < N; ++j) rec[i * N + j] = M[i][j];
      rec[N * N + i] = s[i];
    }
  }
}

// Gradient through the recorded rounds, last step first.  A step Y = X / s
// (s = sums along rows or columns) has dX = (dY − Σ_along dY⊙Y) / s.
template <int N>
__device__ __forceinline__ void sinkhorn_backward(float G[N][N], const float* rec, int iters) {
  constexpr int R = N * N + N;
  for (int it = iters - 1; it >= 0; --it) {
    const float* col = rec + (2 * it + 1) * R;
    const float* row = rec + (2 * it) * R;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) acc += G[i][j] * col[i * N + j];
      const float inv = 1.0f / col[N * N + j];
#pragma unroll
      for (int i = 0; i < N; ++i) G[i][j] = (G[i][j] - acc) * inv;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < N; ++j) acc += G[i][j] * row[i * N + j];
      const float inv = 1.0f / row[N * N + i];
#pragma unroll
      for (int j = 0; j < N; ++j) G[i][j] = (G[i][j] - acc) * inv;
    }
  }
}

}  // namespace mhc
