// Stabilised write-back of openPangu's mHC (openPangu 2.0 analysis, §5.4,
// first two items): an RMSNorm of the sublayer output y with a learnable
// weight w_y[D] before H_post writes it back (the sandwich norm), and an
// RMSNorm of the token's whole N-stream state, flattened to N·D, with a weight
// w_x[N·D] after it (the block-level post-norm).  Either norm may be off.
//
//   ŷ      = (y·r_y)·w_y                  r_y = rsq(mean_d y² + eps)
//   z[n]   = H_post[n]·ŷ + Σ_m H_res[n,m]·x[m]     (hc_post's fma order)
//   x_next = (z·r_z)·w_x                  r_z = rsq(mean_{n,d} z² + eps)
//
// A workgroup holds a whole token in registers: thread i owns the 8-element
// chunks q = j·nthr + i (j < CPT) of y and of every stream, so each wave
// reads and writes 1 KB runs of every row, and the two norms cost one
// workgroup reduction each.  nthr ≤ 640 (ten waves), CPT ∈ {1, 2, 4} and
// N·CPT ≤ 4: D ≤ 5120 at N = 4, 10240 at N = 2, 20480 at N = 1.
//
// Backward, the exact derivative, recomputing ŷ, z and both scales from x and
// y (the recompute policy of the hc_pre backward; nothing of the forward is
// kept):
//   u = w_x ⊙ dx_next,  g_z = r_z·u − (r_z³/K)·Σ(u⊙z)·z     (post-norm on;
//                                                            else g_z = dx_next)
//   dx[m] = Σ_n H_res[n,m]·g_z[n],   g = Σ_n H_post[n]·g_z[n]
//   dH_res[n,m] = <g_z[n], x[m]>,    dH_post[n] = <g_z[n], ŷ>
//   dy = r_y·w_y⊙g − (r_y³/D)·Σ(w_y⊙g⊙y)·y                 (sandwich on; else g)
//   dw_y = Σ_t r_y·g⊙y,              dw_x = Σ_t r_z·dx_next⊙z
// The weight gradients are sums over tokens: a fixed grid of G workgroups
// walks the tokens t ≡ b (mod G), each keeping its share of dw (dw_x in LDS,
// dw_y in registers), and writes one row of partial sums; a second kernel adds the G rows in
// order.
#include "mhc_device.h"
#include "mhc_internal.h"

namespace mhc {
namespace stab {

constexpr int kMaxThreads = 640;
constexpr int kMaxWaves = kMaxThreads / kWave;
constexpr int kSumWaves = 16;  // row split of the weight-gradient sum
constexpr uint32_t kOffOut = 0x80000000u;  // a lane offset outside every buffer descriptor

// Eight I/O elements as loaded, kept packed until used (bf16: four words, so
// a token's x and dx_next cost half the registers).
template <int IO>
struct Pack8;
template <>
struct Pack8<kBF16> {
  uint4 w;
  __device__ __forceinline__ void load(const void* b, int64_t i) {  // non-temporal: a stream
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(static_cast<const uint16_t*>(b) + i));
    w = make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ __forceinline__ void zero() { w = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
  __device__ __forceinline__ float operator[](int j) const {
    const uint32_t v = j < 2 ? w.x : (j < 4 ? w.y : (j < 6 ? w.z : w.w));
    return (j & 1) ? bf16_hi(v) : bf16_lo(v);
  }
  // Makes the words opaque to the compiler, so that fp32 values unpacked
  // before this point are not kept alive to be reused after it.
  __device__ __forceinline__ void fence() { asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w)); }
};
template <>
struct Pack8<kF32> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* p, int64_t i) {
    const float4* q = reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    a = q[0];
    b = q[1];
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff);
  __device__ __forceinline__ float operator[](int j) const {
    const float4& h = j < 4 ? a : b;
    const int k = j & 3;
    return k == 0 ? h.x : (k == 1 ? h.y : (k == 2 ? h.z : h.w));
  }
  __device__ __forceinline__ void fence() {}
};

__device__ __forceinline__ void load_w8(const float* w, int64_t i, float v[8]) {
  const float4* p = reinterpret_cast<const float4*>(w + i);
  const float4 a = p[0], b = p[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void store_f8(float* p, const float v[8]) {
  float4* q = reinterpret_cast<float4*>(p);
  q[0] = make_float4(v[0], v[1], v[2], v[3]);
  q[1] = make_float4(v[4], v[5], v[6], v[7]);
}

typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor over `bytes` bytes from `base` (raw, unswizzled): lanes
// whose offset falls outside read 0 and drop their stores.
__device__ __forceinline__ Rsrc rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy: the norm weights are read for every token and keep the
// default; bf16 tensor streams (read or written once) go non-temporal, which
// measured faster for the hc_post kernels on MI355X (fp32 streams keep the
// default).
constexpr int kStream = 2;  // nt
template <int POLICY = 0>
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, POLICY);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16-byte store.  The scalar offset is always the literal 0 and any stream
// offset goes into the lane offset: with a register there, the compiler
// leaves out the wait state that protects a wide store's data registers from
// the next VALU write, and gfx950 then stores a corrupted first word on some
// lanes.
template <int POLICY>
__device__ __forceinline__ void bstore16(Rsrc r, uint32_t voff, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)voff, 0, POLICY);
}
__device__ __forceinline__ void load_w8(Rsrc r, uint32_t voff, uint32_t soff, float v[8]) {
  const uint4 a = bload16(r, voff, soff), b = bload16(r, voff + 16, soff);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}
// Eight values stored in the I/O dtype (bf16: round to nearest even) at lane
// offset voff + off.
template <int IO>
__device__ __forceinline__ void store8b(Rsrc r, uint32_t voff, uint32_t off, const float v[8]) {
  voff += off;
  if constexpr (IO == kF32) {
    bstore16<0>(r, voff, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])));
    bstore16<0>(r, voff + 16, make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])));
  } else {
    bstore16<kStream>(r, voff, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                       pack_bf16x2(v[6], v[7])));
  }
}

__device__ __forceinline__ void Pack8<kBF16>::load(Rsrc r, uint32_t voff, uint32_t soff) {
  w = bload16<kStream>(r, voff, soff);
}
__device__ __forceinline__ void Pack8<kF32>::load(Rsrc r, uint32_t voff, uint32_t soff) {
  const uint4 p = bload16(r, voff, soff), q = bload16(r, voff + 16, soff);
  a = make_float4(__uint_as_float(p.x), __uint_as_float(p.y), __uint_as_float(p.z), __uint_as_float(p.w));
  b = make_float4(__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z), __uint_as_float(q.w));
}

// z[n] at element e of a chunk: H_post[n]·ŷ + Σ_m H_res[n,m]·x[m], with
// ŷ = (y·r_y)·w_y under the sandwich norm; the fma order of hc_post.
template <int N, int IO, bool SW>
__device__ __forceinline__ float z_at(float hp, const float (&hr)[N], const Pack8<IO> (&xr)[N], float y,
                                      float ry, float wy, int e) {
  const float yh = SW ? (y * ry) * wy : y;
  float a = hp * yh;
#pragma unroll
  for (int m = 0; m < N; ++m) a = __builtin_fmaf(hr[m], xr[m][e], a);
  return a;
}

template <int N, int IO, int CPT, bool SW, bool PN>
__global__ __launch_bounds__(kMaxThreads) void post_stable_fwd(
    const void* __restrict__ x, const void* __restrict__ y, const float* __restrict__ wy,
    const float* __restrict__ H_post, const float* __restrict__ H_res, const float* __restrict__ wx,
    void* __restrict__ x_next, int D, float eps) {
  __shared__ float red[2][kMaxWaves];
  const int64_t t = blockIdx.x;
  const int nthr = blockDim.x;
  const int K = N * D;
  float hp[N], hr[N][N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    hp[n] = H_post[t * N + n];
#pragma unroll
    for (int m = 0; m < N; ++m) hr[n][m] = H_res[(t * N + n) * N + m];
  }
  const int64_t xb = t * (int64_t)K;
  int d0[CPT];
  bool ok[CPT];
  Pack8<IO> xr[CPT][N], yr[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    d0[j] = 8 * (j * nthr + (int)threadIdx.x);
    ok[j] = d0[j] < D;
    if (ok[j]) {
      yr[j].load(y, t * D + d0[j]);
#pragma unroll
      for (int m = 0; m < N; ++m) xr[j][m].load(x, xb + (int64_t)m * D + d0[j]);
    } else {
      yr[j].zero();
#pragma unroll
      for (int m = 0; m < N; ++m) xr[j][m].zero();
    }
  }
  float yh[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) yh[j][e] = yr[j][e];
  if constexpr (SW) {
    float ss[1] = {0.f};
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss[0] += yh[j][e] * yh[j][e];
    const float ry = __builtin_amdgcn_rsqf(lane_f(wg_sum<1, kMaxWaves>(ss, red[0]), 0) / (float)D + eps);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float w[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (ok[j]) load_w8(wy, d0[j], w);
#pragma unroll
      for (int e = 0; e < 8; ++e) yh[j][e] = (yh[j][e] * ry) * w[e];
    }
  }
  float z[CPT][N][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int n = 0; n < N; ++n)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = hp[n] * yh[j][e];
#pragma unroll
        for (int m = 0; m < N; ++m) a = __builtin_fmaf(hr[n][m], xr[j][m][e], a);
        z[j][n][e] = a;
      }
  if constexpr (PN) {
    float ss[1] = {0.f};
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int n = 0; n < N; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) ss[0] += z[j][n][e] * z[j][n][e];
    const float rz = __builtin_amdgcn_rsqf(lane_f(wg_sum<1, kMaxWaves>(ss, red[1]), 0) / (float)K + eps);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      if (!ok[j]) continue;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        float w[8];
        load_w8(wx, (int64_t)n * D + d0[j], w);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[j][n][e] = (z[j][n][e] * rz) * w[e];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (!ok[j]) continue;
#pragma unroll
    for (int n = 0; n < N; ++n) store8_stream<IO>(x_next, xb + (int64_t)n * D + d0[j], z[j][n]);
  }
}

template <int N, int IO, int CPT, bool SW, bool PN>
__global__ __launch_bounds__(kMaxThreads) void post_stable_bwd(
    const void* __restrict__ dxn, const void* __restrict__ x, const void* __restrict__ y,
    const float* __restrict__ wy, const float* __restrict__ H_post, const float* __restrict__ H_res,
    const float* __restrict__ wx, void* __restrict__ dx, void* __restrict__ dy,
    float* __restrict__ dH_post, float* __restrict__ dH_res, float* __restrict__ part, int64_t T,
    int D, float eps) {
  // totals of the last reduction: dH_res[N²], <g_z[n], w_y⊙y or y>[N],
  // then with the sandwich norm Σ g⊙w_y⊙y and (without the post-norm,
  // which needs r_y earlier) Σ y²
  constexpr int kS = N * N + N, kY = kS + 1;
  constexpr int R3 = kS + (SW ? 1 : 0) + ((SW && !PN) ? 1 : 0);
  constexpr int B = IoT<IO>::bytes;
  __shared__ float red1[2][kMaxWaves];
  __shared__ float red2[2][kMaxWaves * 2];
  __shared__ float red3[2][kMaxWaves * R3];
  const int nthr = blockDim.x;
  const int K = N * D;
  const uint32_t rowD = (uint32_t)D * B;  // bytes of one stream row
  // dw_x partial sums of this thread live in LDS, not in registers: slot
  // (j, n, half) of thread i at accx_s[((j·N + n)·2 + half)·nthr + i], so a
  // wave's 16-byte accesses are contiguous.  Dynamic LDS of
  // accx_lds_bytes(N, CPT, nthr): N·CPT ≤ 4 makes it at most 80 KB.
  extern __shared__ float4 accx_s[];
  int d0[CPT];
  bool ok[CPT];
  float wyr[CPT][8], accy[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    d0[j] = 8 * (j * nthr + (int)threadIdx.x);
    ok[j] = d0[j] < D;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      wyr[j][e] = 0.f;
      accy[j][e] = 0.f;
    }
    if (SW && ok[j]) load_w8(wy, d0[j], wyr[j]);
    if constexpr (PN) {
#pragma unroll
      for (int q = 0; q < N * 2; ++q) accx_s[(j * N * 2 + q) * nthr + threadIdx.x] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  // Every access below is a raw buffer access: a scalar descriptor per token
  // row, one 32-bit lane offset per chunk and the stream offset as a scalar
  // offset, which keeps the addresses out of the vector registers.  Lanes
  // past the end of the row (d0 ≥ D) take the lane offset 2^31: with a
  // stream offset (< 2^21) added, in the lane or the scalar offset, it stays
  // beyond every descriptor's size (at most N·D·4 < 2^21 bytes) without 32-bit
  // wrap-around, so those lanes read 0 and their stores are dropped.
  uint32_t vo[CPT], vw[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    vo[j] = ok[j] ? (uint32_t)d0[j] * B : kOffOut;
    vw[j] = ok[j] ? (uint32_t)d0[j] * 4u : kOffOut;
  }
  const Rsrc rwx = rsrc(wx, PN ? (uint32_t)K * 4u : 0u);

  int it = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x, ++it) {
    const int p = it & 1;
    float hp[N], hr[N][N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      hp[n] = H_post[t * N + n];
#pragma unroll
      for (int m = 0; m < N; ++m) hr[n][m] = H_res[(t * N + n) * N + m];
    }
    const int64_t xb = t * (int64_t)K;
    const Rsrc rx = rsrc(static_cast<const char*>(x) + xb * B, (uint32_t)K * B);
    const Rsrc rd = rsrc(static_cast<const char*>(dxn) + xb * B, (uint32_t)K * B);
    const Rsrc ryv = rsrc(static_cast<const char*>(y) + t * D * B, rowD);
    Pack8<IO> xr[CPT][N], dr[CPT][N], yr[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      yr[j].load(ryv, vo[j], 0);
#pragma unroll
      for (int n = 0; n < N; ++n) {
        dr[j][n].load(rd, vo[j], n * rowD);
        xr[j][n].load(rx, vo[j], n * rowD);
      }
    }

    float ry = 1.f;
    float gz[CPT][N][8];
    if constexpr (PN) {
      if constexpr (SW) {
        float ss[1] = {0.f};
#pragma unroll
        for (int j = 0; j < CPT; ++j)
#pragma unroll
          for (int e = 0; e < 8; ++e) ss[0] += yr[j][e] * yr[j][e];
        ry = __builtin_amdgcn_rsqf(lane_f(wg_sum<1, kMaxWaves>(ss, red1[p]), 0) / (float)D + eps);
      }
      // z as in the forward; it is computed twice (for the two sums, then for
      // g_z) rather than kept across the reduction, which would not fit in
      // registers next to dw_x
      float s2[2] = {0.f, 0.f};  // Σ z², Σ (w_x⊙dx_next)⊙z
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
          float w[8];
          load_w8(rwx, vw[j], (uint32_t)(n * D) * 4u, w);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float zz = z_at<N, IO, SW>(hp[n], hr[n], xr[j], yr[j][e], ry, wyr[j][e], e);
            s2[0] += zz * zz;
            s2[1] += (w[e] * dr[j][n][e]) * zz;
          }
        }
      }
      const float t2 = wg_sum<2, kMaxWaves>(s2, red2[p]);
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        yr[j].fence();
#pragma unroll
        for (int n = 0; n < N; ++n) {
          xr[j][n].fence();
          dr[j][n].fence();
        }
      }
      const float rz = __builtin_amdgcn_rsqf(lane_f(t2, 0) / (float)K + eps);
      const float c = rz * rz * rz * lane_f(t2, 1) / (float)K;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
#pragma unroll
        for (int n = 0; n < N; ++n) {
          float w[8], a[8];
          load_w8(rwx, vw[j], (uint32_t)(n * D) * 4u, w);
          float4& s0 = accx_s[((j * N + n) * 2) * nthr + threadIdx.x];
          float4& s1 = accx_s[((j * N + n) * 2 + 1) * nthr + threadIdx.x];
          const float4 a0 = s0, a1 = s1;
          a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
          a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float zz = z_at<N, IO, SW>(hp[n], hr[n], xr[j], yr[j][e], ry, wyr[j][e], e);
            const float d = dr[j][n][e];
            a[e] += (d * zz) * rz;
            gz[j][n][e] = rz * (w[e] * d) - c * zz;
          }
          s0 = make_float4(a[0], a[1], a[2], a[3]);
          s1 = make_float4(a[4], a[5], a[6], a[7]);
        }
      }
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        yr[j].fence();
#pragma unroll
        for (int n = 0; n < N; ++n) xr[j][n].fence();
      }
    } else {
#pragma unroll
      for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int n = 0; n < N; ++n)
#pragma unroll
          for (int e = 0; e < 8; ++e) gz[j][n][e] = dr[j][n][e];
    }

    // dx and the per-token sums
    const Rsrc rdx = rsrc(static_cast<char*>(dx) + xb * B, (uint32_t)K * B);
    float g[CPT][8];
    float acc[R3];
#pragma unroll
    for (int i = 0; i < R3; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
#pragma unroll
      for (int m = 0; m < N; ++m) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = 0.f;
#pragma unroll
          for (int n = 0; n < N; ++n) a += hr[n][m] * gz[j][n][e];
          o[e] = a;
        }
        store8b<IO>(rdx, vo[j], m * rowD, o);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = 0.f;
#pragma unroll
        for (int n = 0; n < N; ++n) a += hp[n] * gz[j][n][e];
        g[j][e] = a;
        const float yv = yr[j][e];
        const float yw = SW ? wyr[j][e] * yv : yv;
#pragma unroll
        for (int n = 0; n < N; ++n) {
#pragma unroll
          for (int m = 0; m < N; ++m) acc[n * N + m] += gz[j][n][e] * xr[j][m][e];
          acc[N * N + n] += gz[j][n][e] * yw;
        }
        if constexpr (SW) acc[kS] += a * yw;
        if constexpr (SW && !PN) acc[kY] += yv * yv;
      }
    }
    const float t3 = wg_sum<R3, kMaxWaves>(acc, red3[p]);
    if constexpr (SW && !PN) ry = __builtin_amdgcn_rsqf(lane_f(t3, kY) / (float)D + eps);
    // lanes of wave 0 write the coefficient gradients of this token
    if (threadIdx.x < N * N)
      dH_res[t * N * N + threadIdx.x] = t3;
    else if (threadIdx.x < kS)
      dH_post[t * N + threadIdx.x - N * N] = SW ? ry * t3 : t3;
    const float cy = SW ? ry * ry * ry * lane_f(t3, SW ? kS : 0) / (float)D : 0.f;
    const Rsrc rdy = rsrc(static_cast<char*>(dy) + t * D * B, rowD);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (SW) {
          const float yv = yr[j][e];
          o[e] = ry * (wyr[j][e] * g[j][e]) - cy * yv;
          accy[j][e] += (g[j][e] * yv) * ry;
        } else {
          o[e] = g[j][e];
        }
      }
      store8b<IO>(rdy, vo[j], 0, o);
    }
  }

  // this workgroup's row of partial weight gradients: [dw_y (D) | dw_x (N·D)]
  const int W = (SW ? D : 0) + (PN ? K : 0);
  float* row = part + (int64_t)blockIdx.x * W;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (!ok[j]) continue;
    if constexpr (SW) store_f8(row + d0[j], accy[j]);
    if constexpr (PN) {
#pragma unroll
      for (int n = 0; n < N; ++n) {
        float4* q = reinterpret_cast<float4*>(row + (SW ? D : 0) + n * D + d0[j]);
        q[0] = accx_s[((j * N + n) * 2) * nthr + threadIdx.x];
        q[1] = accx_s[((j * N + n) * 2 + 1) * nthr + threadIdx.x];
      }
    }
  }
}

// ---------------------------------------------- ten elements a thread ---
// The backward with the post-norm, N = 4, bf16, D = 10·nthr (nthr a multiple
// of 64, at most 512).  Its cost is vector-ALU issue, not memory: every state
// element passes through some fifty instructions (both norms, T = 4096,
// D = 5120: 70 M VALU instructions a call, 113 µs of SIMD time at perfect
// balance, by the SQ counters on MI355X).  Two things of the kernel above
// waste issue slots there: ten waves sit 3/3/2/2 on a CU's four SIMDs, so two
// SIMDs do half as much again as the others between barriers; and with
// ≤ 168 registers a wave it recomputes z after the second reduction and
// unpacks x and dx_next for every use.  Here eight waves (two a SIMD, up to
// 256 registers each) own ten elements of every row per thread, an 8-element
// chunk at 8·i and a 2-element chunk at 8·nthr + 2·i (16- and 4-byte accesses,
// 1 KB and 256 B runs per wave), and keep x and dx_next unpacked and z across
// the reduction.  The loop is pipelined as far as the registers allow: the
// next token's x and dx_next (and, without the sandwich norm, y) are loaded
// once this token's dx pass has consumed them and arrive under the last
// reduction and the dy pass; with the sandwich norm y runs one token further
// ahead and the next token's Σy² rides in this token's last reduction, which
// gives its r_y before it starts.  Arithmetic per element is the kernel
// above's, in the same order.
namespace e10 {

constexpr int kE = 10;
constexpr int kThreads = 512;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bload4(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kStream);
}
// 4-byte store, scalar offset 0 as for bstore16
__device__ __forceinline__ void bstore4(Rsrc r, uint32_t voff, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)voff, 0, kStream);
}

// Ten bf16 of a row as loaded: words 0–3 the 8-element chunk, word 4 the
// 2-element one.
struct Row10 {
  uint32_t w[5];
  __device__ __forceinline__ void load(Rsrc r, uint32_t vA, uint32_t vB, uint32_t soff) {
    const uint4 a = bload16<kStream>(r, vA, soff);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = bload4(r, vB, soff);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float operator[](int e) const {
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  }
  __device__ __forceinline__ void unpack(float (&v)[kE]) const {
#pragma unroll
    for (int e = 0; e < kE; ++e) v[e] = (*this)[e];
  }
};

// Ten fp32 weights: two 16-byte loads at wA and one 8-byte load at wB.
__device__ __forceinline__ void load_w10(Rsrc r, uint32_t wA, uint32_t wB, uint32_t soff, float (&v)[kE]) {
  const uint4 a = bload16(r, wA, soff), b = bload16(r, wA + 16, soff);
  const u32x2_t c = __builtin_amdgcn_raw_buffer_load_b64(r, (int)wB, (int)soff, 0);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  v[8] = __uint_as_float(c.x); v[9] = __uint_as_float(c.y);
}

// Ten values stored as bf16 (round to nearest even), stream offset `off` in
// the lane offset.
__device__ __forceinline__ void store10(Rsrc r, uint32_t vA, uint32_t vB, uint32_t off, const float (&v)[kE]) {
  bstore16<kStream>(r, vA + off, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
  bstore4(r, vB + off, pack_bf16x2(v[8], v[9]));
}

// Column of element e of thread i in a row: 8·i + e, then 8·nthr + 2·i + e − 8.
__device__ __forceinline__ int col(int e, int i, int nthr) { return e < 8 ? 8 * i + e : 8 * nthr + 2 * i + e - 8; }

// Dynamic LDS: the dw_x partial sums, float2 (n, q < 5) of thread i at
// [(n·5 + q)·nthr + i], so a wave's 8-byte accesses are contiguous.
constexpr size_t lds_bytes(int nthr) { return (size_t)4 * 5 * nthr * sizeof(float2); }

template <bool SW>
__global__ __launch_bounds__(kThreads) void post_stable_bwd10(
    const void* __restrict__ dxn, const void* __restrict__ x, const void* __restrict__ y,
    const float* __restrict__ wy, const float* __restrict__ H_post, const float* __restrict__ H_res,
    const float* __restrict__ wx, void* __restrict__ dx, void* __restrict__ dy,
    float* __restrict__ dH_post, float* __restrict__ dH_res, float* __restrict__ part, int64_t T,
    int D, float eps) {
  constexpr int N = 4, E = kE;
  // totals of the last reduction: dH_res[N²], <g_z[n], w_y⊙y or y>[N], then
  // with the sandwich norm Σ g⊙w_y⊙y and the next token's Σ y²
  constexpr int kS = N * N + N, kY = kS + 1;
  constexpr int R3 = kS + (SW ? 2 : 0);
  constexpr int kW = kThreads / kWave;
  __shared__ float red1[kW];
  __shared__ float red2[2][kW * 2];
  __shared__ float red3[2][kW * R3];
  extern __shared__ float2 accx2[];
  const int nthr = blockDim.x, tid = threadIdx.x;
  const int K = N * D;
  const uint32_t rowD = (uint32_t)D * 2u;  // bytes of one bf16 stream row
  const uint32_t vA = 16u * tid, vB = 16u * nthr + 4u * tid;  // bf16 row offsets
  const uint32_t wA = 32u * tid, wB = 32u * nthr + 8u * tid;  // fp32 row offsets
  float wyr[E], accy[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    wyr[e] = 0.f;
    accy[e] = 0.f;
  }
  if constexpr (SW) load_w10(rsrc(wy, (uint32_t)D * 4u), wA, wB, 0, wyr);
#pragma unroll
  for (int q = 0; q < N * 5; ++q) accx2[q * nthr + tid] = make_float2(0.f, 0.f);
  const Rsrc rwx = rsrc(wx, (uint32_t)K * 4u);

  Row10 xr[N], dr[N], yr, y1, y2;
  auto load_xd = [&](int64_t tt) {
    const Rsrc rx = rsrc(static_cast<const char*>(x) + tt * K * 2, (uint32_t)K * 2u);
    const Rsrc rd = rsrc(static_cast<const char*>(dxn) + tt * K * 2, (uint32_t)K * 2u);
#pragma unroll
    for (int n = 0; n < N; ++n) {
      dr[n].load(rd, vA, vB, n * rowD);
      xr[n].load(rx, vA, vB, n * rowD);
    }
  };
  auto load_y = [&](int64_t tt, Row10& yy) {
    yy.load(rsrc(static_cast<const char*>(y) + tt * D * 2, rowD), vA, vB, 0);
  };
  auto sum_y2 = [&](const Row10& yy) {
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) a += yy[e] * yy[e];
    return a;
  };
  const int64_t G = gridDim.x;
  float ry = 1.f;
  // the grid has at most T workgroups: every one has a first token
  load_y(blockIdx.x, yr);
  load_xd(blockIdx.x);
  if constexpr (SW) {
    if (blockIdx.x + G < T) load_y(blockIdx.x + G, y1);
    else y1.zero();
    const float ss[1] = {sum_y2(yr)};
    ry = __builtin_amdgcn_rsqf(lane_f(wg_sum<1, 0, false>(ss, red1), 0) / (float)D + eps);
  }

  int it = 0;
  for (int64_t t = blockIdx.x; t < T; t += G, ++it) {
    const int p = it & 1;
    const int64_t tn = t + G;
    float hp[N], hr[N][N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      hp[n] = H_post[t * N + n];
#pragma unroll
      for (int m = 0; m < N; ++m) hr[n][m] = H_res[(t * N + n) * N + m];
    }
    float xf[N][E], df[N][E];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      xr[n].unpack(xf[n]);
      dr[n].unpack(df[n]);
    }
    // z as in the forward (hc_post's fma order), kept for the second pass
    float yh[E];
#pragma unroll
    for (int e = 0; e < E; ++e) yh[e] = SW ? (yr[e] * ry) * wyr[e] : yr[e];
    float z[N][E];
    float s2[2] = {0.f, 0.f};  // Σ z², Σ (w_x⊙dx_next)⊙z
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float w[E];
      load_w10(rwx, wA, wB, (uint32_t)(n * D) * 4u, w);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float a = hp[n] * yh[e];
#pragma unroll
        for (int m = 0; m < N; ++m) a = __builtin_fmaf(hr[n][m], xf[m][e], a);
        z[n][e] = a;
        s2[0] += a * a;
        s2[1] += (w[e] * df[n][e]) * a;
      }
    }
    const float t2 = wg_sum<2, 0, false>(s2, red2[p]);
    const float rz = __builtin_amdgcn_rsqf(lane_f(t2, 0) / (float)K + eps);
    const float c = rz * rz * rz * lane_f(t2, 1) / (float)K;
    // g_z in place of z, and this token's share of dw_x
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float w[E], a[E];
      load_w10(rwx, wA, wB, (uint32_t)(n * D) * 4u, w);
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        const float2 v = accx2[(n * 5 + q) * nthr + tid];
        a[2 * q] = v.x;
        a[2 * q + 1] = v.y;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float d = df[n][e], zz = z[n][e];
        a[e] += (d * zz) * rz;
        z[n][e] = rz * (w[e] * d) - c * zz;
      }
#pragma unroll
      for (int q = 0; q < 5; ++q) accx2[(n * 5 + q) * nthr + tid] = make_float2(a[2 * q], a[2 * q + 1]);
    }
    // dx and the per-token sums
    const Rsrc rdx = rsrc(static_cast<char*>(dx) + t * K * 2, (uint32_t)K * 2u);
#pragma unroll
    for (int m = 0; m < N; ++m) {
      float o[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float a = 0.f;
#pragma unroll
        for (int n = 0; n < N; ++n) a += hr[n][m] * z[n][e];
        o[e] = a;
      }
      store10(rdx, vA, vB, m * rowD, o);
    }
    float g[E], acc[R3];
#pragma unroll
    for (int i = 0; i < R3; ++i) acc[i] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float a = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) a += hp[n] * z[n][e];
      g[e] = a;
      const float yv = yr[e];
      const float yw = SW ? wyr[e] * yv : yv;
#pragma unroll
      for (int n = 0; n < N; ++n) {
#pragma unroll
        for (int m = 0; m < N; ++m) acc[n * N + m] += z[n][e] * xf[m][e];
        acc[N * N + n] += z[n][e] * yw;
      }
      if constexpr (SW) acc[kS] += a * yw;
    }
    // the next token's loads, then the last reduction
    if (tn < T) {
      load_xd(tn);
      if constexpr (!SW) load_y(tn, y1);
    }
    if constexpr (SW) {
      if (tn + G < T) load_y(tn + G, y2);
      else y2.zero();
      acc[kY] = sum_y2(y1);
    }
    const float t3 = wg_sum<R3, 0, false>(acc, red3[p]);
    // lanes of wave 0 write the coefficient gradients of this token
    if (tid < N * N)
      dH_res[t * N * N + tid] = t3;
    else if (tid < kS)
      dH_post[t * N + tid - N * N] = SW ? ry * t3 : t3;
    const float cy = SW ? ry * ry * ry * lane_f(t3, kS) / (float)D : 0.f;
    float o[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if constexpr (SW) {
        const float yv = yr[e];
        o[e] = ry * (wyr[e] * g[e]) - cy * yv;
        accy[e] += (g[e] * yv) * ry;
      } else {
        o[e] = g[e];
      }
    }
    store10(rsrc(static_cast<char*>(dy) + t * D * 2, rowD), vA, vB, 0, o);
    if constexpr (SW) {
      ry = __builtin_amdgcn_rsqf(lane_f(t3, kY) / (float)D + eps);
      yr = y1;
      y1 = y2;
    } else {
      yr = y1;
    }
  }

  // this workgroup's row of partial weight gradients: [dw_y (D) | dw_x (N·D)]
  float* row = part + (int64_t)blockIdx.x * ((SW ? D : 0) + K);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int cl = col(e, tid, nthr);
    if constexpr (SW) row[cl] = accy[e];
#pragma unroll
    for (int n = 0; n < N; ++n) {
      const float2 v = accx2[(n * 5 + e / 2) * nthr + tid];
      row[(SW ? D : 0) + n * D + cl] = (e & 1) ? v.y : v.x;
    }
  }
}

}  // namespace e10

// dw[c] = Σ_{b<G} part[b][c], rows in order: 64 columns per workgroup, wave v
// adds rows v, v + 16, … in order, then the sixteen wave sums are added in
// wave order.  Columns [0, Dy) go to dwy, the rest to dwx.
__global__ __launch_bounds__(kSumWaves * kWave) void stable_wsum(const float* __restrict__ part, int G,
                                                                  int W, int Dy, float* __restrict__ dwy,
                                                                  float* __restrict__ dwx) {
  __shared__ float s[kSumWaves][kWave];
  const int lane = threadIdx.x & (kWave - 1), v = threadIdx.x / kWave;
  const int c = blockIdx.x * kWave + lane;
  float a = 0.f;
  if (c < W) {
    int b = v;
    for (; b + kSumWaves * 7 < G; b += kSumWaves * 8) {
      float r[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) r[u] = part[(int64_t)(b + kSumWaves * u) * W + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) a += r[u];
    }
    for (; b < G; b += kSumWaves) a += part[(int64_t)b * W + c];
  }
  s[v][lane] = a;
  __syncthreads();
  if (v == 0 && c < W) {
    float r = 0.f;
#pragma unroll
    for (int w = 0; w < kSumWaves; ++w) r += s[w][lane];
    if (c < Dy)
      dwy[c] = r;
    else
      dwx[c - Dy] = r;
  }
}

struct Shape {
  int cpt, nthr;
};

// Chunks per thread and threads per workgroup for D, or false if the token
// does not fit in registers (8·N·CPT > 32 state elements per thread).
bool shape_for(int N, int D, Shape& s) {
  const int chunks = D / 8;
  for (int cpt = 1; cpt <= 4; cpt *= 2) {
    if (N * cpt > 4) return false;
    const int per = (chunks + cpt - 1) / cpt;
    if (per <= kMaxThreads) {
      s.cpt = cpt;
      s.nthr = (per + kWave - 1) / kWave * kWave;
      return true;
    }
  }
  return false;
}

// Calls f(N, IO, CPT, SW, PN as integral constants) for the instantiated
// combinations (N·CPT ≤ 4, at least one norm on).
template <typename F>
bool dispatch(int N, int io, int cpt, bool sw, bool pn, F&& f) {
  bool done = false;
  dispatch_n(N, [&](auto n_) {
    constexpr int Nc = decltype(n_)::value;
    dispatch_io(io, [&](auto io_) {
      auto go_cpt = [&](auto c_) {
        constexpr int C = decltype(c_)::value;
        if constexpr (Nc * C <= 4) {
          if (sw && pn) f(n_, io_, c_, std::true_type{}, std::true_type{});
          else if (sw) f(n_, io_, c_, std::true_type{}, std::false_type{});
          else if (pn) f(n_, io_, c_, std::false_type{}, std::true_type{});
          else return;
          done = true;
        }
      };
      if (cpt == 1) go_cpt(std::integral_constant<int, 1>{});
      else if (cpt == 2) go_cpt(std::integral_constant<int, 2>{});
      else if (cpt == 4) go_cpt(std::integral_constant<int, 4>{});
    });
  });
  return done;
}

// Dynamic LDS of the backward: the dw_x partial sums of every thread.
size_t accx_lds_bytes(int N, int cpt, int nthr, bool pn) {
  return pn ? (size_t)cpt * N * 2 * nthr * sizeof(float4) : 0;
}

// The backward with ten elements a thread takes N = 4 in bf16 with the
// post-norm on, D = 10·nthr, nthr a multiple of 64 up to 512.
bool use_e10(const mhc_desc& d, bool pn) {
  return pn && d.N == 4 && d.io == kBF16 && d.D % (10 * kWave) == 0 && d.D <= e10::kE * e10::kThreads;
}

// Workgroups of the backward: as many as fit on the device at once, at most
// one per token.
int bwd_grid(const mhc_desc& d, bool sw, bool pn) {
  Shape s;
  if (!shape_for(d.N, d.D, s)) return 0;
  int per_cu = 0;
  if (use_e10(d, pn)) {
    const int nthr = d.D / e10::kE;
    const void* k = sw ? reinterpret_cast<const void*>(&e10::post_stable_bwd10<true>)
                       : reinterpret_cast<const void*>(&e10::post_stable_bwd10<false>);
    per_cu = occupancy_per_cu(k, nthr, e10::lds_bytes(nthr));
  } else {
    dispatch(d.N, d.io, s.cpt, sw, pn, [&](auto n_, auto io_, auto c_, auto sw_, auto pn_) {
      const void* k = reinterpret_cast<const void*>(
          &post_stable_bwd<decltype(n_)::value, decltype(io_)::value, decltype(c_)::value,
                           decltype(sw_)::value, decltype(pn_)::value>);
      per_cu = occupancy_per_cu(k, s.nthr, accx_lds_bytes(d.N, s.cpt, s.nthr, pn));
    });
  }
  if (per_cu < 1) per_cu = 1;
  const int64_t g = (int64_t)per_cu * device_cu_count();
  return (int)(d.T < g ? d.T : g);
}

}  // namespace stab

bool post_stable_supported(const mhc_desc& d) {
  stab::Shape s;
  return stab::shape_for(d.N, d.D, s);
}

size_t post_stable_bwd_workspace_bytes(const mhc_desc& d, bool sw, bool pn) {
  if (!sw && !pn) return 0;
  const int G = stab::bwd_grid(d, sw, pn);
  const size_t W = (sw ? (size_t)d.D : 0) + (pn ? (size_t)d.N * d.D : 0);
  return ((size_t)G * W * sizeof(float) + 255) & ~size_t(255);
}

hipError_t launch_post_stable(const mhc_desc& d, const void* x, const void* y, const float* wy,
                              const float* H_post, const float* H_res, const float* wx, void* x_next,
                              hipStream_t s) {
  const bool sw = wy != nullptr, pn = wx != nullptr;
  if (!sw && !pn) return launch_post(d, x, y, H_post, H_res, x_next, s);
  stab::Shape sh;
  if (!stab::shape_for(d.N, d.D, sh)) return hipErrorInvalidValue;
  const bool ok = stab::dispatch(d.N, d.io, sh.cpt, sw, pn, [&](auto n_, auto io_, auto c_, auto sw_, auto pn_) {
    MHC_LAUNCH((stab::post_stable_fwd<decltype(n_)::value, decltype(io_)::value, decltype(c_)::value,
                                              decltype(sw_)::value, decltype(pn_)::value>),
                       dim3((unsigned)d.T), dim3(sh.nthr), 0, s, x, y, wy, H_post, H_res, wx, x_next, d.D,
                       d.eps);
  });
  if (!ok) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_post_stable_bwd(const mhc_desc& d, const void* dxn, const void* x, const void* y,
                                  const float* wy, const float* H_post, const float* H_res,
                                  const float* wx, void* dx, void* dy, float* dwy, float* dwx,
                                  float* dH_post, float* dH_res, void* ws, hipStream_t s) {
  const bool sw = wy != nullptr, pn = wx != nullptr;
  if (!sw && !pn) return launch_post_bwd(d, dxn, x, y, H_post, H_res, dx, dy, dH_post, dH_res, s);
  stab::Shape sh;
  if (!stab::shape_for(d.N, d.D, sh)) return hipErrorInvalidValue;
  const int G = stab::bwd_grid(d, sw, pn);
  if (G < 1) return hipErrorInvalidValue;
  float* part = static_cast<float*>(ws);
  if (stab::use_e10(d, pn)) {
    const int nthr = d.D / stab::e10::kE;
    if (sw)
      MHC_LAUNCH(stab::e10::post_stable_bwd10<true>, dim3((unsigned)G), dim3(nthr), stab::e10::lds_bytes(nthr), s,
                 dxn, x, y, wy, H_post, H_res, wx, dx, dy, dH_post, dH_res, part, d.T, d.D, d.eps);
    else
      MHC_LAUNCH(stab::e10::post_stable_bwd10<false>, dim3((unsigned)G), dim3(nthr), stab::e10::lds_bytes(nthr), s,
                 dxn, x, y, wy, H_post, H_res, wx, dx, dy, dH_post, dH_res, part, d.T, d.D, d.eps);
  } else {
    const bool ok = stab::dispatch(d.N, d.io, sh.cpt, sw, pn, [&](auto n_, auto io_, auto c_, auto sw_, auto pn_) {
      MHC_LAUNCH((stab::post_stable_bwd<decltype(n_)::value, decltype(io_)::value, decltype(c_)::value,
                                                decltype(sw_)::value, decltype(pn_)::value>),
                         dim3((unsigned)G), dim3(sh.nthr), stab::accx_lds_bytes(d.N, sh.cpt, sh.nthr, pn), s,
                         dxn, x, y, wy, H_post, H_res, wx, dx, dy,
                         dH_post, dH_res, part, d.T, d.D, d.eps);
    });
    if (!ok) return hipErrorInvalidValue;
  }
  const int Dy = sw ? d.D : 0;
  const int W = Dy + (pn ? d.N * d.D : 0);
  MHC_LAUNCH(stab::stable_wsum, dim3((unsigned)((W + kWave - 1) / kWave)), dim3(stab::kSumWaves * kWave),
                     0, s, part, G, W, Dy, dwy, dwx);
  return hipGetLastError();
}

}  // namespace mhc
