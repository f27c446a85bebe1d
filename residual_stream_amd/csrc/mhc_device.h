// Device-side helpers shared by the mHC kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mhc {

constexpr int kWave = 64;

enum Io : int { kF32 = 0, kBF16 = 1 };

template <int IO>
struct IoT;
template <>
struct IoT<kF32> {
  using elem = float;
  static constexpr int bytes = 4;
};
template <>
struct IoT<kBF16> {
  using elem = uint16_t;
  static constexpr int bytes = 2;
};

// bf16 → fp32 is exact: the 16 bits are the top half of the fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 → bf16 with the hardware converter (round to nearest even, NaN stays
// NaN); two values per instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }
// The parts of (lo, hi) that their bf16 pair w = pack_bf16x2(lo, hi) leaves
// out, rounded to bf16 in turn: with it, a value is carried as two bf16
// parts whose sum keeps about 16 mantissa bits.
__device__ __forceinline__ uint32_t pack_bf16x2_rest(float lo, float hi, uint32_t w) {
  return pack_bf16x2(lo - bf16_lo(w), hi - bf16_hi(w));
}
__device__ __forceinline__ uint4 pack_bf16x8_rest(const float v[8], uint4 w) {
  return make_uint4(pack_bf16x2_rest(v[0], v[1], w.x), pack_bf16x2_rest(v[2], v[3], w.y),
                    pack_bf16x2_rest(v[4], v[5], w.z), pack_bf16x2_rest(v[6], v[7], w.w));
}

// Eight consecutive elements starting at element index `i` (i % 8 == 0,
// 16-byte aligned base), widened to fp32.
template <int IO>
__device__ __forceinline__ void load8(const void* base, int64_t i, float v[8]) {
  if constexpr (IO == kF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + i);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + i);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
}

template <int IO>
__device__ __forceinline__ void store8(void* base, int64_t i, const float v[8]) {
  if constexpr (IO == kF32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + i);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 w;
    w.x = pack_bf16x2(v[0], v[1]);
    w.y = pack_bf16x2(v[2], v[3]);
    w.z = pack_bf16x2(v[4], v[5]);
    w.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + i) = w;
  }
}

// load8 / store8 with the non-temporal hint (global_load/store … nt) for bf16
// streams, for the streaming hc_post kernels: measured on MI355X, the hint
// takes hc_post from ≈75 to ≈65 µs and its backward from ≈112 to ≈101 µs
// (≈82 to ≈72 µs without dx) at T = 4096, N = 4, D = 5120, bf16.  fp32
// streams keep the default policy (the hint slowed the fp32 backward).  The split-K hc_pre and the
// hc_pre backward passes keep the default policy: there the hint cost more
// than it gained (the next call re-reads the same tensors while they are
// still cached).
template <int IO>
__device__ __forceinline__ void load8_stream(const void* base, int64_t i, float v[8]) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(static_cast<const char*>(base) + i * IoT<IO>::bytes);
  if constexpr (IO == kF32) {
    load8<IO>(base, i, v);
  } else {
    const u32x4_t w = __builtin_nontemporal_load(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
}

template <int IO>
__device__ __forceinline__ void store8_stream(void* base, int64_t i, const float v[8]) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t* p = reinterpret_cast<u32x4_t*>(static_cast<char*>(base) + i * IoT<IO>::bytes);
  if constexpr (IO == kF32) {
    store8<IO>(base, i, v);
  } else {
    __builtin_nontemporal_store(u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                        pack_bf16x2(v[6], v[7])}, p);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum `n` per-thread values over the block; the totals land in red[0..n) for
// every thread.  `red` needs n * (blockDim.x / 64) floats of LDS.  Fixed
// order: butterfly within each wave, then waves in index order.
template <int n>
__device__ __forceinline__ void block_sum(float (&v)[n], float* red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
#pragma unroll
  for (int i = 0; i < n; ++i) {
    float s = wave_sum(v[i]);
    if (lane == 0) red[wave * n + i] = s;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += red[w * n + i];
    red[(nw - 1) * n + i] = s;  // last wave's slot holds the total (read after the barrier)
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < n; ++i) v[i] = red[(nw - 1) * n + i];
  __syncthreads();
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  // rows outside ROWS read 0
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Total of v over the 64 lanes of a wave, left in lane 63: sums over 2, 4, 8
// and 16 lanes by DPP (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror: each lane adds its partner's partial sum), then
// row_bcast:15 into rows 1 and 3 and row_bcast:31 into rows 2 and 3, so lane 63
// holds (r3 + r2) + (r1 + r0).  No LDS round trip, so the sums of many values
// pipeline.
__device__ __forceinline__ float wave_total63(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  v += dpp_f<0x142, 0xA>(v);
  v += dpp_f<0x143, 0xC>(v);
  return v;
}

// Wave totals of R ≤ 32 values at once, transposed: each step pairs every
// lane with a partner whose partial sums cover other lanes, and every lane
// keeps half of its values, adding the partner's partial of that half.  Lanes
// l and l ^ 32 by permlane32_swap (lanes < 32 keep values i < 16), l and
// l ^ 16 by permlane16_swap, then the partners of the single-value sum above
// (row_mirror, row_half_mirror, quad_perm [2,3,0,1], quad_perm [1,0,3,2]).
// Lane l ends with the wave's total of value l >> 1 (lanes l and l ^ 1
// alike): about 70 instructions for 32 values, against ten a value one by
// one.
template <int R>
__device__ __forceinline__ float wave_sums_transposed(const float (&v)[R]) {
  static_assert(R <= 32, "two lanes a value");
  const int lane = threadIdx.x & (kWave - 1);
  float a[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) a[i] = i < R ? v[i] : 0.f;
  float b[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[i]), __float_as_uint(a[i + 16]), false, false);
    b[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(b[i]), __float_as_uint(b[i + 8]), false, false);
    c[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  float d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t0 = c[i] + dpp_f<0x140>(c[i]), t1 = c[i + 4] + dpp_f<0x140>(c[i + 4]);
    d[i] = (lane & 8) ? t1 : t0;
  }
  float e[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float t0 = d[i] + dpp_f<0x141>(d[i]), t1 = d[i + 2] + dpp_f<0x141>(d[i + 2]);
    e[i] = (lane & 4) ? t1 : t0;
  }
  const float t0 = e[0] + dpp_f<0x4E>(e[0]), t1 = e[1] + dpp_f<0x4E>(e[1]);
  const float f = (lane & 2) ? t1 : t0;
  return f + dpp_f<0xB1>(f);
}

// Sum of R ≤ 64 per-thread values over the workgroup in a fixed order (each
// wave's total, then the waves in index order).  Returns the totals spread
// over the lanes: lane i of every wave holds total i (i < R).  `red` holds
// (blockDim.x / 64)·R floats.  One barrier; a caller that reduces again into
// the same buffer alternates between two buffers, so that no wave can
// overwrite partial sums another wave has not read yet.  MAXW bounds the
// caller's waves per workgroup, so that the waves' partial sums are read all
// at once; MAXW = 0 reads them one by one, and TRANSPOSED = false takes the
// wave totals one value at a time: both use fewer registers, which a kernel
// at the register limit measured faster with (MI355X).
template <int R, int MAXW = 1024 / kWave, bool TRANSPOSED = true>
__device__ __forceinline__ float wg_sum(const float (&v)[R], float* red) {
  static_assert(R <= kWave, "one value per lane");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave, nw = blockDim.x / kWave;
  if constexpr (TRANSPOSED && R >= 8 && R <= 32) {
    const float t = wave_sums_transposed<R>(v);
    if (!(lane & 1) && (lane >> 1) < R) red[wave * R + (lane >> 1)] = t;
  } else {
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const float t = lane_f(wave_total63(v[i]), kWave - 1);
      mine = lane == i ? t : mine;
    }
    if (lane < R) red[wave * R + lane] = mine;
  }
  __syncthreads();
  float s = 0.f;
  if (lane < R) {
    if constexpr (MAXW == 0) {
      for (int w = 0; w < nw; ++w) s += red[w * R + lane];
    } else {
      // every load in flight at once (rows past the last wave re-read it and
      // add nothing)
      float p[MAXW];
#pragma unroll
      for (int w = 0; w < MAXW; ++w) p[w] = red[(w < nw ? w : nw - 1) * R + lane];
#pragma unroll
      for (int w = 0; w < MAXW; ++w) s += w < nw ? p[w] : 0.f;
    }
  }
  return s;
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

// Calls f(std::integral_constant<int, N>) for the supported stream counts.
template <typename F>
__host__ bool dispatch_n(int n, F&& f) {
  switch (n) {
    case 1: f(std::integral_constant<int, 1>{}); return true;
    case 2: f(std::integral_constant<int, 2>{}); return true;
    case 4: f(std::integral_constant<int, 4>{}); return true;
    case 8: f(std::integral_constant<int, 8>{}); return true;
    default: return false;
  }
}
template <typename F>
__host__ bool dispatch_io(int io, F&& f) {
  switch (io) {
    case kF32: f(std::integral_constant<int, kF32>{}); return true;
    case kBF16: f(std::integral_constant<int, kBF16>{}); return true;
    default: return false;
  }
}

}  // namespace mhc
