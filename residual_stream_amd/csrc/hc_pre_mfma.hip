// hc_pre forward on the matrix cores (N = 4 streams, D a multiple of 32).
//
// The method (openPangu 2.0 analysis, §5.3 "mHC" formula block) needs, per
// token, the sum of squares and C = 24 projections of the 4·D-element state
// (one coalesced read), then gates, Sinkhorn and the collapse
// h = Σ_n H_pre[n]·x[n], which cannot start before the whole-token reduction.
//
// Layout on the chip: a workgroup of 8 waves owns a tile of TM tokens and keeps
// the tile's x in VGPRs (≈320 KB per CU) from the projection to the collapse,
// so x crosses HBM exactly once.  The projection x·φ runs on
// v_mfma_f32_16x16x32_bf16: the 16 A rows are TM tokens × R = 16/TM stream
// ranges, the 16 B columns are R ranges × TM logit columns, and only the
// diagonal range blocks of the 16×16 result are kept (the others pair x of one
// stream with φ rows of another and are ignored).  This keeps every lane's
// registers full of x while the tile is small enough to stay resident.  φ is
// pre-packed (phi_pack_kernel) into exactly the B-fragment order, as bf16 (hi),
// plus a bf16 residual (lo) for fp32 I/O so the product keeps ~16 mantissa bits.
//
// The k index of the contraction is permuted freely (the sum does not care) so
// that a lane's registers hold, for one token and 8 consecutive d, the values of
// R streams; the other N/R streams of the same (token, d) sit in lanes of the
// same 16-lane row, so the collapse is a register FMA plus one or two shuffles.
#include "mhc_coef.h"
#include "mhc_internal.h"

namespace mhc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfmaWaves = 8;
constexpr int kMfmaThreads = kMfmaWaves * kWave;
constexpr int kN4 = 4;
constexpr int kC4 = kN4 * kN4 + 2 * kN4;  // 24 logit columns
#ifndef PRE_RING_VGPRS
#define PRE_RING_VGPRS 36  // VGPRs per lane for in-flight φ fragments
#endif

template <int TM>
struct PreTile {
  static constexpr int R = 16 / TM;             // stream ranges per MFMA row block
  static constexpr int SPB = kN4 / R;           // MFMA k-steps per 32-wide d-block
  static constexpr int CG = (kC4 + TM - 1) / TM;  // B column groups covering 24 logits
};

// ---------------------------------------------------------------- φ pack ---
// phi_packed[((step·CG + cg)·PS + part)·64 + lane] = 8 bf16 (16 B): for lane l,
// column j = l%16 → (range j/TM, logit c = cg·TM + j%TM), k-group g = l/16 →
// φ[n·D + 32·dblk + 8g + v][c], v = 0..7, with step = dblk·SPB + sp and stream
// n = sp·R + j/TM.  part 0 = bf16(φ), part 1 = bf16(φ − part0) (fp32 I/O only).
template <int TM, int PS>
__global__ __launch_bounds__(256) void phi_pack_kernel(const float* __restrict__ phi,
                                                       uint4* __restrict__ out, int D,
                                                       int nsteps) {
  using P = PreTile<TM>;
  const int64_t total = (int64_t)nsteps * P::CG * PS * 64;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int lane = (int)(idx & 63);
  int64_t rest = idx >> 6;
  const int part = (int)(rest % PS);
  rest /= PS;
  const int cg = (int)(rest % P::CG);
  const int step = (int)(rest / P::CG);
  const int j = lane & 15, g = lane >> 4;
  const int c = cg * TM + (j % TM);
  const int sp = step % P::SPB, dblk = step / P::SPB;
  const int n = sp * P::R + j / TM;
  uint32_t w[4];
#pragma unroll
  for (int v = 0; v < 8; v += 2) {
    float f0 = 0.f, f1 = 0.f;
    if (c < kC4) {
      const int64_t k = (int64_t)n * D + 32 * dblk + 8 * g + v;
      f0 = phi[k * kC4 + c];
      f1 = phi[(k + 1) * kC4 + c];
    }
    uint32_t hw = pack_bf16x2(f0, f1);
    if (part == 1) hw = pack_bf16x2(f0 - bf16_lo(hw), f1 - bf16_hi(hw));
    w[v / 2] = hw;
  }
  out[idx] = make_uint4(w[0], w[1], w[2], w[3]);
}

// ------------------------------------------------------------ main kernel ---

// LDS per buffer: raw projection partials red[wave][range][token][32], sums
// of squares ss[wave][token], then per-token totals tot[token][32] (column 24
// holds the sum of squares).  Two buffers, so wave 0 can finish the previous
// tile's Sinkhorn while the other waves already reduce the next tile.
template <int TM>
struct PreLds {
  static constexpr int R = 16 / TM;
  static constexpr int kRed = kMfmaWaves * R * TM * 32;
  static constexpr int kSs = kMfmaWaves * TM;
  static constexpr int kTot = TM * 32;
  static constexpr int kBuf = kRed + kSs + kTot;
};

// Lane exchanges through DPP (a VALU operand modifier, no LDS round trip):
// quad_perm(1,0,3,2) swaps neighbours, quad_perm(2,3,0,1) swaps pairs,
// row_ror:n rotates each 16-lane row by n.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

// Sum over the lanes l, l±TM, l±2TM, ... of one 16-lane row; rotating by TM
// and its multiples visits exactly that orbit.  Result in every lane.
template <int TM>
__device__ __forceinline__ float row_orbit_sum(float v) {
  if constexpr (TM == 4) {
    v += dpp<kDppRowRor4>(v);
    v += dpp<kDppRowRor8>(v);
  } else if constexpr (TM == 8) {
    v += dpp<kDppRowRor8>(v);
  }
  return v;
}

// A zero the compiler cannot see through, produced once per tile, so that
// tile-invariant address arithmetic stays inside the loop (next to its loads)
// instead of being hoisted out of it and pinning registers for the whole kernel.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

// Raw buffer resource over `bytes` bytes from `base`; loads at byte offsets
// (VGPR offset + immediate) beyond `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// voff: per-lane offset (VGPR); soff: wave-uniform offset (SGPR), kept out
// of VGPRs so that unrolled loads share one address register.
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff = 0) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// 1/(1+e^-z) with the hardware reciprocal (1 ulp) instead of the IEEE division sequence.
__device__ __forceinline__ float fast_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + expf(-z)); }

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// NB = 32-wide d-blocks per wave, the same for all 8 waves: D = 256·NB.
template <int IO, int TM, int NB>
__global__ __launch_bounds__(kMfmaThreads, 1) void hc_pre_mfma_kernel(
    const void* __restrict__ x, const uint4* __restrict__ phip, const float* __restrict__ bias,
    void* __restrict__ h, float* __restrict__ H_pre, float* __restrict__ H_post,
    float* __restrict__ H_res, int64_t T, int iters, float eps, float a_pre, float a_post,
    float a_res, const float* __restrict__ alpha_dev) {
  if (alpha_dev != nullptr) {  // the gate scalars are held on the device (trained α)
    a_pre = alpha_dev[0];
    a_post = alpha_dev[1];
    a_res = alpha_dev[2];
  }
  using P = PreTile<TM>;
  constexpr int R = P::R, SPB = P::SPB, CG = P::CG;
  constexpr int PS = IO == kF32 ? 2 : 1;
  constexpr int XW = IO == kF32 ? 2 : 1;  // uint4 words per A fragment (fp32 keeps full x)
  constexpr int E = IO == kF32 ? 4 : 2;   // bytes per element
  constexpr int D = 256 * NB;
  constexpr int K = kN4 * D;
  constexpr int NS = NB * SPB;                        // k-steps per wave
  constexpr uint32_t kStepBytes = CG * PS * 64 * 16;  // packed φ per k-step
  constexpr int LA = (PRE_RING_VGPRS / (CG * PS * 4)) > 1 ? (PRE_RING_VGPRS / (CG * PS * 4)) : 1;  // φ look-ahead
  constexpr int L = PreLds<TM>::kBuf;
  __shared__ float lds[2 * L];
  __shared__ float bias_s[32];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b0 = wave * NB;   // first d-block of this wave
  const int64_t ntiles = (T + TM - 1) / TM;
  const float rK = 1.0f / (float)K;

  // φ of this wave's d-blocks: one resource, lane offset + per-step constants.
  const __amdgpu_buffer_rsrc_t rphi =
      make_rsrc(phip + (int64_t)b0 * SPB * (CG * PS * 64), NS * kStepBytes);

  // bias in LDS: reading it there never waits behind the x loads in flight
  if (threadIdx.x < 32) bias_s[threadIdx.x] = threadIdx.x < kC4 ? bias[threadIdx.x] : 0.f;
  __syncthreads();

  uint4 xr[NB][SPB][XW];
  int buf = 0;
  int64_t prev_tile = -1;

  for (int64_t tile = blockIdx.x; tile < ntiles || prev_tile >= 0; tile += gridDim.x) {
    const bool have = tile < ntiles;
    const int z = opaque_zero();
    // Lane-derived values are rebuilt from the lane id each tile (a few VALU ops)
    // rather than kept live across the loop beside the 160 VGPRs of x.
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, (unsigned)z));
    const int tid = wave * 64 + lane;
    const int row = lane & 15;  // MFMA A row
    const int g = lane >> 4;    // k group (8 consecutive d)
    const int tt = row % TM;    // token within the tile
    const int rr = row / TM;    // stream range of this lane's A rows
    // x offset of this lane inside a tile (bytes): token tt, stream range rr, group g
    const uint32_t xlane = (uint32_t)(((tt * kN4 + rr) * D + 32 * b0 + 8 * g) * E);
    const int64_t t0 = tile * TM;
    const int64_t my_t = t0 + tt;
    const bool tok_ok = have && my_t < T;

    // ---- 1. issue every x load of this tile (kept in VGPRs until the
    // collapse); rows past the last token fall outside the resource and read
    // as zero.
    if (have) {
      const int64_t valid = (T - t0) < TM ? (T - t0) : TM;
      const __amdgpu_buffer_rsrc_t rx =
          make_rsrc(static_cast<const char*>(x) + t0 * (int64_t)K * E, (uint32_t)(valid * K * E));
      const uint32_t xo = xlane;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int sp = 0; sp < SPB; ++sp)
#pragma unroll
          for (int q = 0; q < XW; ++q)
            xr[b][sp][q] = ld16(rx, xo + (uint32_t)(32 * b * E + 16 * q), (uint32_t)(sp * R * D * E) + z);
    }

    // ---- 2. wave 0 finishes the previous tile: H_post, Sinkhorn, stores of the
    // coefficients.  LDS reads and DPP only, so nothing waits for the loads.
    if (prev_tile >= 0 && wave == 0) {
      const float* tot = lds + (buf ^ 1) * L + PreLds<TM>::kRed + PreLds<TM>::kSs;
      const int tk = (lane / kN4) % TM, i = lane % kN4;  // token, H_res row
      const int64_t t = prev_tile * TM + tk;
      const float rstd = __builtin_amdgcn_rsqf(tot[tk * 32 + kC4] * rK + eps);
      const float lp = a_pre * (rstd * tot[tk * 32 + i]) + bias_s[i];
      const float lq = a_post * (rstd * tot[tk * 32 + kN4 + i]) + bias_s[kN4 + i];
      float m[kN4], mx = -__builtin_huge_valf();
#pragma unroll
      for (int j = 0; j < kN4; ++j) {
        const int c = 2 * kN4 + i * kN4 + j;
        m[j] = a_res * (rstd * tot[tk * 32 + c]) + bias_s[c];
        mx = fmaxf(mx, m[j]);
      }
#pragma unroll
      for (int j = 0; j < kN4; ++j) m[j] = expf(m[j] - mx);
      for (int it = 0; it < iters; ++it) {
        const float rinv = __builtin_amdgcn_rcpf((m[0] + m[1]) + (m[2] + m[3]));
#pragma unroll
        for (int j = 0; j < kN4; ++j) m[j] *= rinv;
#pragma unroll
        for (int j = 0; j < kN4; ++j) {
          // column sum over the 4 lanes (rows) of this token
          const float s1 = m[j] + dpp<kDppQuadXor1>(m[j]);
          const float s = s1 + dpp<kDppQuadXor2>(s1);
          m[j] *= __builtin_amdgcn_rcpf(s);
        }
      }
      if (lane < TM * kN4 && t < T) {
        H_pre[t * kN4 + i] = fast_sigmoid(lp);
        H_post[t * kN4 + i] = 2.0f * fast_sigmoid(lq);
        reinterpret_cast<float4*>(H_res)[t * kN4 + i] = make_float4(m[0], m[1], m[2], m[3]);
      }
    }
    if (!have) break;

    // ---- 3. projection on the matrix cores + sum of squares.  The B fragments
    // (φ, L2-resident) stream through a ring of LA k-steps so that several L2
    // round trips are in flight per wave.
    f32x4_t acc[CG];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) acc[cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ss = 0.f;
    {
      const uint32_t po = (uint32_t)(lane * 16);
      uint4 ring[LA][CG * PS];
#pragma unroll
      for (int s0 = 0; s0 < LA; ++s0)
#pragma unroll
        for (int f = 0; f < CG * PS; ++f) ring[s0][f] = ld16(rphi, po + f * 1024, s0 * kStepBytes + z);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int b = st / SPB, sp = st % SPB, slot = st % LA;
        uint4 cur[CG * PS];
#pragma unroll
        for (int f = 0; f < CG * PS; ++f) cur[f] = ring[slot][f];
        if (st + LA < NS) {
#pragma unroll
          for (int f = 0; f < CG * PS; ++f)
            ring[slot][f] = ld16(rphi, po + f * 1024, (st + LA) * kStepBytes + z);
        }
        // keep the look-ahead loads here: without this fence the scheduler sinks
        // them next to their use and only one L2 round trip is in flight
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (IO == kF32) {
          float v[8];
          const uint4 a0 = xr[b][sp][0], a1 = xr[b][sp][1];
          v[0] = __uint_as_float(a0.x); v[1] = __uint_as_float(a0.y);
          v[2] = __uint_as_float(a0.z); v[3] = __uint_as_float(a0.w);
          v[4] = __uint_as_float(a1.x); v[5] = __uint_as_float(a1.y);
          v[6] = __uint_as_float(a1.z); v[7] = __uint_as_float(a1.w);
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // x = hi + lo to ~16 mantissa bits: both halves exact in bf16
            hi[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
            lo[q] = pack_bf16x2(v[2 * q] - bf16_lo(hi[q]), v[2 * q + 1] - bf16_hi(hi[q]));
            ss += v[2 * q] * v[2 * q] + v[2 * q + 1] * v[2 * q + 1];
          }
          const uint4 ahi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          const uint4 alo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) {
            acc[cg] = mfma_bf16(ahi, cur[cg * PS + 0], acc[cg]);
            acc[cg] = mfma_bf16(ahi, cur[cg * PS + 1], acc[cg]);
            acc[cg] = mfma_bf16(alo, cur[cg * PS + 0], acc[cg]);
          }
        } else {
          const uint4 a = xr[b][sp][0];
          const uint32_t wv[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float lo = bf16_lo(wv[q]), hi = bf16_hi(wv[q]);
            ss += lo * lo + hi * hi;
          }
#pragma unroll
          for (int cg = 0; cg < CG; ++cg) acc[cg] = mfma_bf16(a, cur[cg], acc[cg]);
        }
      }
    }

    // ---- 4. partials to LDS (diagonal range blocks only); sum of squares over
    // the lanes of one token (row orbit, then the four 16-lane rows)
    float* rb = lds + buf * L;
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 4 * g + q;  // D row held by this lane
        const int j = row;        // D column held by this lane
        const int c = cg * TM + (j % TM);
        if ((i / TM) == (j / TM) && c < kC4)
          rb[((wave * R + i / TM) * TM + (i % TM)) * 32 + c] = acc[cg][q];
      }
    }
    ss = row_orbit_sum<TM>(ss);
    ss += __shfl_xor(ss, 16, kWave);
    ss += __shfl_xor(ss, 32, kWave);
    if (lane < TM) rb[PreLds<TM>::kRed + wave * TM + lane] = ss;
    __syncthreads();
    // per-token totals in a fixed order (waves, then ranges)
    float* tot = rb + PreLds<TM>::kRed + PreLds<TM>::kSs;
    if (tid < TM * 32) {
      const int tk = tid / 32, c = tid % 32;
      float a = 0.f;
      if (c < kC4) {
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w)
#pragma unroll
          for (int r = 0; r < R; ++r) a += rb[((w * R + r) * TM + tk) * 32 + c];
      } else if (c == kC4) {
#pragma unroll
        for (int w = 0; w < kMfmaWaves; ++w) a += rb[PreLds<TM>::kRed + w * TM + tk];
      }
      tot[tid] = a;
    }
    __syncthreads();

    // ---- 5. H_pre of this lane's token, then the collapse from registers
    float hpre[kN4];
    {
      const float rstd = __builtin_amdgcn_rsqf(tot[tt * 32 + kC4] * rK + eps);
#pragma unroll
      for (int n = 0; n < kN4; ++n) hpre[n] = fast_sigmoid(a_pre * (rstd * tot[tt * 32 + n]) + bias_s[n]);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float o[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) o[v] = 0.f;
#pragma unroll
      for (int sp = 0; sp < SPB; ++sp) {
        const float hw = hpre[sp * R + rr];
        if constexpr (IO == kF32) {
          const uint4 a0 = xr[b][sp][0], a1 = xr[b][sp][1];
          o[0] += hw * __uint_as_float(a0.x); o[1] += hw * __uint_as_float(a0.y);
          o[2] += hw * __uint_as_float(a0.z); o[3] += hw * __uint_as_float(a0.w);
          o[4] += hw * __uint_as_float(a1.x); o[5] += hw * __uint_as_float(a1.y);
          o[6] += hw * __uint_as_float(a1.z); o[7] += hw * __uint_as_float(a1.w);
        } else {
          const uint4 a = xr[b][sp][0];
          o[0] += hw * bf16_lo(a.x); o[1] += hw * bf16_hi(a.x);
          o[2] += hw * bf16_lo(a.y); o[3] += hw * bf16_hi(a.y);
          o[4] += hw * bf16_lo(a.z); o[5] += hw * bf16_hi(a.z);
          o[6] += hw * bf16_lo(a.w); o[7] += hw * bf16_hi(a.w);
        }
      }
      // add the other ranges' streams (lanes row ± TM·k in the same 16-lane row)
#pragma unroll
      for (int v = 0; v < 8; ++v) o[v] = row_orbit_sum<TM>(o[v]);
      // range rr stores its 8/R share of the 8 d values
      constexpr int share = 8 / R;
      float sv[share];
#pragma unroll
      for (int v = 0; v < share; ++v) {
        float pick = o[v];
#pragma unroll
        for (int r = 1; r < R; ++r)
          if (rr == r) pick = o[r * share + v];
        sv[v] = pick;
      }
      if (tok_ok) {
        const int64_t e = my_t * (int64_t)D + 32 * (b0 + b) + 8 * g + rr * share;
        if constexpr (IO == kF32) {
          float* hp = static_cast<float*>(h) + e;
          if constexpr (share == 8) {
            reinterpret_cast<float4*>(hp)[0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
            reinterpret_cast<float4*>(hp)[1] = make_float4(sv[4], sv[5], sv[6], sv[7]);
          } else if constexpr (share == 4) {
            *reinterpret_cast<float4*>(hp) = make_float4(sv[0], sv[1], sv[2], sv[3]);
          } else {
            *reinterpret_cast<float2*>(hp) = make_float2(sv[0], sv[1]);
          }
        } else {
          uint16_t* hp = static_cast<uint16_t*>(h) + e;
          if constexpr (share == 8) {
            *reinterpret_cast<uint4*>(hp) = make_uint4(pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]),
                                                       pack_bf16x2(sv[4], sv[5]), pack_bf16x2(sv[6], sv[7]));
          } else if constexpr (share == 4) {
            *reinterpret_cast<uint2*>(hp) = make_uint2(pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3]));
          } else {
            *reinterpret_cast<uint32_t*>(hp) = pack_bf16x2(sv[0], sv[1]);
          }
        }
      }
    }
    prev_tile = tile;
    buf ^= 1;
  }
}

// ------------------------------------------------------------------ host ---

struct PreConfig {
  int tm = 0;  // 0: not eligible for the matrix-core kernel
  int nsteps = 0, cg = 0, ps = 0;
};

static PreConfig pick_pre(const mhc_desc& d) {
  PreConfig pc;
  if (d.N != 4 || d.D % 256 != 0) return pc;
  const int ndb = d.D / 32;
  const int per_wave = ndb / kMfmaWaves;
  if (d.io == kBF16) {
    if (per_wave == 10) pc.tm = 16;
    else if (per_wave == 20) pc.tm = 8;
    pc.ps = 1;
  } else {
    if (per_wave == 10) pc.tm = 8;
    else if (per_wave == 20) pc.tm = 4;
    pc.ps = 2;
  }
  if (pc.tm == 0) return pc;
  const int R = 16 / pc.tm, spb = 4 / R;
  pc.nsteps = ndb * spb;
  pc.cg = (kC4 + pc.tm - 1) / pc.tm;
  return pc;
}

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t pre_workspace_bytes(const mhc_desc& d) {
  if (pre_decode_eligible(d)) return pre_decode_workspace_bytes(d);
  if (pre_tile_eligible(d)) return pre_tile_workspace_bytes(d);
  const PreConfig pc = pick_pre(d);
  if (pc.tm == 0) return 0;
  return align256((size_t)pc.nsteps * pc.cg * pc.ps * 64 * sizeof(uint4));
}

size_t post_pre_workspace_bytes(const mhc_desc& d) { return pre_workspace_bytes(d); }

hipError_t launch_pre_generic(const mhc_desc& d, const void* x, const float* phi,
                              const float* bias, void* h, float* H_pre, float* H_post,
                              float* H_res, hipStream_t s);

template <int IO, int TM, int NB>
static hipError_t launch_mfma(const mhc_desc& d, const PreConfig& pc, const void* x,
                              const float* phi, const float* bias, void* h, float* H_pre,
                              float* H_post, float* H_res, void* ws, hipStream_t s) {
  constexpr int PS = IO == kF32 ? 2 : 1;
  uint4* phip = static_cast<uint4*>(ws);
  const int64_t npack = (int64_t)pc.nsteps * pc.cg * PS * 64;
  MHC_LAUNCH((phi_pack_kernel<TM, PS>), dim3((unsigned)((npack + 255) / 256)), dim3(256),
                     0, s, phi, phip, d.D, pc.nsteps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ntiles = (d.T + TM - 1) / TM;
  const int cus = device_cu_count();
  const int64_t grid = ntiles < cus ? ntiles : cus;
  MHC_LAUNCH((hc_pre_mfma_kernel<IO, TM, NB>), dim3((unsigned)grid), dim3(kMfmaThreads), 0,
                     s, x, phip, bias, h, H_pre, H_post, H_res, (int64_t)d.T,
                     d.sinkhorn_iters, d.eps, d.alpha_pre, d.alpha_post, d.alpha_res, d.alpha);
  return hipGetLastError();
}

hipError_t launch_pre(const mhc_desc& d, const void* x, const float* phi, const float* bias,
                      void* h, float* H_pre, float* H_post, float* H_res, void* ws,
                      hipStream_t s) {
  if (pre_decode_eligible(d)) return launch_pre_decode(d, x, phi, bias, h, H_pre, H_post, H_res, ws, s);
  const PreConfig pc = pick_pre(d);
  if (pre_tile_eligible(d)) return launch_pre_tile(d, x, phi, bias, h, H_pre, H_post, H_res, ws, s);
  if (pc.tm == 0) return launch_pre_generic(d, x, phi, bias, h, H_pre, H_post, H_res, s);
  if (d.io == kBF16) {
    if (pc.tm == 16) return launch_mfma<kBF16, 16, 10>(d, pc, x, phi, bias, h, H_pre, H_post, H_res, ws, s);
    return launch_mfma<kBF16, 8, 20>(d, pc, x, phi, bias, h, H_pre, H_post, H_res, ws, s);
  }
  if (pc.tm == 8) return launch_mfma<kF32, 8, 10>(d, pc, x, phi, bias, h, H_pre, H_post, H_res, ws, s);
  return launch_mfma<kF32, 4, 20>(d, pc, x, phi, bias, h, H_pre, H_post, H_res, ws, s);
}

hipError_t launch_post_pre(const mhc_desc& d, const void* x, const void* y, const float* H_post_in,
                           const float* H_res_in, void* x_next, const float* phi, const float* bias,
                           void* h, float* H_pre, float* H_post, float* H_res, void* ws, hipStream_t s) {
  // x_next keeps the default cache policy here: hc_pre reads it next
  const hipError_t e = launch_post(d, x, y, H_post_in, H_res_in, x_next, s, true);
  if (e != hipSuccess) return e;
  return launch_pre(d, x_next, phi, bias, h, H_pre, H_post, H_res, ws, s);
}

}  // namespace mhc
