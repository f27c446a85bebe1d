// hc_pre backward, tiled (N = 4, D a multiple of 256): the matrix cores for
// bf16 I/O, the fp32 vector ALUs for fp32 I/O.
//
// Exact derivative of the openPangu 2.0 analysis §5.3 formula block, with the
// forward recomputed from x (Ascend mHC Triton article, intra-layer recompute
// paragraph).  Three passes:
//
//  1. bwd_proj_kernel — split-K reduction.  A persistent workgroup keeps one
//     d-slice of φ (all four streams) in registers as bf16 high and low parts
//     (φ = hi + lo: x is exact in bf16, so x·hi + x·lo keeps fp32 accuracy)
//     and streams x and dh for a contiguous token range: per (token, slice) it writes the raw
//     projections x·φ (matrix cores), the sum of squares and <dh, x[n]>.
//  2. bwd_coef_kernel — per token, sixteen lanes (one per H_res entry): sums the
//     slices, recomputes rstd, logits, gates and the Sinkhorn rounds (keeping
//     the row/column scalings u, v of every round in LDS), walks the rounds
//     backwards and emits G = rstd·α⊙dℓ (the token's factor in dφ and in
//     dx̄ = G·φᵀ), β = rstd³·(dq·p)/K, H_pre, dℓ and the dα terms.
//  3. bwd_dx_kernel — per k-slice: dx += G·φᵀ − β·x + H_pre[n]·dh (matrix
//     cores, φ slice in registers) and the partial dφ = Σ_t x_tᵀ G_t over its
//     token range (matrix cores on an LDS-transposed copy of the x tile); G
//     enters the matrix cores as bf16 high and low parts, so dφ keeps fp32
//     accuracy; φ enters G·φᵀ rounded to bf16 (an error of the order of the
//     bf16 rounding of the dx that product is added to).
// A final kernel sums the dφ partials and the per-16-token dbias / dα rows
// (fixed orders).
#include "mhc_coef.h"
#include "mhc_internal.h"

namespace mhc {
namespace bwdm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kN = 4;
constexpr int kC = kN * kN + 2 * kN;  // 24
constexpr int kPartStride = 32;       // floats per (slice, token): p[24], ss, dhp[4], pad
constexpr int kSliceD = 256;          // granularity of D for this path

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
template <int POLICY = 0>
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, POLICY);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Stores of dx, the pass's output, written once: bf16 with the non-temporal
// hint (measured on MI355X: the calls that follow run faster when dx does not
// linger in the caches), fp32 with the default policy.
template <int POLICY = 2>
__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint4 v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)voff, 0, POLICY);
}

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ------------------------------------------------------------- pass 1 ---
// Persistent split-K reduction.  A workgroup = W waves walks a contiguous
// token range in 16-token blocks for one slice of 32·W d (all four streams).
// Global traffic is linear: thread i moves the 16-byte pieces i, i + 64W, …
// of a block (x piece q: token q / (16W), stream (q / 4W) mod 4, 8-d chunk
// q mod 4W; dh piece i: token i / 4W, chunk i mod 4W), so each wave access
// reads runs of 64W bytes of every token row (640 B at W = 10) instead of the
// 64-byte pieces a matrix-core fragment covers.  Pieces stream three blocks
// ahead in a ring of four register slots (row-bounded buffer descriptors) and
// meet the matrix cores in LDS: each block is written to one of two padded
// tiles, then every wave reads its fragments (its own 32-d block) from there.
// Wave w projects its block with the φ B fragments it keeps in VGPRs; sums of
// squares and <dh, x[n]> go to v_dot2_f32_bf16.  The waves' partials meet in
// LDS and one summed record per (slice, token) goes to the workspace, a block
// late (after the next block's barrier): one barrier per block.
// register slots of x/dh pieces per thread: three blocks in flight at W = 8,
// two at W = 10 (whose 640 threads keep as many bytes in flight; a fourth
// slot there spills next to φ's high and low fragments)
template <int W>
constexpr int kPRing = W == 10 ? 3 : 4;

// f(integral_constant<int, i>) for i = I .. N − 1, in order.
template <int I, int N, typename F>
__device__ __forceinline__ void unroll_slots(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    unroll_slots<I + 1, N>(f);
  }
}
constexpr int kPRec = 29;    // record: p[24], ss, dhp[4]

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}
// Σ of the products of the two bf16 pairs in a and b, added to c.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         c, false);
}

template <int W>
struct ProjTile {
  static constexpr int kCh = 4 * W;                  // 8-d chunks of a stream row in the slice
  static constexpr int kXRow = kN * kCh * 16 + 16;   // bytes per token of the x tile (+16: banks)
  static constexpr int kHRow = kCh * 16 + 16;        // bytes per token of the dh tile
  static constexpr int kBytes = 16 * (kXRow + kHRow);
};

template <int W>
__global__ __launch_bounds__(64 * W, 1) void bwd_proj_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dh, const float* __restrict__ phi,
    float* __restrict__ part, int64_t T, int D, int64_t R) {
  constexpr int kThr = 64 * W;
  constexpr int kSl = 32 * W;  // d per slice
  using TL = ProjTile<W>;
  constexpr int kCh = TL::kCh;
  __shared__ __align__(16) float red[2][W][16][kPartStride];
  __shared__ __align__(16) char tile[2][TL::kBytes];
  // Token indices are 32-bit (T < 2^31): uniform compares then stay scalar,
  // and no VGPR temporary (which could alias an in-flight load) is needed.
  const int slice = blockIdx.x;
  const int tb = (int)(blockIdx.y * R);
  const int te = (int64_t)tb + R < T ? tb + (int)R : (int)T;
  const int nblk = te > tb ? (te - tb + 15) / 16 : 0;
  const int K = kN * D;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int row = lane & 15, g = lane >> 4;

  // this thread's pieces: global byte offsets within a block and LDS offsets
  uint32_t gx[4], lx[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = threadIdx.x + j * kThr;
    const int tk = q / (kN * kCh), n = (q / kCh) % kN, c = q % kCh;
    gx[j] = (uint32_t)((tk * K + n * D + slice * kSl + 8 * c) * 2);
    lx[j] = (uint32_t)(tk * TL::kXRow + (n * kCh + c) * 16);
  }
  const int htk = threadIdx.x / kCh, hc = threadIdx.x % kCh;
  const uint32_t gh = (uint32_t)((htk * D + slice * kSl + 8 * hc) * 2);
  const uint32_t lh = (uint32_t)(16 * TL::kXRow + htk * TL::kHRow + hc * 16);

  constexpr int kRing = kPRing<W>;
  uint4 xs[kRing][4], hs[kRing];
  auto load_blk = [&](int b, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    const int t0 = tb + 16 * b;
    const int rows = b < nblk ? ((te - t0) < 16 ? (te - t0) : 16) : 0;
    const int base = rows > 0 ? t0 : 0;
    const auto rx = make_rsrc(x + (int64_t)base * K, (uint32_t)rows * (uint32_t)K * 2u);
    const auto rh = make_rsrc(dh + (int64_t)base * D, (uint32_t)rows * (uint32_t)D * 2u);
#pragma unroll
    for (int j = 0; j < 4; ++j) xs[SL][j] = ld16(rx, gx[j]);
    hs[SL] = ld16(rh, gh);
  };

  // φ: stream by stream through LDS (the red buffer).  Its global loads go out
  // first, then those of the first kRing − 1 blocks, so that x and dh stream
  // while φ is staged: a CU's vector-memory path is the bottleneck here, and
  // φ queued behind three blocks of x and dh would hold up the first block by
  // their transfer time.
  // φ as two bf16 parts, φ = hi + lo (x is exact in bf16, so x·hi + x·lo
  // keeps about 16 mantissa bits of φ in the fp32 accumulation)
  uint4 bfr[kN][2], bfl[kN][2];
  {
    constexpr int kV4 = kSl * kC / 4;  // float4 of one stream's slice rows
    constexpr int kPer = (kV4 + kThr - 1) / kThr;
    float4 f[kN][kPer];
#pragma unroll
    for (int n = 0; n < kN; ++n)
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + k * kThr;
        f[n][k] = i < kV4 ? reinterpret_cast<const float4*>(phi + ((int64_t)n * D + slice * kSl) * kC)[i]
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    __builtin_amdgcn_sched_barrier(0);
    // (kept in issue order: the wait counts in the loop assume slot 0 oldest)
    unroll_slots<0, kRing - 1>([&](auto sl) {
      load_blk(decltype(sl)::value, sl);
      __builtin_amdgcn_sched_barrier(0);
    });
    float* stage = &red[0][0][0][0];
    static_assert(kSl * kC <= 2 * W * 16 * kPartStride, "one stream's φ slice fits the red buffer");
#pragma unroll
    for (int n = 0; n < kN; ++n) {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = threadIdx.x + k * kThr;
        if (i < kV4) reinterpret_cast<float4*>(stage)[i] = f[n][k];
      }
      __syncthreads();
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        const int c = cg * 16 + row;
        float v8[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) v8[v] = c < kC ? stage[(wave * 32 + 8 * g + v) * kC + c] : 0.f;
        bfr[n][cg] = make_uint4(pack_bf16x2(v8[0], v8[1]), pack_bf16x2(v8[2], v8[3]),
                                pack_bf16x2(v8[4], v8[5]), pack_bf16x2(v8[6], v8[7]));
        bfl[n][cg] = pack_bf16x8_rest(v8, bfr[n][cg]);
      }
      __syncthreads();
    }
  }

  // record of block b: the W waves' partials summed in a fixed order; rows
  // past the range fall outside the store descriptor
  auto record = [&](int b) {
    const int t0 = tb + 16 * b;
    const int rows = b < nblk ? ((te - t0) < 16 ? (te - t0) : 16) : 0;
    const auto rp = make_rsrc(part + ((int64_t)slice * T + (rows > 0 ? t0 : 0)) * kPartStride,
                              (uint32_t)rows * kPartStride * 4u);
    static_assert(16 * kPRec <= kThr, "one record value per thread");
    if (threadIdx.x < 16 * kPRec) {
      const int tk = threadIdx.x / kPRec, c = threadIdx.x % kPRec;
      float v = red[b & 1][0][tk][c];
#pragma unroll
      for (int w = 1; w < W; ++w) v += red[b & 1][w][tk][c];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rp, (tk * kPartStride + c) * 4, 0, 0);
    }
  };

  auto block = [&](int b, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    load_blk(b + kRing - 1, std::integral_constant<int, (SL + kRing - 1) % kRing>{});
    __builtin_amdgcn_sched_barrier(0);
    char* tl = tile[b & 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(tl + lx[j]) = xs[SL][j];
    *reinterpret_cast<uint4*>(tl + lh) = hs[SL];
    __syncthreads();
    if (b > 0) record(b - 1);
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    float ss = 0.f, dhp[kN] = {0.f, 0.f, 0.f, 0.f};
    const uint4 hv = *reinterpret_cast<const uint4*>(tl + 16 * TL::kXRow + row * TL::kHRow + (4 * wave + g) * 16);
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const uint4 a = *reinterpret_cast<const uint4*>(tl + row * TL::kXRow + (n * kCh + 4 * wave + g) * 16);
      acc0 = mfma(a, bfr[n][0], acc0);
      acc1 = mfma(a, bfr[n][1], acc1);
      acc0 = mfma(a, bfl[n][0], acc0);
      acc1 = mfma(a, bfl[n][1], acc1);
      ss = dot2(a.x, a.x, ss);
      ss = dot2(a.y, a.y, ss);
      ss = dot2(a.z, a.z, ss);
      ss = dot2(a.w, a.w, ss);
      dhp[n] = dot2(a.x, hv.x, dhp[n]);
      dhp[n] = dot2(a.y, hv.y, dhp[n]);
      dhp[n] = dot2(a.z, hv.z, dhp[n]);
      dhp[n] = dot2(a.w, hv.w, dhp[n]);
    }
    float(*rw)[kPartStride] = red[b & 1][wave];
    // D layout: lane holds tokens 4g+q of logit column row (+16)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rw[4 * g + q][row] = acc0[q];
      if (row < kC - 16) rw[4 * g + q][16 + row] = acc1[q];
    }
    // sums over the four k-groups of a token (lanes row + 16g)
    ss += __shfl_xor(ss, 16, kWave);
    ss += __shfl_xor(ss, 32, kWave);
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      dhp[n] += __shfl_xor(dhp[n], 16, kWave);
      dhp[n] += __shfl_xor(dhp[n], 32, kWave);
    }
    if (g == 0) {
      rw[row][kC] = ss;
#pragma unroll
      for (int n = 0; n < kN; ++n) rw[row][kC + 1 + n] = dhp[n];
    }
  };

  // Whole ring turns only (blocks past the range load and store nothing): a
  // loop with a single exit keeps each slot in the same registers on every
  // pass, so the wait counts stay exact across the back edge.
  int b = 0;
  for (; b < nblk; b += kRing) unroll_slots<0, kRing>([&](auto sl) { block(b + decltype(sl)::value, sl); });
  if (b > 0) {
    __syncthreads();
    record(b - 1);
  }
}

// ------------------------------------------------------------- pass 2 ---
// Per-token outputs, fp32: coef[t][64] = G[0..31] (c ≥ 24 zero), β at 32,
// H_pre[33..36]; dlog[r][24] and dal[r][4], one row per four tokens.
// A wave takes four tokens, one H_res entry per lane (lane 16·tk + 4·i + j:
// token tk, row i, column j), so the Sinkhorn rounds and their reverse walk
// are a few instructions per lane each: sums along a row of H_res over the
// lane quad, along a column over the rotations by 4 and 8 of the 16-lane DPP
// row.  The pass has no HBM volume to speak of; its time is the latency of
// those chains, which four times as many lanes per token shorten.
constexpr int kCoefStride = 64;
constexpr int kCoefThreads = 64;
constexpr int kCoefTokens = 4;  // tokens per workgroup (and per dlog / dal row)

__device__ __forceinline__ float row_sum4(float v) {  // Σ_j of entry (i, j)
  v += dpp<0xB1>(v);  // quad_perm(1,0,3,2)
  v += dpp<0x4E>(v);  // quad_perm(2,3,0,1)
  return v;
}
__device__ __forceinline__ float col_sum4(float v) {  // Σ_i of entry (i, j)
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  return v;
}
__global__ __launch_bounds__(kCoefThreads) void bwd_coef_kernel(
    const float* __restrict__ part, int nslices, const float* __restrict__ bias,
    const float* __restrict__ dH_post, const float* __restrict__ dH_res, float* __restrict__ coef,
    float* __restrict__ dlog, float* __restrict__ dal, int64_t T, int D, int iters, float eps,
    float a_pre, float a_post, float a_res, const float* __restrict__ alpha_dev) {
  if (alpha_dev != nullptr) {  // the gate scalars are held on the device (trained α)
    a_pre = alpha_dev[0];
    a_post = alpha_dev[1];
    a_res = alpha_dev[2];
  }
  extern __shared__ float hist[];  // per lane and round: u_i, then v_j
  const int lane = threadIdx.x;
  const int e = lane & 15, i = e >> 2, j = e & 3;
  const int64_t t = (int64_t)blockIdx.x * kCoefTokens + (lane >> 4);
  const bool tok = t < T;
  const int64_t tc = tok ? t : T - 1;
  const int K = kN * D;

  // slice sums (fixed order): pre i, post i, res (i, j), ss, dhp i.  Sixteen
  // slices' loads in flight at once (every slice of D = 5120 in one round
  // trip); slices past the count read slice 0 and add nothing, so the sums
  // keep the slice order
  float p_pre = 0.f, p_post = 0.f, p_res = 0.f, ss = 0.f, dhp = 0.f;
  constexpr int kChunk = 16;
  for (int s0 = 0; s0 < nslices; s0 += kChunk) {
    float va[kChunk], vb[kChunk], vc[kChunk], vd[kChunk], ve[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int s = s0 + u < nslices ? s0 + u : 0;
      const float* pp = part + ((int64_t)s * T + tc) * kPartStride;
      va[u] = pp[2 * kN + e];
      vc[u] = pp[i];
      vd[u] = pp[kN + i];
      ve[u] = pp[kC];
      vb[u] = pp[kC + 1 + i];
    }
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if (s0 + u < nslices) {
        p_pre += vc[u];
        p_post += vd[u];
        p_res += va[u];
        ss += ve[u];
        dhp += vb[u];
      }
    }
  }
  // same arithmetic as the forward kernels (hardware reciprocal and
  // reciprocal square root)
  const float rstd = __builtin_amdgcn_rsqf(ss / (float)K + eps);
  const float q_pre = rstd * p_pre, q_post = rstd * p_post, q_res = rstd * p_res;
  const float l_pre = a_pre * q_pre + bias[i];
  const float l_post = a_post * q_post + bias[kN + i];
  const float s_pre = __builtin_amdgcn_rcpf(1.0f + expf(-l_pre));
  const float s_post = __builtin_amdgcn_rcpf(1.0f + expf(-l_post));
  float m0 = a_res * q_res + bias[2 * kN + e];
  float mx = fmaxf(m0, dpp<0xB1>(m0));
  mx = fmaxf(mx, dpp<0x4E>(mx));
  m0 = expf(m0 - mx);

  // forward rounds on the scalings: M = diag(u)·M0·diag(v)
  float u = 1.f, v = 1.f;
  float* h = hist + lane;  // stride 64 floats between entries
  for (int it = 0; it < iters; ++it) {
    u = __builtin_amdgcn_rcpf(row_sum4(m0 * v));         // row i now sums to 1
    v = v * __builtin_amdgcn_rcpf(col_sum4(u * m0 * v));  // column j now sums to 1
    h[(it * 2 + 0) * 64] = u;
    h[(it * 2 + 1) * 64] = v;
  }

  // backward: G = dL/dM, walked from the last column step to the first row step
  float G = tok ? dH_res[tc * kN * kN + e] : 0.f;
  for (int it = iters - 1; it >= 0; --it) {
    const float u_s = h[(it * 2) * 64], v_s = h[(it * 2 + 1) * 64];
    const float u_p = it > 0 ? h[((it - 1) * 2) * 64] : 1.f;
    const float v_p = it > 0 ? h[((it - 1) * 2 + 1) * 64] : 1.f;
    // column step: X = M0·u_s·v_p, Y = M0·u_s·v_s, divisor c_j = v_p/v_s
    const float colacc = col_sum4(G * (m0 * u_s * v_s));
    G = (G - colacc) * (v_s * __builtin_amdgcn_rcpf(v_p));
    // row step: X = M0·u_p·v_p, Y = M0·u_s·v_p, divisor r_i = u_p/u_s
    const float rowacc = row_sum4(G * (m0 * u_s * v_p));
    G = (G - rowacc) * (u_s * __builtin_amdgcn_rcpf(u_p));
  }
  // dℓ_res = dM0 ⊙ M0 (the row-max shift contributes nothing: rows are
  // rescaled away by the first row step)
  const float dl_res = G * m0;
  const float dl_pre = dhp * s_pre * (1.0f - s_pre);
  const float dl_post = (tok ? dH_post[tc * kN + i] : 0.f) * 2.0f * s_post * (1.0f - s_post);
  // per token over its 24 columns (the pre and post columns of row i counted
  // by the lane of column 0): dq·p with raw p (q/rstd), and the dα terms
  const bool c0 = j == 0;
  const float dqp = col_sum4(row_sum4(a_res * dl_res * p_res +
                                      (c0 ? a_pre * dl_pre * p_pre + a_post * dl_post * p_post : 0.f)));
  const float da_pre = col_sum4(row_sum4(c0 ? dl_pre * q_pre : 0.f));
  const float da_post = col_sum4(row_sum4(c0 ? dl_post * q_post : 0.f));
  const float da_res = col_sum4(row_sum4(dl_res * q_res));
  if (tok) {
    float* co = coef + t * kCoefStride;
    co[2 * kN + e] = rstd * a_res * dl_res;
    if (j == 0) co[i] = rstd * a_pre * dl_pre;
    else if (j == 1) co[kN + i] = rstd * a_post * dl_post;
    else if (j == 2) co[33 + i] = s_pre;
    else {
      co[kC + i] = 0.f;
      co[kC + 4 + i] = 0.f;
    }
    if (e == 0) co[32] = rstd * rstd * rstd * dqp / (float)K;
  }
  // dbias and dα terms summed over the workgroup's four tokens (fixed
  // butterfly order); tokens past T contribute zero.  One row per workgroup.
  float red[5] = {tok ? dl_res : 0.f, tok && j < 2 ? (j == 0 ? dl_pre : dl_post) : 0.f, tok ? da_pre : 0.f,
                  tok ? da_post : 0.f, tok ? da_res : 0.f};
#pragma unroll
  for (int m = 16; m < 64; m <<= 1)
#pragma unroll
    for (int q = 0; q < 5; ++q) red[q] += __shfl_xor(red[q], m, kWave);
  if (lane < 16) {
    float* dl = dlog + (int64_t)blockIdx.x * kC;
    dl[2 * kN + e] = red[0];
    if (j == 0) dl[i] = red[1];
    else if (j == 1) dl[kN + i] = red[1];
  }
  if (lane == 0) {
    dal[(int64_t)blockIdx.x * 4 + 0] = red[2];
    dal[(int64_t)blockIdx.x * 4 + 1] = red[3];
    dal[(int64_t)blockIdx.x * 4 + 2] = red[4];
    dal[(int64_t)blockIdx.x * 4 + 3] = 0.f;
  }
}

// ------------------------------------------------------------- pass 3 ---
// Workgroup = one k-slice (128 d of each stream, 512 k: a 256-byte run of
// every token row) × a token range, in tiles of 16 tokens.  Global traffic is
// linear: thread i moves the 16-byte pieces i, i + 256, i + 512, i + 768 of a
// tile (piece q: token q/64, stream (q/16) mod 4, d chunk q mod 16), so every
// wave access covers whole 128-byte lines.  The matrix-core work meets that
// layout in LDS:
//  * dx̄ = G·φᵀ: wave w owns stream w's 128 d (eight 16-row k blocks), A = its
//    φ rows (bf16, in VGPRs for the whole kernel), B = the tile's G (bf16
//    high and low parts); results to LDS as [t][k];
//  * dφ += xᵀ·G over the tile's 16 tokens: the same k blocks × two column
//    blocks, A = xᵀ gathered from the LDS copy of the x tile, B = Gᵀ (both
//    parts).
// Each thread then finishes its pieces: dx += dx̄ − β·x + H_pre[n]·dh.
// The next tile's x, dx, dh and coefficients are loaded while a tile is
// worked on (two register buffers; vector memory completes in order, so those
// loads never wait on the stores issued after them).
// MIX: the kernel reads dx_next and H_res instead of dx and writes
// dx = H_resᵀ·dx_next + dx̄ − β·x + H_pre[n]·dh.  A thread's four pieces are
// then the four streams of one token and d-chunk, so the mix needs no other
// lane; it is rounded to bf16 exactly as mhc_post_bwd rounds its dx, which
// makes the result that of mhc_post_bwd followed by mhc_pre_bwd, bit for bit.
constexpr int kDxThreads = 256;
constexpr int kDxWd = 128;        // d per stream per slice
constexpr int kDxK = kN * kDxWd;  // 512 k per slice
constexpr int kDxTile = 16;       // tokens per tile
constexpr int kXRow = kDxK + 8;   // bf16 per x row in LDS
constexpr int kRRow = kDxK + 4;   // floats per dx̄ row in LDS
constexpr int kGRow = 40;         // bf16 per G row (32 c + pad)
constexpr int kTRow = 24;         // bf16 per Gᵀ row (16 t + pad)
constexpr int kHRow = kDxWd + 8;  // bf16 per dh row

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(s16x4_t a, s16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <bool MIX>
__global__ __launch_bounds__(kDxThreads, 2) void bwd_dx_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ dh, const float* __restrict__ phi,
    const float* __restrict__ coef, uint16_t* __restrict__ dx, float* __restrict__ dphi_part,
    int64_t T, int D, int64_t tok_per_split, const uint16_t* __restrict__ dxn,
    const float* __restrict__ hres) {
  __shared__ __align__(16) uint16_t xs[kDxTile * kXRow];     // x[t][k] of the tile
  __shared__ __align__(16) float dxr[kDxTile * kRRow];       // (G·φᵀ)[t][k]
  __shared__ __align__(16) uint16_t Gs[2][kDxTile * kGRow];  // G[t][c]: bf16 high, low parts
  __shared__ __align__(16) uint16_t GTs[2][32 * kTRow];      // Gᵀ[c][t]: the same two parts
  __shared__ __align__(16) uint16_t hs[2][kDxTile * kHRow];  // dh[t][d], by tile parity
  __shared__ float bs[2][kDxTile];                           // β, by tile parity
  __shared__ __align__(16) float hps[2][kDxTile][kN];        // H_pre, by tile parity
  __shared__ __align__(16) float hrs[MIX ? 2 : 1][kDxTile][kN * kN];  // H_res (MIX), by tile parity

  const int K = kN * D;
  const int d_base = blockIdx.x * kDxWd;
  const int64_t tb = (int64_t)blockIdx.y * tok_per_split;
  int64_t te = tb + tok_per_split;
  if (te > T) te = T;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, g = lane >> 4;

  // φ A fragments of this wave: rows k = stream w, d_base + 16·kb + row;
  // columns c = 8g .. 8g+7 (g = 3: c ≥ 24, zero), rounded to bf16
  uint4 af[8];
  {
    float4 f[8][2];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const float* src = phi + ((int64_t)wave * D + d_base + 16 * kb + row) * kC + 8 * (g < 3 ? g : 0);
      f[kb][0] = reinterpret_cast<const float4*>(src)[0];
      f[kb][1] = reinterpret_cast<const float4*>(src)[1];
    }
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      af[kb] = g < 3 ? make_uint4(pack_bf16x2(f[kb][0].x, f[kb][0].y), pack_bf16x2(f[kb][0].z, f[kb][0].w),
                                  pack_bf16x2(f[kb][1].x, f[kb][1].y), pack_bf16x2(f[kb][1].z, f[kb][1].w))
                     : make_uint4(0u, 0u, 0u, 0u);
    }
  }

  f32x4_t dacc[8][2];
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) dacc[kb][0] = dacc[kb][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // This thread's pieces j = 0..3, chunk pc: token 4j + tid/64 and stream pn,
  // or (MIX) token tid/16 and stream j.  Either way a wave access covers four
  // 256-byte runs.
  const int pn = (tid >> 4) & 3, pc = tid & 15;
  auto ptok = [&](int j) { return MIX ? tid >> 4 : 4 * j + (tid >> 6); };
  auto pstr = [&](int j) { return MIX ? j : pn; };
  uint32_t vo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    vo[j] = (uint32_t)(((ptok(j) * (int64_t)K) + (int64_t)pstr(j) * D + d_base + 8 * pc) * 2);
  // its dh piece: token tid/16, chunk tid mod 16
  const int ht = tid >> 4;
  const uint32_t vh = (uint32_t)(((int64_t)ht * D + d_base + 8 * pc) * 2);
  // its coefficient float4: threads < 128 G[t][4·(tid mod 8)..] of token tid/8;
  // 128..143 [β, H_pre 0..2] and 144..159 [H_pre 3, -] of token tid mod 16
  const int ct = tid < 128 ? tid >> 3 : tid & 15;
  const int cc = tid < 128 ? 4 * (tid & 7) : (tid < 144 ? 32 : 36);
  // MIX: the last wave loads the tile's H_res, lane l row l mod 4 of token
  // l / 4 (the other waves issue no load for it)
  static_assert(4 * kDxTile == kWave && kDxThreads / kWave == 4, "one H_res row per lane of wave 3");
  const bool hr_wave = __builtin_amdgcn_readfirstlane(wave) == 3;
  const uint32_t hr_off = (uint32_t)(lane * 16);

  auto rows_in = [&](int64_t t0) -> uint32_t {
    const int64_t r = te - t0;
    return (uint32_t)(r <= 0 ? 0 : (r < kDxTile ? r : kDxTile));
  };
  uint4 bx[2][4], bd[2][4], bh[2];
  float4 bc[2];
  uint4 bq[2];  // MIX: an H_res row
  // raw loads only: a value computed from a load here would make the wave wait
  // for it, and so for every load issued before it.  x, dh and dx (dx_next)
  // are read for the last time in the step here: non-temporal loads (measured
  // on MI355X: 102 instead of 115 µs at T = 4096, D = 5120, since the lines
  // they would otherwise keep are the ones this pass has yet to read; the same
  // hint on the projection pass's loads, whose x and dh this pass reads next,
  // makes this pass slower by more than it saves there)
  auto load_tile = [&](int64_t t0, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    const uint32_t rows = rows_in(t0);
    const int64_t tbase = rows > 0 ? t0 : 0;
    const auto rx = make_rsrc(x + tbase * K, rows * (uint32_t)K * 2);
    const auto rd = make_rsrc((MIX ? dxn : dx) + tbase * K, rows * (uint32_t)K * 2);
    const auto rh = make_rsrc(dh + tbase * D, rows * (uint32_t)D * 2);
    const auto rc = make_rsrc(coef + tbase * kCoefStride, rows * (uint32_t)kCoefStride * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) bx[SL][j] = ld16<2>(rx, vo[j]);
#pragma unroll
    for (int j = 0; j < 4; ++j) bd[SL][j] = ld16<2>(rd, vo[j]);
    bh[SL] = ld16<2>(rh, vh);
    const uint4 cv = ld16(rc, (uint32_t)((ct * kCoefStride + cc) * 4));
    bc[SL] = make_float4(__uint_as_float(cv.x), __uint_as_float(cv.y), __uint_as_float(cv.z),
                         __uint_as_float(cv.w));
    if constexpr (MIX) {
      if (hr_wave) {
        const auto rr = make_rsrc(hres + tbase * kN * kN, rows * (uint32_t)(kN * kN * 4));
        bq[SL] = ld16(rr, hr_off);
      }
    }
  };

  auto tile = [&](int64_t t0, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    // ---- stage: x tile, G / Gᵀ, β, H_pre, dh (rows past the range are zero:
    // their loads read zeros)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(&xs[ptok(j) * kXRow + pstr(j) * kDxWd + 8 * pc]) = bx[SL][j];
    *reinterpret_cast<uint4*>(&hs[SL][ht * kHRow + 8 * pc]) = bh[SL];
    {
      const float4 v = bc[SL];
      if (tid < 128) {
        // G as bf16 high and low parts, G = hi + lo
        const uint32_t w0 = pack_bf16x2(v.x, v.y), w1 = pack_bf16x2(v.z, v.w);
        const uint32_t r0 = pack_bf16x2_rest(v.x, v.y, w0), r1 = pack_bf16x2_rest(v.z, v.w, w1);
        *reinterpret_cast<uint2*>(&Gs[0][ct * kGRow + cc]) = make_uint2(w0, w1);
        *reinterpret_cast<uint2*>(&Gs[1][ct * kGRow + cc]) = make_uint2(r0, r1);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const uint32_t a = p ? r0 : w0, b = p ? r1 : w1;
          GTs[p][(cc + 0) * kTRow + ct] = (uint16_t)(a & 0xffffu);
          GTs[p][(cc + 1) * kTRow + ct] = (uint16_t)(a >> 16);
          GTs[p][(cc + 2) * kTRow + ct] = (uint16_t)(b & 0xffffu);
          GTs[p][(cc + 3) * kTRow + ct] = (uint16_t)(b >> 16);
        }
      } else if (tid < 144) {
        bs[SL][ct] = v.x;
        hps[SL][ct][0] = v.y;
        hps[SL][ct][1] = v.z;
        hps[SL][ct][2] = v.w;
      } else if (tid < 160) {
        hps[SL][ct][3] = v.x;
      }
    }
    if constexpr (MIX) {
      if (hr_wave) *reinterpret_cast<uint4*>(&hrs[SL][lane >> 2][4 * (lane & 3)]) = bq[SL];
    }
    // ---- the next tile into the other buffer
    load_tile(t0 + kDxTile, std::integral_constant<int, SL ^ 1>{});
    __syncthreads();
    // ---- matrix cores
    {
      // B: Gᵀ[c][t], high and low parts (φ enters as its bf16 rounding: the
      // error that leaves in G·φᵀ is of the order of the bf16 rounding of
      // the dx it is added to)
      const uint4 gb = *reinterpret_cast<const uint4*>(&Gs[0][row * kGRow + 8 * g]);
      const uint4 gbl = *reinterpret_cast<const uint4*>(&Gs[1][row * kGRow + 8 * g]);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        f32x4_t r = mfma(af[kb], gb, f32x4_t{0.f, 0.f, 0.f, 0.f});
        r = mfma(af[kb], gbl, r);
        *reinterpret_cast<f32x4_t*>(&dxr[row * kRRow + wave * kDxWd + 16 * kb + 4 * g]) = r;
      }
      s16x4_t gt[2][2];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
          gt[p][cb] = *reinterpret_cast<const s16x4_t*>(&GTs[p][(16 * cb + row) * kTRow + 4 * g]);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const int k = wave * kDxWd + 16 * kb + row;
        const s16x4_t a = {(short)xs[(4 * g + 0) * kXRow + k], (short)xs[(4 * g + 1) * kXRow + k],
                           (short)xs[(4 * g + 2) * kXRow + k], (short)xs[(4 * g + 3) * kXRow + k]};
        dacc[kb][0] = mfma16(a, gt[0][0], dacc[kb][0]);
        dacc[kb][1] = mfma16(a, gt[0][1], dacc[kb][1]);
        dacc[kb][0] = mfma16(a, gt[1][0], dacc[kb][0]);
        dacc[kb][1] = mfma16(a, gt[1][1], dacc[kb][1]);
      }
    }
    __syncthreads();
    // ---- finish this thread's pieces
    const uint32_t rows = rows_in(t0);
    const auto ro = make_rsrc(dx + (rows > 0 ? t0 : 0) * K, rows * (uint32_t)K * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = ptok(j), sn = pstr(j);
      const float* rp = &dxr[t * kRRow + sn * kDxWd + 8 * pc];
      const float4 r0 = *reinterpret_cast<const float4*>(rp);
      const float4 r1 = *reinterpret_cast<const float4*>(rp + 4);
      const uint4 hv = *reinterpret_cast<const uint4*>(&hs[SL][t * kHRow + 8 * pc]);
      const float beta = bs[SL][t], hp = hps[SL][t][sn];
      const float rv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
      uint4 dv;
      if constexpr (MIX) {
        // the token's hc_post part for stream j, Σ_n H_res[n][j]·dx_next[n], in
        // the arithmetic of mhc_post_bwd (fused multiply-adds over n from
        // zero, rounded to bf16); formed piece by piece to keep registers free
        float hc[kN];
#pragma unroll
        for (int n = 0; n < kN; ++n) hc[n] = hrs[SL][t][n * kN + j];
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int n = 0; n < kN; ++n) {
            const uint32_t gw = (&bd[SL][n].x)[q];
            a0 += hc[n] * bf16_lo(gw);
            a1 += hc[n] * bf16_hi(gw);
          }
          w[q] = pack_bf16x2(a0, a1);
        }
        dv = make_uint4(w[0], w[1], w[2], w[3]);
      } else {
        dv = bd[SL][j];
      }
      const uint4 xv = bx[SL][j];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w}, hw[4] = {hv.x, hv.y, hv.z, hv.w},
                     dw[4] = {dv.x, dv.y, dv.z, dv.w};
      float base[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        base[2 * q] = bf16_lo(dw[q]);
        base[2 * q + 1] = bf16_hi(dw[q]);
      }
      uint32_t ow[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float o0 = base[2 * q] + rv[2 * q] - beta * bf16_lo(xw[q]) + hp * bf16_lo(hw[q]);
        const float o1 = base[2 * q + 1] + rv[2 * q + 1] - beta * bf16_hi(xw[q]) + hp * bf16_hi(hw[q]);
        ow[q] = pack_bf16x2(o0, o1);
      }
      st16(ro, vo[j], make_uint4(ow[0], ow[1], ow[2], ow[3]));
    }
  };

  __builtin_amdgcn_sched_barrier(0);
  load_tile(tb, std::integral_constant<int, 0>{});
  // four stores that write nothing (empty descriptor): the loop is entered with
  // the same vector-memory queue as on every later pass (a tile's loads, then
  // the previous tile's four stores), so its wait counts need not drain it
  {
    const auto r0 = make_rsrc(dx, 0u);
#pragma unroll
    for (int j = 0; j < 4; ++j) st16(r0, vo[j], make_uint4(0u, 0u, 0u, 0u));
  }
  __builtin_amdgcn_sched_barrier(0);
  // Whole pairs of tiles only (a tile past the range loads and stores
  // nothing and adds zero to dφ): a loop with a single exit keeps each buffer
  // in the same registers on every pass, so the wait counts stay exact.
  for (int64_t t0 = tb; t0 < te; t0 += 2 * kDxTile) {
    tile(t0, std::integral_constant<int, 0>{});
    tile(t0 + kDxTile, std::integral_constant<int, 1>{});
  }
  // partial dφ of this (slice, token split): lane holds rows k = 16·kb + 4g + q
  // of stream `wave`, column c = 16·cb + row
#pragma unroll
  for (int kb = 0; kb < 8; ++kb) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = (int64_t)wave * D + d_base + 16 * kb + 4 * g + q;
      float* dst = dphi_part + ((int64_t)blockIdx.y * K + k) * kC;
      dst[row] = dacc[kb][0][q];
      if (row < kC - 16) dst[16 + row] = dacc[kb][1][q];
    }
  }
}

// ------------------------------------------------- fp32 I/O, passes 1 and 3 ---
// The same three passes for fp32 x, dh and dx, on the fp32 vector ALUs (the
// matrix cores' bf16 inputs would not keep fp32 accuracy).  Both kernels own a
// slice of 128 d (all four streams: 512 k) and walk a token range in tiles of
// 16 tokens, with φ's slice in LDS for the whole range, so φ is read once per
// workgroup instead of once per token.  Global traffic is linear (thread i
// moves the float4 pieces i, i + 256, … of a tile: 512-byte runs of every
// token row); products run from LDS with register blocking (eight or more
// fused multiply-adds per LDS read).  They write the records and the dφ
// partials of the bf16 path's layout, so its coefficient and sum kernels
// finish the job.
constexpr int kFD = 128;               // d per slice
constexpr int kFK = kN * kFD;          // k per slice
constexpr int kFT = 16;                // tokens per tile
constexpr int kFThreads = 256;
constexpr int kFRow = kFK + 4;         // floats per token row of an x / dx̄ tile in LDS
constexpr int kFHRow = kFD + 4;        // floats per token row of a dh tile
constexpr int kFX4 = kFT * kFK / 4 / kFThreads;  // x float4 pieces per thread per tile (8)
constexpr int kFH4 = kFT * kFD / 4 / kFThreads;  // dh float4 pieces per thread per tile (2)
static_assert(kFX4 == 8 && kFH4 == 2, "tile pieces");

__device__ __forceinline__ float4 ldf4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const uint4 v = ld16(r, voff);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// Tile pieces of thread `tid`: x piece q = tid + 256j is token q / 128,
// stream (q / 32) mod 4, d4 = q mod 32 (d = 4·d4 within the slice); dh piece
// q = tid + 256j is token q / 32, d4 = q mod 32.
struct FPieces {
  uint32_t gx[kFX4], gh[kFH4];  // byte offsets within the tile's rows in HBM
  int lx[kFX4], lh[kFH4];       // float offsets in the LDS tiles
  __device__ FPieces(int tid, int D, int slice) {
    const int K = kN * D;
#pragma unroll
    for (int j = 0; j < kFX4; ++j) {
      const int q = tid + kFThreads * j, tk = q / 128, n = (q / 32) % kN, d4 = q % 32;
      gx[j] = (uint32_t)((tk * K + n * D + slice * kFD + 4 * d4) * 4);
      lx[j] = tk * kFRow + n * kFD + 4 * d4;
    }
#pragma unroll
    for (int j = 0; j < kFH4; ++j) {
      const int q = tid + kFThreads * j, tk = q / 32, d4 = q % 32;
      gh[j] = (uint32_t)((tk * D + slice * kFD + 4 * d4) * 4);
      lh[j] = tk * kFHRow + 4 * d4;
    }
  }
};

// Pass 1, fp32.  Grid (D / 128 slices, token splits of R tokens).  Record of
// each (slice, token): p[24] = x·φ over the slice, ss = Σ x², dhp[n] = Σ_d
// dh·x[n] (the layout of the bf16 pass).
__global__ __launch_bounds__(kFThreads, 1) void bwd_proj_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ dh, const float* __restrict__ phi,
    float* __restrict__ part, int64_t T, int D, int64_t R) {
  __shared__ __align__(16) float phs[kFK * kC];         // φ[k][c] of the slice
  __shared__ __align__(16) float xs[kFT * kFRow];       // x[t][k] of the tile
  __shared__ __align__(16) float hsh[kFT * kFHRow];     // dh[t][d]
  __shared__ __align__(16) float red[16][kFT][kC];      // products by k-split
  const int slice = blockIdx.x, tid = threadIdx.x;
  const int64_t tb = (int64_t)blockIdx.y * R;
  const int64_t te = tb + R < T ? tb + R : T;
  const int nblk = te > tb ? (int)((te - tb + kFT - 1) / kFT) : 0;
  const int K = kN * D;
  const FPieces pc(tid, D, slice);
  // φ slice: rows n·D + slice·128 + dd of every stream, contiguous per stream
  for (int i = tid; i < kFK * kC / 4; i += kFThreads) {
    const int kl = i / (kC / 4), c4 = i % (kC / 4), n = kl / kFD, dd = kl % kFD;
    reinterpret_cast<float4*>(phs)[i] =
        reinterpret_cast<const float4*>(phi + ((int64_t)n * D + slice * kFD + dd) * kC)[c4];
  }
  float4 rx[kFX4], rh[kFH4];
  auto load = [&](int b) {
    const int64_t t0 = tb + (int64_t)kFT * b;
    const int64_t rows = b < nblk ? (te - t0 < kFT ? te - t0 : kFT) : 0;
    const int64_t base = rows > 0 ? t0 : 0;
    const auto ax = make_rsrc(x + base * K, (uint32_t)(rows * K * 4));
    const auto ah = make_rsrc(dh + base * D, (uint32_t)(rows * D * 4));
#pragma unroll
    for (int j = 0; j < kFX4; ++j) rx[j] = ldf4(ax, pc.gx[j]);
#pragma unroll
    for (int j = 0; j < kFH4; ++j) rh[j] = ldf4(ah, pc.gh[j]);
  };
  // product roles: k-split ks (32 k), tokens 4·tb4 .. +3, columns 6·cb .. +5
  const int ks = tid / 16, tb4 = (tid / 4) % 4, cb = tid % 4;
  // sum roles: token st, stream sn, quarter sq (32 d)
  const int st = tid / 16, sn = (tid / 4) % 4, sq = tid % 4;
  load(0);
  for (int b = 0; b < nblk; ++b) {
#pragma unroll
    for (int j = 0; j < kFX4; ++j) *reinterpret_cast<float4*>(xs + pc.lx[j]) = rx[j];
#pragma unroll
    for (int j = 0; j < kFH4; ++j) *reinterpret_cast<float4*>(hsh + pc.lh[j]) = rh[j];
    __syncthreads();
    load(b + 1);  // the next tile streams while this one is worked on
    float acc[4][6];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 6; ++c) acc[a][c] = 0.f;
    for (int kk = 0; kk < 32; kk += 4) {
      const int k = ks * 32 + kk;
      float4 xv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) xv[a] = *reinterpret_cast<const float4*>(xs + (4 * tb4 + a) * kFRow + k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2* pr = reinterpret_cast<const float2*>(phs + (k + e) * kC + 6 * cb);
        const float2 f0 = pr[0], f1 = pr[1], f2 = pr[2];
        const float ph[6] = {f0.x, f0.y, f1.x, f1.y, f2.x, f2.y};
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float xe = e == 0 ? xv[a].x : (e == 1 ? xv[a].y : (e == 2 ? xv[a].z : xv[a].w));
#pragma unroll
          for (int c = 0; c < 6; ++c) acc[a][c] = __builtin_fmaf(xe, ph[c], acc[a][c]);
        }
      }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int c = 0; c < 6; ++c) red[ks][4 * tb4 + a][6 * cb + c] = acc[a][c];
    // Σ x² and <dh, x[n]> of token st over quarter sq of stream sn
    float ssp = 0.f, dpp = 0.f;
#pragma unroll 8
    for (int dd = 0; dd < 32; ++dd) {
      const float xv = xs[st * kFRow + sn * kFD + sq * 32 + dd];
      ssp = __builtin_fmaf(xv, xv, ssp);
      dpp = __builtin_fmaf(hsh[st * kFHRow + sq * 32 + dd], xv, dpp);
    }
    // lanes 16·st .. 16·st + 15 hold (sn, sq): quads sum the quarters, the
    // row sums the streams (fixed order)
    dpp = dpp_f<0x4E>(dpp) + dpp;  // sq ^ 2
    dpp = dpp_f<0xB1>(dpp) + dpp;  // sq ^ 1
    ssp = dpp_f<0x4E>(ssp) + ssp;
    ssp = dpp_f<0xB1>(ssp) + ssp;
    ssp = dpp_f<0x141>(ssp) + ssp;
    ssp = dpp_f<0x140>(ssp) + ssp;
    __syncthreads();
    const int64_t t0 = tb + (int64_t)kFT * b;
    for (int o = tid; o < kFT * kC; o += kFThreads) {
      const int tk = o / kC, c = o % kC;
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) v += red[q][tk][c];
      if (t0 + tk < te) part[((int64_t)slice * T + t0 + tk) * kPartStride + c] = v;
    }
    if (sq == 0 && t0 + st < te) {
      float* rec = part + ((int64_t)slice * T + t0 + st) * kPartStride;
      rec[kC + 1 + sn] = dpp;
      if (sn == 0) rec[kC] = ssp;
    }
    __syncthreads();  // the tiles and red are rewritten next
  }
}

// Pass 3, fp32.  Grid (D / 128 slices, TS token splits of tps tokens).  Per
// tile: dx̄ = G·φᵀ into LDS; dφ += xᵀ·G kept in registers for the whole
// range; then dx += dx̄ − β·x + H_pre[n]·dh piece by piece.  The workgroup's dφ
// partial rows go to dphi_part[split][k][c].
__global__ __launch_bounds__(kFThreads, 1) void bwd_dx_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ dh, const float* __restrict__ phi,
    const float* __restrict__ coef, float* __restrict__ dx, float* __restrict__ dphi_part, int64_t T,
    int D, int64_t tps) {
  __shared__ __align__(16) float pht[kC * kFK];        // φ[k][c] of the slice, transposed: [c][k]
  __shared__ __align__(16) float xs[kFT * kFRow];      // x[t][k]
  __shared__ __align__(16) float dxr[kFT * kFRow];     // (G·φᵀ)[t][k]
  __shared__ __align__(16) float hsh[kFT * kFHRow];    // dh[t][d]
  __shared__ __align__(16) float gct[kC * kFT];        // G[c][t]
  __shared__ __align__(16) float gtc[kFT * kC];        // G[t][c]
  __shared__ float bs[kFT];                            // β
  __shared__ __align__(16) float hps[kFT][kN];         // H_pre
  const int slice = blockIdx.x, split = blockIdx.y, tid = threadIdx.x;
  const int64_t tb = (int64_t)split * tps;
  const int64_t te = tb + tps < T ? tb + tps : T;
  const int nblk = te > tb ? (int)((te - tb + kFT - 1) / kFT) : 0;
  const int K = kN * D;
  const FPieces pc(tid, D, slice);
  for (int i = tid; i < kFK * kC; i += kFThreads) {
    const int kl = i / kC, c = i % kC, n = kl / kFD, dd = kl % kFD;
    pht[c * kFK + kl] = phi[((int64_t)n * D + slice * kFD + dd) * kC + c];
  }
  float4 rx[kFX4], rh[kFH4], rd[kFX4];
  float4 rc;  // coefficients: threads < 160 hold float4 (tid mod 10) of token tid / 10
  auto load = [&](int b) {
    const int64_t t0 = tb + (int64_t)kFT * b;
    const int64_t rows = b < nblk ? (te - t0 < kFT ? te - t0 : kFT) : 0;
    const int64_t base = rows > 0 ? t0 : 0;
    const auto ax = make_rsrc(x + base * K, (uint32_t)(rows * K * 4));
    const auto ad = make_rsrc(dx + base * K, (uint32_t)(rows * K * 4));
    const auto ah = make_rsrc(dh + base * D, (uint32_t)(rows * D * 4));
    const auto ac = make_rsrc(coef + base * kCoefStride, (uint32_t)(rows * kCoefStride * 4));
#pragma unroll
    for (int j = 0; j < kFX4; ++j) rx[j] = ldf4(ax, pc.gx[j]);
#pragma unroll
    for (int j = 0; j < kFX4; ++j) rd[j] = ldf4(ad, pc.gx[j]);
#pragma unroll
    for (int j = 0; j < kFH4; ++j) rh[j] = ldf4(ah, pc.gh[j]);
    // token tid / 10, floats 4·(tid mod 10) .. +3 of its 40 (G[24], pad, β at 32, H_pre 33..36)
    rc = ldf4(ac, tid < kFT * 10 ? (uint32_t)(((tid / 10) * kCoefStride + 4 * (tid % 10)) * 4) : 0x7FFFFFF0u);
  };
  // dx̄ roles: tokens 4·db .. +3, k 8·dk .. +7
  const int db = tid / 64, dk = tid % 64;
  // dφ roles: k 8·fk .. +7, columns 6·fc .. +5
  const int fk = tid / 4, fc = tid % 4;
  float dph[8][6];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int c = 0; c < 6; ++c) dph[e][c] = 0.f;
  load(0);
  for (int b = 0; b < nblk; ++b) {
    const int64_t t0 = tb + (int64_t)kFT * b;
#pragma unroll
    for (int j = 0; j < kFX4; ++j) *reinterpret_cast<float4*>(xs + pc.lx[j]) = rx[j];
#pragma unroll
    for (int j = 0; j < kFH4; ++j) *reinterpret_cast<float4*>(hsh + pc.lh[j]) = rh[j];
    float4 dxin[kFX4];
#pragma unroll
    for (int j = 0; j < kFX4; ++j) dxin[j] = rd[j];
    if (tid < kFT * 10) {
      const int tk = tid / 10, q = tid % 10;
      const float v[4] = {rc.x, rc.y, rc.z, rc.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 4 * q + e;
        if (f < kC) {
          gct[f * kFT + tk] = v[e];
          gtc[tk * kC + f] = v[e];
        } else if (f == 32) {
          bs[tk] = v[e];
        } else if (f >= 33 && f < 33 + kN) {
          hps[tk][f - 33] = v[e];
        }
      }
    }
    __syncthreads();
    load(b + 1);
    // dx̄ = G·φᵀ for 4 tokens × 8 k
    {
      float acc[4][8];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[a][e] = 0.f;
#pragma unroll 4
      for (int c = 0; c < kC; ++c) {
        const float4 g = *reinterpret_cast<const float4*>(gct + c * kFT + 4 * db);
        const float4 p0 = *reinterpret_cast<const float4*>(pht + c * kFK + 8 * dk);
        const float4 p1 = *reinterpret_cast<const float4*>(pht + c * kFK + 8 * dk + 4);
        const float gv[4] = {g.x, g.y, g.z, g.w};
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[a][e] = __builtin_fmaf(gv[a], pv[e], acc[a][e]);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float* r = dxr + (4 * db + a) * kFRow + 8 * dk;
        *reinterpret_cast<float4*>(r) = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
        *reinterpret_cast<float4*>(r + 4) = make_float4(acc[a][4], acc[a][5], acc[a][6], acc[a][7]);
      }
    }
    // dφ += xᵀ·G over the tile's tokens (tokens past the range have x = 0, G = 0)
#pragma unroll 4
    for (int tk = 0; tk < kFT; ++tk) {
      const float4 x0 = *reinterpret_cast<const float4*>(xs + tk * kFRow + 8 * fk);
      const float4 x1 = *reinterpret_cast<const float4*>(xs + tk * kFRow + 8 * fk + 4);
      const float2* gp = reinterpret_cast<const float2*>(gtc + tk * kC + 6 * fc);
      const float2 g0 = gp[0], g1 = gp[1], g2 = gp[2];
      const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float gv[6] = {g0.x, g0.y, g1.x, g1.y, g2.x, g2.y};
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int c = 0; c < 6; ++c) dph[e][c] = __builtin_fmaf(xv[e], gv[c], dph[e][c]);
    }
    __syncthreads();
    // dx += dx̄ − β·x + H_pre[n]·dh, piece by piece (stores dropped past the range)
    {
      const int64_t rows = t0 < te ? (te - t0 < kFT ? te - t0 : kFT) : 0;
      const auto ad = make_rsrc(dx + (rows > 0 ? t0 : 0) * K, (uint32_t)(rows * K * 4));
#pragma unroll
      for (int j = 0; j < kFX4; ++j) {
        const int q = tid + kFThreads * j, tk = q / 128, n = (q / 32) % kN, d4 = q % 32;
        const float4 r = *reinterpret_cast<const float4*>(dxr + pc.lx[j]);
        const float4 xv = *reinterpret_cast<const float4*>(xs + pc.lx[j]);
        const float4 hv = *reinterpret_cast<const float4*>(hsh + tk * kFHRow + 4 * d4);
        const float be = bs[tk], hp = hps[tk][n];
        float4 o = dxin[j];
        o.x += r.x - be * xv.x + hp * hv.x;
        o.y += r.y - be * xv.y + hp * hv.y;
        o.z += r.z - be * xv.z + hp * hv.z;
        o.w += r.w - be * xv.w + hp * hv.w;
        st16<0>(ad, pc.gx[j], make_uint4(__float_as_uint(o.x), __float_as_uint(o.y), __float_as_uint(o.z),
                                      __float_as_uint(o.w)));
      }
    }
    __syncthreads();  // the tiles are rewritten next
  }
  // this split's dφ rows of the slice
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kl = 8 * fk + e, n = kl / kFD, dd = kl % kFD;
    float* row = dphi_part + ((int64_t)split * K + (int64_t)n * D + slice * kFD + dd) * kC + 6 * fc;
#pragma unroll
    for (int c = 0; c < 6; ++c) row[c] = dph[e][c];
  }
}

// dφ = Σ_s part[s] in split order.  Workgroup 0 sums the dbias / dα rows
// instead (one row per four tokens), in a fixed order.
__global__ __launch_bounds__(256) void dphi_bias_sum_kernel(const float* __restrict__ part,
                                                            float* __restrict__ dphi, int64_t KC, int S,
                                                            const float* __restrict__ dlog,
                                                            const float* __restrict__ dal,
                                                            float* __restrict__ dbias,
                                                            float* __restrict__ dalpha, int64_t R) {
  if (blockIdx.x == 0) {
    // thread t adds rows t, t + 256, … (all of a row's loads in flight at
    // once); the per-thread sums then meet by wave totals and the four waves
    // in index order
    constexpr int kV = kC + 3;
    __shared__ float red[(256 / kWave) * kV];
    const int t = threadIdx.x;
    float acc[kV];
#pragma unroll
    for (int c = 0; c < kV; ++c) acc[c] = 0.f;
    // four rows' loads in flight at once; rows past R read row r0 and add
    // nothing, so the sums keep the row order
    constexpr int kRows = 4;
    for (int64_t r0 = t; r0 < R; r0 += kRows * 256) {
      float4 v[kRows][kC / 4 + 1];
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        const int64_t r = r0 + u * 256 < R ? r0 + u * 256 : r0;
#pragma unroll
        for (int q = 0; q < kC / 4; ++q) v[u][q] = reinterpret_cast<const float4*>(dlog + r * kC)[q];
        v[u][kC / 4] = reinterpret_cast<const float4*>(dal + r * 4)[0];
      }
#pragma unroll
      for (int u = 0; u < kRows; ++u) {
        if (r0 + u * 256 >= R) continue;
#pragma unroll
        for (int q = 0; q < kC / 4 + 1; ++q) {
          const float w[4] = {v[u][q].x, v[u][q].y, v[u][q].z, v[u][q].w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * q + e < kV) acc[4 * q + e] += w[e];
        }
      }
    }
    const float v = wg_sum<kV, 256 / kWave>(acc, red);
    if (t < kC) dbias[t] = v;
    else if (t < kV && dalpha) dalpha[t - kC] = v;
    return;
  }
  // four consecutive entries a thread (KC is a multiple of 4), so that the
  // whole sum fits one round of workgroups
  const int64_t i = ((int64_t)(blockIdx.x - 1) * 256 + threadIdx.x) * 4;
  if (i >= KC) return;
  // the splits' loads in flight together (sixteen: one round trip for the
  // usual split counts), summed in split order
  constexpr int kChunk = 16;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < S; j0 += kChunk) {
    float4 v[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      v[u] = *reinterpret_cast<const float4*>(part + (int64_t)(j0 + u < S ? j0 + u : 0) * KC + i);
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (j0 + u < S) {
        s.x += v[u].x;
        s.y += v[u].y;
        s.z += v[u].z;
        s.w += v[u].w;
      }
  }
  *reinterpret_cast<float4*>(dphi + i) = s;
}

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct Layout {
  int W, S, PS, TS;   // projection: waves per workgroup, slices, token splits; dx: token splits
  int64_t R;          // projection tokens per split
  size_t part, coef, dlog, dal, dphi, total;
};

static Layout layout(const mhc_desc& d) {
  Layout L;
  const size_t T = (size_t)d.T, K = (size_t)kN * d.D;
  // projection slices of 320 d (ten waves) when D allows, else 256 d (eight);
  // fp32: slices of 128 d.  About one workgroup per CU of a 256-CU chip,
  // whole 16-token blocks
  L.W = d.D % 320 == 0 ? 10 : 8;
  L.S = d.io == kF32 ? d.D / kFD : d.D / (32 * L.W);
  const int64_t blocks = (d.T + 15) / 16;
  int64_t ps = 256 / L.S;
  if (ps > blocks) ps = blocks;
  if (ps < 1) ps = 1;
  L.R = (blocks + ps - 1) / ps * 16;
  L.PS = (int)((d.T + L.R - 1) / L.R);
  // token splits of the dx/dφ pass: about two workgroups per CU of a
  // 256-CU chip (K/512 slices × TS ≤ 512, two resident per CU), at most one
  // split per 16-token tile
  const int64_t nsl = (int64_t)K / kDxK;
  // (the fp32 kernel holds one workgroup per CU: one round of them)
  int64_t ts = (d.io == kF32 ? 256 : 512) / nsl;
  const int64_t tiles = (d.T + kDxTile - 1) / kDxTile;
  if (ts > tiles) ts = tiles;
  L.TS = (int)(ts < 1 ? 1 : (ts > 32 ? 32 : ts));
  L.part = 0;
  L.coef = L.part + align256((size_t)L.S * T * kPartStride * 4);
  L.dlog = L.coef + align256(T * kCoefStride * 4);
  L.dal = L.dlog + align256(T * kC * 4);
  L.dphi = L.dal + align256(T * 4 * 4);
  L.total = L.dphi + align256((size_t)L.TS * K * kC * 4);
  return L;
}

}  // namespace bwdm

bool pre_bwd_mfma_eligible(const mhc_desc& d) {
  return d.N == 4 && (d.io == kBF16 || d.io == kF32) && d.D % bwdm::kSliceD == 0 && d.sinkhorn_iters <= 64;
}

size_t pre_bwd_mfma_workspace_bytes(const mhc_desc& d) { return bwdm::layout(d).total; }

hipError_t launch_pre_bwd_mfma(const mhc_desc& d, const void* dh, const void* x, const float* phi,
                               const float* bias, const float* dH_post, const float* dH_res,
                               void* dx, float* dphi, float* dbias, float* dalpha, void* ws,
                               hipStream_t s, const void* dxn, const float* H_res) {
  if (dxn != nullptr && d.io != kBF16) return hipErrorInvalidValue;  // the fp32 passes do not mix
  using namespace bwdm;
  const Layout L = layout(d);
  char* w = static_cast<char*>(ws);
  float* part = reinterpret_cast<float*>(w + L.part);
  float* coef = reinterpret_cast<float*>(w + L.coef);
  float* dlog = reinterpret_cast<float*>(w + L.dlog);
  float* dal = reinterpret_cast<float*>(w + L.dal);
  float* dphi_part = reinterpret_cast<float*>(w + L.dphi);
  const int64_t T = d.T;
  const int K = kN * d.D;
  const dim3 pgrid((unsigned)L.S, (unsigned)L.PS);
  if (d.io == kF32)
    MHC_LAUNCH(bwd_proj_f32_kernel, pgrid, dim3(kFThreads), 0, s, static_cast<const float*>(x),
                       static_cast<const float*>(dh), phi, part, T, d.D, L.R);
  else if (L.W == 10)
    MHC_LAUNCH(bwd_proj_kernel<10>, pgrid, dim3(640), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(dh), phi, part, T, d.D, L.R);
  else
    MHC_LAUNCH(bwd_proj_kernel<8>, pgrid, dim3(512), 0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(dh), phi, part, T, d.D, L.R);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t hist_bytes = (size_t)d.sinkhorn_iters * 2 * 64 * sizeof(float);
  const int64_t coef_rows = (T + kCoefTokens - 1) / kCoefTokens;
  MHC_LAUNCH(bwd_coef_kernel, dim3((unsigned)coef_rows), dim3(kCoefThreads), hist_bytes,
                     s, part, L.S, bias, dH_post, dH_res, coef, dlog, dal, T, d.D, d.sinkhorn_iters,
                     d.eps, d.alpha_pre, d.alpha_post, d.alpha_res, d.alpha);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t tps = ((T + L.TS - 1) / L.TS + kDxTile - 1) / kDxTile * kDxTile;  // tokens per split
  if (d.io == kF32)
    MHC_LAUNCH(bwd_dx_f32_kernel, dim3((unsigned)(d.D / kFD), (unsigned)L.TS), dim3(kFThreads), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(dh), phi, coef,
                       static_cast<float*>(dx), dphi_part, T, d.D, tps);
  else if (dxn != nullptr)
    MHC_LAUNCH(bwd_dx_kernel<true>, dim3((unsigned)(K / kDxK), (unsigned)L.TS), dim3(kDxThreads), 0,
                       s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dh), phi, coef,
                       static_cast<uint16_t*>(dx), dphi_part, T, d.D, tps, static_cast<const uint16_t*>(dxn),
                       H_res);
  else
    MHC_LAUNCH(bwd_dx_kernel<false>, dim3((unsigned)(K / kDxK), (unsigned)L.TS), dim3(kDxThreads), 0,
                       s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(dh), phi, coef,
                       static_cast<uint16_t*>(dx), dphi_part, T, d.D, tps, nullptr, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t KC = (int64_t)K * kC;
  static_assert(kC % 4 == 0, "dφ rows are whole float4s");
  MHC_LAUNCH(dphi_bias_sum_kernel, dim3((unsigned)((KC / 4 + 255) / 256 + 1)), dim3(256), 0, s,
                     dphi_part, dphi, KC, L.TS, dlog, dal, dbias, dalpha, coef_rows);
  return hipGetLastError();
}

}  // namespace mhc
