// hc_pre forward, split-K pipeline across workgroups (bf16 I/O, N = 4, D = 5120 or 2560).
//
// Same computation as hc_pre_mfma_kernel (openPangu 2.0 analysis, §5.3 "mHC"
// formula block), organised so that HBM streams continuously:
//
//  * The d range is cut into S slices of 320 (all four streams).  A group of S
//    workgroups, one per CU, walks the group's 16-token tiles in lock step;
//    each keeps the bf16 B fragments of its φ slice in LDS for the whole kernel.
//  * Ten compute waves each own one 32-d block of the slice.  Period p: they
//    collapse tile p−5 (h = Σ_n H_pre[n]·x[n], straight from registers), issue
//    the loads of tile p+2 into the registers just freed, and project tile p on
//    v_mfma_f32_16x16x32_bf16 into LDS.  Seven register buffers: two tiles in
//    flight, five waiting for their H_pre.  x crosses HBM once.
//  * Two communication waves share, by tile parity, the exchange: in period p
//    one takes the totals of tile p−4 whose loads it issued two periods
//    earlier (rstd and H_pre of the 16 tokens, and the other logits of the
//    16/S tokens this workgroup finishes) and issues the loads of tile p−2's
//    records; the other publishes tile p−1's slice partials (24 raw
//    projections and the sum of squares per token) and, once 16 of this
//    workgroup's tokens are complete, runs their gates and Sinkhorn (one token
//    per lane quad) and writes H_pre, H_post, H_res.  No wave waits on a
//    memory round trip inside a period.
//  * One workgroup barrier per period hands the LDS buffers over.
//
// Exchange records are 64-bit words, a float and a 32-bit call tag, written
// and read with relaxed device-scope atomics: a reader that sees the tag sees
// the value, so no fence or flag is needed (release/acquire fences at device
// scope would write back or invalidate the whole L2).  Tags differ between
// calls, so stale records from an earlier call are never taken.
//
// Progress without a cooperative launch: a workgroup takes its role from a
// ticket drawn from a counter when it starts, and groups are runs of S
// consecutive tickets (modulo the grid size).  So at any time at most two
// groups (the newest, and the one the modulo wraps) have members not yet
// running; every other group has all its members running and finishes
// without help, freeing CUs for the missing members.  Each wait is also
// bounded: a wait that runs out gives up and writes NaN coefficients (and so
// NaN h) for the tokens of that tile — never a hang, never silently wrong
// values.
#include "mhc_coef.h"
#include "mhc_internal.h"

#include <atomic>
#include <chrono>
#include <type_traits>

namespace mhc {
namespace coop {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kN = 4;
constexpr int kC = 24;                  // logits: pre[4] post[4] res[16]
constexpr int kTM = 16;                 // tokens per tile (one 16-row MFMA block)
constexpr int kW = 10;                  // compute waves, one 32-d block each
constexpr int kThreads = (kW + 2) * 64; // + two communication waves
constexpr int kSliceD = kW * 32;        // 320 d per slice
constexpr int kLag = 5;                 // periods from projection to collapse
constexpr int kHq = kN + kN * kN;       // incoming H_post[4] and H_res[16] of a token (fused)
constexpr int kHead = 5;                // record entries every slice needs: pre[4], ss
constexpr int kRest = 20;               // record entries of the finishing slice: post[4], res[16]
constexpr int kRecA = kHead * kTM;      // part A of a (tile, slice) block: [entry][token]
constexpr int kRecWords = kRecA + kTM * kRest;  // + part B: [token][entry]; 3200 bytes
constexpr int kHeader = 256;            // workspace bytes holding the ticket counter
constexpr uint32_t kSpinLimit = 1u << 20;

__device__ __forceinline__ f32x4_t mfma(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                               0xF, 0xF, true));
}

__device__ __forceinline__ float fast_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + expf(-z)); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint4 v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)voff, 0, 0);
}

// Sum of squares of the two bf16 in w, added to c (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t w, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, c, false);
}

// Hides a value from the optimiser so that work on it is not merged with
// earlier work on the same registers.
__device__ __forceinline__ void opaque(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

__device__ __forceinline__ uint64_t entry(float v, uint32_t tag) {
  return ((uint64_t)tag << 32) | __float_as_uint(v);
}
__device__ __forceinline__ void put(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t get(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-scope (sc1) 64-bit record load through a buffer descriptor: the
// same instruction a relaxed agent-scope atomic load compiles to.
__device__ __forceinline__ uint64_t ld_rec(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 16);
  return ((uint64_t)v.y << 32) | v.x;
}
__device__ __forceinline__ float value_of(uint64_t e) { return __uint_as_float((uint32_t)e); }
__device__ __forceinline__ bool tagged(uint64_t e, uint32_t tag) { return (uint32_t)(e >> 32) == tag; }

// Record word of logit column c (0..23) of token tk; the sum of squares of
// token tk is word kSSWord + tk.
constexpr int kSSWord = 4 * kTM;
__device__ __forceinline__ int word_of(int c, int tk) {
  return c < 4 ? c * kTM + tk : kRecA + tk * kRest + (c - 4);
}

// Workspace: ticket counter (uint64) in the first kHeader bytes, then
// rec[tile][slice][kRecWords]
// uint64: part A [entry][token] holds pre[4] and ss (read by every slice,
// 128 contiguous bytes per entry), part B [token][entry] post[4] and res[16]
// (read by the slice that finishes the token).
// Calls f(integral_constant<J>) for J = 0 .. n−1 (one turn of a register ring).
template <typename F, int... J>
__device__ __forceinline__ void each_slot(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}

// FUSED: x is the previous layer's state; each tile's state is first mixed
// and written back, x_next = H_res·x + H_post ⊗ y (hc_post, in the same
// arithmetic order as the hc_post kernel), and hc_pre then runs on x_next
// (openPangu 2.0 analysis §11.3: merge, RMSNorm and H_pre in one pass).
template <int S, bool FUSED>
__device__ __forceinline__ void coop_body(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ y, const float* __restrict__ Hq_in,
    const float* __restrict__ Hr_in, uint16_t* __restrict__ xn,
    const float* __restrict__ bias, uint16_t* __restrict__ h,
    float* __restrict__ H_pre, float* __restrict__ H_post, float* __restrict__ H_res,
    const float* __restrict__ phi, uint64_t* ctr, uint64_t* rec, int64_t T, int Q, uint32_t tag,
    int iters, float eps, float a_pre, float a_post, float a_res) {
  constexpr int D = S * kSliceD;
  constexpr int K = kN * D;
  constexpr int kShare = kTM / S;  // tokens whose gates and Sinkhorn this workgroup finishes
  static_assert(kTM % S == 0 && (S == 16 || S == 8), "slice count");
  // periods per turn of the compute waves' register ring
  constexpr int kTurn = FUSED ? kLag : kLag + 2;
  __shared__ __align__(16) float red[2][kW][kRecWords];  // per-wave partials in record order, by period parity
  __shared__ __align__(16) float hpre_s[2][kTM][kN];
  __shared__ float rstd_s[2][kTM];
  // Gates + Sinkhorn run in batches of 16 tokens (kBatch tiles of this
  // workgroup's share): per token post[4], res[16], rstd, H_pre[4], in a
  // ring of two batches.
  constexpr int kBatch = 16 / kShare;
  __shared__ float shv[2 * kBatch * kShare][kRest + 1 + kN];
  __shared__ float bias_s[kC];
  __shared__ __align__(16) uint4 phis[kW][kN][2][64];  // φ B fragments of each compute wave
  __shared__ int ticket_s;
  __shared__ __align__(16) float hq_s[FUSED ? 2 : 1][kTM][kHq];  // incoming coefficients, by tile parity
  // collapsed h of a tile, by period parity (plain hc_pre): written by the
  // compute waves in fragment order, stored to HBM the next period as 640-byte
  // runs per token (a wave's fragment covers only 64 bytes of a token row)
  __shared__ __align__(16) uint4 hst[FUSED ? 1 : 2][kTM][kW * 4];

  // Every call draws exactly gridDim.x tickets, so any run of gridDim.x
  // consecutive counter values covers each residue once: the counter needs
  // no reset between calls and no initial value.
  if (threadIdx.x == 0)
    ticket_s = (int)(__hip_atomic_fetch_add(ctr, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) %
                     gridDim.x);
  if (threadIdx.x < kC) bias_s[threadIdx.x] = bias[threadIdx.x];
  for (int i = threadIdx.x; i < 2 * kTM * kN; i += kThreads) (&hpre_s[0][0][0])[i] = 0.f;
  __syncthreads();
  const int ticket = ticket_s;
  const int grp = ticket / S, slice = ticket % S;
  if (grp >= Q) return;  // whole workgroup: not part of any group

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  constexpr float rK = 1.0f / (float)K;
  const int64_t ntiles = (T + kTM - 1) / kTM;
  const int64_t nloc = grp < ntiles ? (ntiles - grp + Q - 1) / Q : 0;  // this group's tiles
  // periods: a whole number of turns of the compute waves' register ring
  // (periods past the last collapse do nothing), so that their loop has a
  // single exit and keeps each slot in the same registers on every pass
  const int64_t nper = (nloc + kLag + kTurn - 1) / kTurn * kTurn;
  auto tile_of = [&](int64_t p) { return grp + p * Q; };
  auto rows_of = [&](int64_t p) -> int64_t {  // valid tokens of the group's p-th tile
    if (p < 0 || p >= nloc) return 0;
    const int64_t r = T - tile_of(p) * kTM;
    return r < kTM ? r : kTM;
  };

  // φ slice → bf16 B fragments in LDS (all waves; the compute waves issue
  // their first tiles' loads right behind the φ loads).  Reads are coalesced
  // (the slice's rows of each stream are contiguous); each value goes to its
  // fragment position: wave dd/32, lane (c mod 16) + 16·g, column group c/16,
  // element v, for d = slice·320 + dd, g = (dd mod 32)/8, v = dd mod 8.
  // Columns 24..31 of the second group are zero.
  auto stage_phi = [&](auto&& between) {
    uint16_t* const ph = reinterpret_cast<uint16_t*>(&phis[0][0][0][0]);
    for (int i = threadIdx.x; i < kW * kN * 64; i += kThreads) {
      const int l = i & 63;
      if ((l & 15) >= kC - 16) (&phis[0][0][1][0])[(i >> 6) * 128 + l] = make_uint4(0u, 0u, 0u, 0u);
    }
    constexpr int kRow4 = kC / 4;  // float4 per φ row
    constexpr int kPer = kN * kSliceD * kRow4 / kThreads;
    static_assert(kN * kSliceD * kRow4 == kPer * kThreads, "φ slice in whole passes");
    float4 f[kPer];  // all loads in flight before the first LDS write
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + k * kThreads;
      const int n = i / (kSliceD * kRow4), rem = i % (kSliceD * kRow4);
      f[k] = *reinterpret_cast<const float4*>(phi + ((int64_t)n * D + slice * kSliceD) * kC + rem * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int i = threadIdx.x + k * kThreads;
      const int n = i / (kSliceD * kRow4), rem = i % (kSliceD * kRow4);
      const int dd = rem / kRow4, c0 = (rem % kRow4) * 4;
      const int w = dd >> 5, gg = (dd >> 3) & 3, v = dd & 7;
      const float fv[4] = {f[k].x, f[k].y, f[k].z, f[k].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + q, cg = c >> 4, ln = (c & 15) + 16 * gg;
        ph[((((w * kN + n) * 2 + cg) * 64 + ln) * 8) + v] = (uint16_t)f32_to_bf16_bits(fv[q]);
      }
    }
    __syncthreads();
  };

  if (wave < kW) {
   if constexpr (!FUSED) {
    // ================= compute waves =================
  constexpr int kAhead = 2;              // tiles whose loads are in flight
  constexpr int kSlots = kLag + kAhead;  // register buffers of x
  // Compute-wave lane roles: (row, g) holds token row, d block d0 + 8g .. +8.
  const int row = lane & 15, g = lane >> 4;
  const int d0 = slice * kSliceD + wave * 32;
  uint4 xb[kSlots][kN];
  // Loads and stores go through descriptors sized to the tile's valid rows, so
  // tails and tiles past the end need no branches (the wait counts then never
  // have to cover a path without them).
  auto load_tile = [&](int64_t p, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    const int64_t rows = rows_of(p);
    const uint16_t* base = x + (rows > 0 ? tile_of(p) * kTM * K : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (uint32_t)(rows * K * 2));
#pragma unroll
    for (int n = 0; n < kN; ++n) xb[SL][n] = ld16(rs, (uint32_t)(((row * kN + n) * D + d0 + 8 * g) * 2));
  };
  static_assert(kAhead == 2, "prologue below issues two tiles");
  stage_phi([&]() {
    // kept in issue order: the wait counts in the loop assume slot 0 oldest
    load_tile(0, std::integral_constant<int, 0>{});
    __builtin_amdgcn_sched_barrier(0);
    load_tile(1, std::integral_constant<int, 1>{});
  });
  // the slots of tiles before the first are collapsed into dropped stores
#pragma unroll
  for (int s = kAhead; s < kSlots; ++s)
#pragma unroll
    for (int n = 0; n < kN; ++n) xb[s][n] = make_uint4(0u, 0u, 0u, 0u);
  const uint4(*bf)[2][64] = phis[wave];


    // h of the tile collapsed in period q, from LDS to HBM: thread i stores
    // piece i (token i / 4kW, 8-d chunk i mod 4kW of the slice)
    auto flush_h = [&](int64_t q) {
      static_assert(kTM * kW * 4 == kW * kWave, "one h piece per compute thread");
      const int64_t rows = rows_of(q - kLag);
      uint16_t* base = h + (rows > 0 ? tile_of(q - kLag) * kTM * D : 0);
      const __amdgpu_buffer_rsrc_t hr = make_rsrc(base, (uint32_t)(rows * D * 2));
      const int tk = threadIdx.x / (kW * 4), c = threadIdx.x % (kW * 4);
      st16(hr, (uint32_t)((tk * D + slice * kSliceD + 8 * c) * 2), hst[q & 1][tk][c]);
    };
    auto period = [&](int64_t p, auto j_c) {
      constexpr int J = decltype(j_c)::value;  // p mod kSlots
      constexpr int SP = J;                    // slot of tile p
      constexpr int SC = (J + kAhead) % kSlots;  // slot of tile p − kLag (then of p + kAhead)
      flush_h(p - 1);  // its LDS buffer is complete: the last period ended with a barrier
      // collapse tile p − kLag
      {
        const float4 hw = *reinterpret_cast<const float4*>(&hpre_s[(p - kLag) & 1][row][0]);
        const float hv[kN] = {hw.x, hw.y, hw.z, hw.w};
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < kN; ++n) {
          uint4 a = xb[SC][n];
          opaque(a);  // unpack here, not at the projection (keeps floats out of VGPRs)
          o[0] += hv[n] * bf16_lo(a.x);
          o[1] += hv[n] * bf16_hi(a.x);
          o[2] += hv[n] * bf16_lo(a.y);
          o[3] += hv[n] * bf16_hi(a.y);
          o[4] += hv[n] * bf16_lo(a.z);
          o[5] += hv[n] * bf16_hi(a.z);
          o[6] += hv[n] * bf16_lo(a.w);
          o[7] += hv[n] * bf16_hi(a.w);
        }
        hst[p & 1][row][wave * 4 + g] = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                                   pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
      }
      // loads of tile p + kAhead into the slot just freed
      load_tile(p + kAhead, std::integral_constant<int, SC>{});
      __builtin_amdgcn_sched_barrier(0);
      // projection and sum of squares of tile p
      {
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        float ss = 0.f;
#pragma unroll
        for (int n = 0; n < kN; ++n) {
          const uint4 a = xb[SP][n];
          acc0 = mfma(a, bf[n][0][lane], acc0);
          acc1 = mfma(a, bf[n][1][lane], acc1);
          ss = dot2(a.x, ss);
          ss = dot2(a.y, ss);
          ss = dot2(a.z, ss);
          ss = dot2(a.w, ss);
        }
        float* rw = red[p & 1][wave];
        // D layout: lane holds tokens 4g+q of logit column row (+16)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rw[word_of(row, 4 * g + q)] = acc0[q];
          if (row < kC - 16) rw[word_of(16 + row, 4 * g + q)] = acc1[q];
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        if (g == 0) rw[kSSWord + row] = ss;
      }
      __syncthreads();
    };

    static_assert(kSlots == 7, "unroll below");
    for (int64_t p = 0; p < nper; p += kSlots) {
      period(p, std::integral_constant<int, 0>{});
      period(p + 1, std::integral_constant<int, 1>{});
      period(p + 2, std::integral_constant<int, 2>{});
      period(p + 3, std::integral_constant<int, 3>{});
      period(p + 4, std::integral_constant<int, 4>{});
      period(p + 5, std::integral_constant<int, 5>{});
      period(p + 6, std::integral_constant<int, 6>{});
    }
    flush_h(nper - 1);  // the last period ended with a barrier
   } else {
    // ============ compute waves, fused with the previous hc_post ============
  // Ring of kLag registers sets holding x_next of the tiles waiting for their
  // H_pre (indexed by p mod kLag); one set for the next tile's incoming state
  // and y.  In period p: collapse tile p − kLag (freeing its set), mix tile p
  // into that set (x_next = H_res·x + H_post ⊗ y, written back), issue the
  // loads of tile p + 1 into the incoming set, project tile p.
  const int row = lane & 15, g = lane >> 4;
  const int d0 = slice * kSliceD + wave * 32;
  uint4 xs[kLag][kN];
  uint4 raw[kN], yr;
  float4 hq_reg;  // incoming coefficients of the next tile (waves 0, 1; zero elsewhere)
  auto load_raw = [&](int64_t p) {
    const int64_t rows = rows_of(p);
    const int64_t t0 = rows > 0 ? tile_of(p) * kTM : 0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(x + t0 * K, (uint32_t)(rows * K * 2));
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(y + t0 * D, (uint32_t)(rows * D * 2));
#pragma unroll
    for (int n = 0; n < kN; ++n) raw[n] = ld16(rs, (uint32_t)(((row * kN + n) * D + d0 + 8 * g) * 2));
    yr = ld16(ry, (uint32_t)((row * D + d0 + 8 * g) * 2));
  };
  // lanes i < 80 of waves 0, 1 load float4 i of a tile's incoming
  // coefficients (token i/5: H_res row-major in chunks 0..3, H_post in 4).
  // Every wave issues the load (others through an empty descriptor) so that
  // all waves see the same vector-memory queue and the same wait counts.
  const int ci = wave * 64 + lane, ct = ci / 5, cc = ci % 5;
  const bool c_lane = ci < kTM * 5;
  auto load_coef = [&](int64_t p) {
    const int64_t rows = wave < 2 ? rows_of(p) : 0;
    const int64_t t0 = rows > 0 ? tile_of(p) * kTM : 0;
    const bool in = c_lane && ct < rows;
    constexpr uint32_t kOut = 0x7FFFFFF0u;  // past every descriptor: reads zero
    // both descriptors are wave-uniform; each lane reads one of them and
    // zero from the other
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(Hr_in + t0 * kN * kN, (uint32_t)(rows * kN * kN * 4));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Hq_in + t0 * kN, (uint32_t)(rows * kN * 4));
    const uint4 vr = ld16(rr, in && cc < 4 ? (uint32_t)((ct * kN * kN + 4 * cc) * 4) : kOut);
    const uint4 vq = ld16(rq, in && cc == 4 ? (uint32_t)(ct * kN * 4) : kOut);
    hq_reg = make_float4(__uint_as_float(vr.x | vq.x), __uint_as_float(vr.y | vq.y),
                         __uint_as_float(vr.z | vq.z), __uint_as_float(vr.w | vq.w));
  };
  auto stage_coef = [&](int64_t p) {  // hq_reg → hq_s[p & 1]
    if (wave < 2 && c_lane) *reinterpret_cast<float4*>(&hq_s[p & 1][ct][cc < 4 ? kN + 4 * cc : 0]) = hq_reg;
  };
  stage_phi([&]() {
    load_coef(0);
    __builtin_amdgcn_sched_barrier(0);
    load_raw(0);
    __builtin_amdgcn_sched_barrier(0);
    stage_coef(0);
  });
  // the sets of tiles before the first are collapsed into dropped stores
#pragma unroll
  for (int s = 0; s < kLag; ++s)
#pragma unroll
    for (int n = 0; n < kN; ++n) xs[s][n] = make_uint4(0u, 0u, 0u, 0u);
  const uint4(*bf)[2][64] = phis[wave];

    auto period = [&](int64_t p_in, auto j_c) {
      constexpr int J = decltype(j_c)::value;  // p mod kLag: set of tile p − kLag, then of tile p
      // p passes through an SGPR the compiler cannot see into, so that the
      // addresses of the unrolled periods are computed where used rather than
      // all held from the loop head (scalar registers are short here)
      int p32 = (int)p_in;
      asm volatile("" : "+s"(p32));
      const int64_t p = p32;
      // collapse tile p − kLag
      {
        const int64_t rows = rows_of(p - kLag);
        uint16_t* base = h + (rows > 0 ? tile_of(p - kLag) * kTM * D : 0);
        const __amdgpu_buffer_rsrc_t hr = make_rsrc(base, (uint32_t)(rows * D * 2));
        const float4 hw = *reinterpret_cast<const float4*>(&hpre_s[(p - kLag) & 1][row][0]);
        const float hv[kN] = {hw.x, hw.y, hw.z, hw.w};
        float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < kN; ++n) {
          uint4 a = xs[J][n];
          opaque(a);
          o[0] += hv[n] * bf16_lo(a.x);
          o[1] += hv[n] * bf16_hi(a.x);
          o[2] += hv[n] * bf16_lo(a.y);
          o[3] += hv[n] * bf16_hi(a.y);
          o[4] += hv[n] * bf16_lo(a.z);
          o[5] += hv[n] * bf16_hi(a.z);
          o[6] += hv[n] * bf16_lo(a.w);
          o[7] += hv[n] * bf16_hi(a.w);
        }
        st16(hr, (uint32_t)((row * D + d0 + 8 * g) * 2),
             make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                        pack_bf16x2(o[6], o[7])));
      }
      // coefficients of tile p + 1, ahead of its state loads
      load_coef(p + 1);
      __builtin_amdgcn_sched_barrier(0);
      // x_next of tile p: H_res·x + H_post ⊗ y in the hc_post kernel's order
      // (fused multiply-adds over m after H_post·y), rounded to bf16, written
      // back and kept as the state hc_pre reads
      {
        const int64_t rows = rows_of(p);
        const int64_t t0 = rows > 0 ? tile_of(p) * kTM : 0;
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(xn + t0 * K, (uint32_t)(rows * K * 2));
        const float* hq = hq_s[p & 1][row];
#pragma unroll
        for (int n = 0; n < kN; ++n) {
          __builtin_amdgcn_sched_barrier(0);
          const float4 r4 = *reinterpret_cast<const float4*>(hq + kN + kN * n);  // H_res row n
          const float hr_n[kN] = {r4.x, r4.y, r4.z, r4.w};
          const float hp_n = hq[n];
          uint32_t w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t yw = (&yr.x)[q];
            float o[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              float a = hp_n * (e ? bf16_hi(yw) : bf16_lo(yw));
#pragma unroll
              for (int m = 0; m < kN; ++m) {
                const uint32_t xw = (&raw[m].x)[q];
                a = __builtin_fmaf(hr_n[m], e ? bf16_hi(xw) : bf16_lo(xw), a);
              }
              o[e] = a;
            }
            w[q] = pack_bf16x2(o[0], o[1]);
          }
          xs[J][n] = make_uint4(w[0], w[1], w[2], w[3]);
          st16(ro, (uint32_t)(((row * kN + n) * D + d0 + 8 * g) * 2), xs[J][n]);
        }
      }
      // loads of tile p + 1 into the incoming set just consumed
      load_raw(p + 1);
      __builtin_amdgcn_sched_barrier(0);
      // projection and sum of squares of tile p
      {
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        float ss = 0.f;
#pragma unroll
        for (int n = 0; n < kN; ++n) {
          // one stream's B fragments at a time (registers are short here)
          __builtin_amdgcn_sched_barrier(0);
          const uint4 a = xs[J][n];
          acc0 = mfma(a, bf[n][0][lane], acc0);
          acc1 = mfma(a, bf[n][1][lane], acc1);
          ss = dot2(a.x, ss);
          ss = dot2(a.y, ss);
          ss = dot2(a.z, ss);
          ss = dot2(a.w, ss);
        }
        float* rw = red[p & 1][wave];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          rw[word_of(row, 4 * g + q)] = acc0[q];
          if (row < kC - 16) rw[word_of(16 + row, 4 * g + q)] = acc1[q];
        }
        ss += __shfl_xor(ss, 16, kWave);
        ss += __shfl_xor(ss, 32, kWave);
        if (g == 0) rw[kSSWord + row] = ss;
      }
      stage_coef(p + 1);
      __syncthreads();
    };

    // whole turns of the register ring, no early exit
    for (int64_t p = 0; p < nper; p += kLag)
      each_slot([&](auto j) { period(p + decltype(j)::value, j); }, std::make_integer_sequence<int, kLag>{});
   }
  } else {
    // ================= communication waves =================
    // Wave X = 0, 1 owns the tiles of parity X: in periods p ≡ X (mod 2) it
    // takes tile p − 4 (records it loaded two periods earlier) and issues the
    // record loads of tile p − 2; in the other periods it publishes tile p − 1
    // and, when a batch of its workgroup's tokens is complete, runs their gates
    // and Sinkhorn.
    const int X = wave - kW;
    stage_phi([]() {});
    // gather (a), rstd and H_pre of the 16 tokens: lane (tk, n) = (lane / 4,
    // lane mod 4) sums entry pre[n] of token tk over all S slices (one 512-byte
    // run per slice across the wave) and the sum of squares over S/4 slices;
    // the four lanes of a token then add their sums of squares by DPP.
    constexpr int S4 = S / 4;
    const int tk = lane >> 2, n = lane & 3;
    // gather (b), post + res logits of this workgroup's share: lane (ts or
    // slice half, j) sums entry 5 + j of its token over 8 slices
    constexpr int kHalves = kShare == 1 ? 2 : 1;  // lanes ≥ 32: second slice half, or second token
    constexpr int SB = S / kHalves;               // slices per lane (8)
    const int hi = lane >> 5, j = lane & 31;
    const int ts = kShare == 1 ? 0 : hi;
    const int tb = slice * kShare + ts;
    const int jc = j < kRest ? j : kRest - 1;  // idle lanes read a valid word
    // Record registers: wave X issues the loads of tile q (parity X) at the
    // end of period q + 2, after the record was published in period q + 1, and
    // takes the tile in period q + 4.
    uint64_t va[S], vs[S4], vb[SB];
    // Record loads: one descriptor per tile, per-lane offset registers and
    // uniform slice offsets.
    const uint32_t voff_a = (uint32_t)((n * kTM + tk) * 8);
    const uint32_t voff_s = (uint32_t)(((n * S4) * kRecWords + kSSWord + tk) * 8);
    const uint32_t voff_b =
        (uint32_t)((((kShare == 1 ? hi : 0) * SB) * kRecWords + kRecA + tb * kRest + jc) * 8);
    auto load_all = [&](int64_t pt) {  // records of the group's pt-th tile
      asm volatile("" ::: "memory");  // the records change behind the compiler's back
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(rec + tile_of(pt) * S * (int64_t)kRecWords, S * kRecWords * 8);
#pragma unroll
      for (int i = 0; i < S; ++i) va[i] = ld_rec(rs, voff_a, i * kRecWords * 8);
#pragma unroll
      for (int i = 0; i < S4; ++i) vs[i] = ld_rec(rs, voff_s, i * kRecWords * 8);
#pragma unroll
      for (int i = 0; i < SB; ++i) vb[i] = ld_rec(rs, voff_b, i * kRecWords * 8);
    };
    auto all_tagged = [&]() {
      bool ok = true;
#pragma unroll
      for (int i = 0; i < S; ++i) ok = ok && tagged(va[i], tag);
#pragma unroll
      for (int i = 0; i < S4; ++i) ok = ok && tagged(vs[i], tag);
#pragma unroll
      for (int i = 0; i < SB; ++i) ok = ok && tagged(vb[i], tag);
      return __all(ok);
    };
    constexpr int kTake = kLag - 1;  // tile taken in period p
    static_assert(kTake % 2 == 0, "a wave loads and takes the tiles of its parity");
    for (int64_t p = 0; p < nper; ++p) {
      if ((int)(p & 1) == X) {
        // take tile p − kTake (reload while a slice is late)
        if (p >= kTake && p - kTake < nloc) {
          uint32_t spins = 0;
          while (!all_tagged() && ++spins < kSpinLimit) {
            __builtin_amdgcn_s_sleep(2);
            load_all(p - kTake);
          }
          // a wait that ran out (a group member never published) poisons the
          // tile's coefficients, and so h, H_pre, H_post and H_res of its
          // tokens, with NaN: a loud failure instead of silently wrong values
          const float poison = spins < kSpinLimit ? 0.f : __builtin_nanf("");
          const int bt = (p - kTake) & 1;
          const int ring = (int)((p - kTake) % (2 * kBatch)) * kShare;  // ring row of the tile's share
          // (a): slice sums in a fixed order; quad sum of the squares
          float pre = poison, ss = poison;
#pragma unroll
          for (int i = 0; i < S; ++i) pre += value_of(va[i]);
#pragma unroll
          for (int i = 0; i < S4; ++i) ss += value_of(vs[i]);
          ss += dpp<0xB1>(ss);  // quad_perm(1,0,3,2)
          ss += dpp<0x4E>(ss);  // quad_perm(2,3,0,1)
          const float rstd = __builtin_amdgcn_rsqf(ss * rK + eps);
          const float hp = fast_sigmoid(a_pre * (rstd * pre) + bias_s[n]);
          hpre_s[bt][tk][n] = hp;
          if (n == 0) rstd_s[bt][tk] = rstd;
          if (tk / kShare == slice) {  // a token this workgroup finishes
            float* r = shv[ring + tk % kShare];
            if (n == 0) r[kRest] = rstd;
            r[kRest + 1 + n] = hp;
          }
          // (b): slice sums of the share's post + res logits
          float v = poison;
#pragma unroll
          for (int i = 0; i < SB; ++i) v += value_of(vb[i]);
          if (kShare == 1) v += __shfl_xor(v, 32, kWave);
          if (j < kRest && (kShare != 1 || hi == 0)) shv[ring + ts][j] = v;
        }
        // loads of tile p − 2's records (published during the previous period)
        if (p >= 2 && p - 2 < nloc) load_all(p - 2);
      } else {
        // publish tile p − 1: the ten waves' partials summed in a fixed order
        if (p >= 1 && p - 1 < nloc) {
          const float(*rp)[kRecWords] = red[(p - 1) & 1];
          uint64_t* mine = rec + (tile_of(p - 1) * S + slice) * (int64_t)kRecWords;
#pragma unroll 1
          for (int i = 2 * lane; i < kRecWords; i += 128) {
            float2 a = *reinterpret_cast<const float2*>(&rp[0][i]);
#pragma unroll
            for (int w = 1; w < kW; ++w) {
              const float2 b = *reinterpret_cast<const float2*>(&rp[w][i]);
              a.x += b.x;
              a.y += b.y;
            }
            put(mine + i, entry(a.x, tag));
            put(mine + i + 1, entry(a.y, tag));
          }
        }
        // gates + Sinkhorn of the batch ending with tile q = p − kLag: the
        // ring rows of tile q were filled in period q + kTake, and are not
        // refilled before period q + kBatch + kTake + 1
        const int64_t q = p - kLag;
        if (q >= 0 && q < nloc && (q % kBatch == kBatch - 1 || q == nloc - 1)) {
          const int64_t q0 = q - q % kBatch;
          const int ntok = (int)(q - q0 + 1) * kShare;
          const int u = lane >> 2, i = lane & 3;  // token of the batch, row of H_res
          if (u < ntok) {
            const int64_t qt = q0 + u / kShare;
            const int us = u % kShare;
            const float* r = shv[(int)(qt % (2 * kBatch)) * kShare + us];  // post[4], res[16], rstd, H_pre[4]
            const float rstd = r[kRest];
            float m[kN], mx = -__builtin_huge_valf();
#pragma unroll
            for (int jj = 0; jj < kN; ++jj) {
              m[jj] = a_res * (rstd * r[kN + i * kN + jj]) + bias_s[2 * kN + i * kN + jj];
              mx = fmaxf(mx, m[jj]);
            }
#pragma unroll
            for (int jj = 0; jj < kN; ++jj) m[jj] = expf(m[jj] - mx);
            for (int it = 0; it < iters; ++it) {
              const float rinv = __builtin_amdgcn_rcpf((m[0] + m[1]) + (m[2] + m[3]));
#pragma unroll
              for (int jj = 0; jj < kN; ++jj) m[jj] *= rinv;
#pragma unroll
              for (int jj = 0; jj < kN; ++jj) {
                const float s1 = m[jj] + dpp<0xB1>(m[jj]);  // quad_perm(1,0,3,2)
                const float sc = s1 + dpp<0x4E>(s1);        // quad_perm(2,3,0,1)
                m[jj] *= __builtin_amdgcn_rcpf(sc);
              }
            }
            const int64_t tt = tile_of(qt) * kTM + slice * kShare + us;
            if (tt < T) {
              H_pre[tt * kN + i] = r[kRest + 1 + i];
              H_post[tt * kN + i] = 2.0f * fast_sigmoid(a_post * (rstd * r[i]) + bias_s[kN + i]);
              reinterpret_cast<float4*>(H_res)[tt * kN + i] = make_float4(m[0], m[1], m[2], m[3]);
            }
          }
        }
      }
      __syncthreads();
    }
  }
}

#define MHC_COOP_PARAMS                                                                          \
  const uint16_t *__restrict__ x, const uint16_t *__restrict__ y, const float *__restrict__ Hq_in, \
      const float *__restrict__ Hr_in, uint16_t *__restrict__ xn, const float *__restrict__ bias,  \
      uint16_t *__restrict__ h, float *__restrict__ H_pre, float *__restrict__ H_post,             \
      float *__restrict__ H_res, const float *__restrict__ phi, uint64_t *ctr, uint64_t *rec,      \
      int64_t T, int Q, uint32_t tag, int iters, float eps, float a_pre, float a_post, float a_res
#define MHC_COOP_ARGS \
  x, y, Hq_in, Hr_in, xn, bias, h, H_pre, H_post, H_res, phi, ctr, rec, T, Q, tag, iters, eps, a_pre, a_post, a_res

// hc_pre (y, Hq_in, Hr_in, xn unused)
template <int S>
__global__ __launch_bounds__(kThreads, 1) void hc_pre_coop_kernel(MHC_COOP_PARAMS) {
  coop_body<S, false>(MHC_COOP_ARGS);
}

// hc_post of a layer fused with hc_pre of the next
template <int S>
__global__ __launch_bounds__(kThreads, 1) void hc_post_pre_coop_kernel(MHC_COOP_PARAMS) {
  coop_body<S, true>(MHC_COOP_ARGS);
}

#undef MHC_COOP_PARAMS
#undef MHC_COOP_ARGS

// Tags of the exchange records: one per call, not repeated for 2^31 calls in
// a process; the top bit is set so that zeroed memory never matches.
uint32_t next_tag() {
  static std::atomic<uint32_t> counter{
      (uint32_t)((uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761u)};
  return counter.fetch_add(1, std::memory_order_relaxed) | 0x80000000u;
}

}  // namespace coop

// ------------------------------------------------------------------ host ---

bool pre_coop_eligible(const mhc_desc& d) {
  return d.N == 4 && d.io == kBF16 && (d.D == 5120 || d.D == 2560);
}

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

size_t pre_coop_workspace_bytes(const mhc_desc& d) {
  const size_t S = (size_t)(d.D / coop::kSliceD);
  const size_t ntiles = (size_t)((d.T + coop::kTM - 1) / coop::kTM);
  return coop::kHeader + align256(ntiles * S * coop::kRecWords * sizeof(uint64_t));
}

namespace {

template <bool FUSED>
hipError_t launch_coop(const mhc_desc& d, const void* x, const void* y, const float* Hq_in,
                       const float* Hr_in, void* x_next, const float* phi, const float* bias, void* h,
                       float* H_pre, float* H_post, float* H_res, void* ws, hipStream_t s) {
  const int S = d.D / coop::kSliceD;
  const int Q = device_cu_count() / S;
  if (Q < 1) return hipErrorInvalidConfiguration;
  char* w = static_cast<char*>(ws);
  uint64_t* ctr = reinterpret_cast<uint64_t*>(w);
  uint64_t* rec = reinterpret_cast<uint64_t*>(w + coop::kHeader);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const uint16_t* yp = static_cast<const uint16_t*>(y);
  uint16_t* xnp = static_cast<uint16_t*>(x_next);
  uint16_t* hp = static_cast<uint16_t*>(h);
  const uint32_t tag = coop::next_tag();
  const dim3 grid((unsigned)(Q * S)), block(coop::kThreads);
  if (S == 16)
    hipLaunchKernelGGL((FUSED ? coop::hc_post_pre_coop_kernel<16> : coop::hc_pre_coop_kernel<16>), grid, block, 0, s, xp, yp, Hq_in, Hr_in,
                       xnp, bias, hp, H_pre, H_post, H_res, phi, ctr, rec, (int64_t)d.T, Q, tag,
                       d.sinkhorn_iters, d.eps, d.alpha_pre, d.alpha_post, d.alpha_res);
  else
    hipLaunchKernelGGL((FUSED ? coop::hc_post_pre_coop_kernel<8> : coop::hc_pre_coop_kernel<8>), grid, block, 0, s, xp, yp, Hq_in, Hr_in,
                       xnp, bias, hp, H_pre, H_post, H_res, phi, ctr, rec, (int64_t)d.T, Q, tag,
                       d.sinkhorn_iters, d.eps, d.alpha_pre, d.alpha_post, d.alpha_res);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pre_coop(const mhc_desc& d, const void* x, const float* phi, const float* bias,
                           void* h, float* H_pre, float* H_post, float* H_res, void* ws,
                           hipStream_t s) {
  return launch_coop<false>(d, x, nullptr, nullptr, nullptr, nullptr, phi, bias, h, H_pre, H_post,
                            H_res, ws, s);
}

hipError_t launch_post_pre_coop(const mhc_desc& d, const void* x, const void* y, const float* H_post_in,
                                const float* H_res_in, void* x_next, const float* phi, const float* bias,
                                void* h, float* H_pre, float* H_post, float* H_res, void* ws,
                                hipStream_t s) {
  return launch_coop<true>(d, x, y, H_post_in, H_res_in, x_next, phi, bias, h, H_pre, H_post, H_res,
                           ws, s);
}

}  // namespace mhc
