// hc_pre forward, bf16 I/O, N = 4, D = 2560 or 5120: whole token tiles held
// on chip, each token's reduction split over a group of four workgroups.
//
// The computation is the §5.3 "mHC" formula block of the openPangu 2.0
// analysis: per token the sum of squares and the 24 projections of the
// flattened 4·D state, then rstd, the gates, Sinkhorn, and the collapse
// h = Σ_n H_pre[n]·x[n], which needs the whole-token reduction first.
//
// Layout on the chip:
//  * A tile is M = 16, 32 or 64 consecutive tokens.  A group of S = 8 or 4
//    workgroups (one per CU) takes a tile; workgroup `slice` owns the d range
//    [slice·D/S, (slice+1)·D/S) of all four streams, so the collapse of its
//    d range needs no other workgroup's x.  Its share of the tile stays in
//    VGPRs (and AGPRs) from the projection to the collapse: x crosses HBM
//    once.
//  * Four or eight waves; a wave owns 160 d of the slice (all four streams:
//    20 steps of 32 k) for 16·TBW tokens.  Its registers hold x as the A
//    fragments of v_mfma_f32_16x16x32_bf16 (lane: token row l mod 16, 8
//    consecutive d), so the four streams of a (token, d) sit in one lane and
//    the collapse is lane-local.
//  * φ keeps fp32 accuracy as two bf16 parts, φ = hi + lo (x is exact in
//    bf16, so x·hi + x·lo carries about 16 mantissa bits of φ into an fp32
//    accumulation).  A packing kernel writes both parts once per call in the
//    B-fragment order of the matrix cores: per 32-k step three 16-column
//    groups [hi 0..15 | hi 16..23, lo 0..7 | lo 8..23], 3 KB, which each wave
//    streams from L2 into a ring of LDS slots with direct-to-LDS loads, five
//    steps ahead, beside its x loads.
//  * After the last step each workgroup sums its waves' partials in LDS (fixed
//    order), publishes 25 numbers per token (24 raw projections and the sum
//    of squares) as tagged 64-bit records, and gathers the other slices':
//    pre[4] and the sum of squares of every token of the tile, and post[4],
//    res[16] of the M/S tokens it finishes.  Every workgroup derives rstd and
//    H_pre of all M tokens (the same arithmetic in the same order, so the
//    same bits); the finishing one also runs the gates and Sinkhorn (sixteen
//    lanes per token, one H_res entry each, DPP row and column sums) and
//    writes H_pre, H_post, H_res.
//  * Records are 64-bit words (value | 32-bit call tag) written and read with
//    relaxed device-scope accesses: a reader that sees the tag sees the
//    value.  The tag is a per-process seed plus a per-device call number that
//    the packing kernel of the same call takes from a device-wide counter and
//    stores in the workspace header, so no two calls of the process on a
//    device share a tag (until 2^31 calls) whatever memory their workspaces
//    used before, and a replayed HIP graph gets a new tag on every replay.
//    Workgroup b owns slice b mod S and takes its group from a ticket of
//    that slice's counter (S counters, 256 bytes apart): group g is the
//    g-th workgroup of every slice to start, so the earliest groups are
//    complete as soon as each slice has a workgroup running, and finish
//    whatever else holds the chip.  (One counter for all slices serialised
//    the grid's atomics on one address: 3.7 µs a call at T = 4096, D = 5120
//    on MI355X.)  Each wait is bounded and one that runs out writes NaN for
//    the tile's tokens.
#include "mhc_coef.h"
#include "mhc_internal.h"

#include <type_traits>

namespace mhc {
namespace tile {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kN = 4;
constexpr int kC = 24;               // logits: pre[4] post[4] res[16]
constexpr int kE = kC + 1;           // record entries per token: 24 projections, sum of squares
constexpr int kSteps = 20;           // 32-k MFMA steps per wave
constexpr int kDB = kSteps / kN;     // 32-d blocks per stream per wave
constexpr int kWaveD = kDB * 32;     // d per wave (160)
constexpr int kCG = 3;               // B column groups per step
constexpr int kCols = 16 * kCG;      // hi[0..24) then lo[0..24)
constexpr int kAhead = 5;            // steps whose loads are in flight
constexpr int kCounters = 8;         // ticket counters at most, one per 256 bytes
// workspace bytes: ticket counter c at byte 256·c, a copy of the call number
// at byte 256·c + 8
constexpr int kHeader = 256 * kCounters;
constexpr uint32_t kSpinLimit = 1u << 20;  // polls of one record wait before it gives up
// calls of the split-K hc_pre on this device so far (one copy per device)
__device__ uint64_t g_calls = 0;
static_assert(kSteps % kN == 0, "each step is 32 d of one stream");

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
// 16-byte load: per-lane offset, wave-uniform offset.
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16-byte store of h with the non-temporal hint (h is written once and not
// read back by this call; measured on MI355X it shortens the kernel by about
// 1.5 µs at T = 4096, D = 5120).  The scalar offset is the literal 0 (a wide
// buffer store with a register scalar offset has lost data on this chip).
__device__ __forceinline__ void st16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint4 v) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{v.x, v.y, v.z, v.w}, r, (int)voff, 0, 2);
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16·i.  Counted by vmcnt like any vector-memory load.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, (int)voff, (int)soff, 0, 0);
}
// The three φ fragments of one step, read back from LDS.  Written as one asm
// block so that the compiler, which would otherwise wait for every pending
// LDS DMA (vmcnt(0)) before any LDS read, leaves the ring in flight; the
// caller waits for this step's DMA with an exact vmcnt first.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
template <int OFF>
__device__ __forceinline__ void lds_read3(uint32_t addr, u32x4_t& a, u32x4_t& b, u32x4_t& c) {
  asm volatile(
      "ds_read_b128 %0, %3 offset:%4\n\t"
      "ds_read_b128 %1, %3 offset:%5\n\t"
      "ds_read_b128 %2, %3 offset:%6\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=v"(a), "=v"(b), "=v"(c)
      : "v"(addr), "i"(OFF), "i"(OFF + 1024), "i"(OFF + 2048)
      : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ float dot2(uint32_t w, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, w);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, c, false);
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
__device__ __forceinline__ bool tagged(uint64_t e, uint32_t tag) { return (uint32_t)(e >> 32) == tag; }

// A zero the compiler cannot see through, produced inside a loop: indices
// derived from it are recomputed where they are used instead of being hoisted
// out of the loop and held in registers for the whole kernel.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("s_mov_b32 %0, 0" : "=s"(z));
  return z;
}

template <typename F, int... J>
__device__ __forceinline__ void each(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}

// ---------------------------------------------------------------- φ pack ---
// Fragment (dw, j, cg), lane l = 16·gq + c holds 8 bf16: for k rows
// n·D + 160·WD·sl + 32·(jd·WD + wd) + 8·gq + v (v = 0..7; n = j / 5,
// jd = j mod 5; wave wd of slice sl, dw = sl·WD + wd; WD waves along d) of
// column cg = 0: hi(c); cg = 1: c < 8 ? hi(16 + c) : lo(c − 8); cg = 2:
// lo(8 + c); hi = bf16(φ), lo = bf16(φ − hi), both rounded to nearest even.
// A workgroup packs kPackItems consecutive (dw, j) fragments: each is 32
// rows, 3 KB of consecutive φ, read as one coalesced run into LDS (every
// item's loads issued before the first is used); the three fragments (3 KB)
// go out the same way.  One item a workgroup (640 workgroups at D = 5120)
// measured 0.6 µs faster per hc_pre call on MI355X than four (160).
constexpr int kPackThreads = kCG * 64;
constexpr int kPackItems = 1;
__global__ __launch_bounds__(kPackThreads) void phi_pack_tile_kernel(const float* __restrict__ phi,
                                                                     uint4* __restrict__ out, int D, int WD,
                                                                     uint64_t* call_no) {
  // every call takes a number of its own from the device-wide counter, before
  // the main kernel starts, and leaves it in its workspace header: the main
  // kernel tags its records with it (also on every replay of a HIP graph)
  // (one copy beside each slice's ticket counter, so that the main kernel's
  // workgroups read it from S addresses rather than one)
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    const uint64_t v = __hip_atomic_fetch_add(&g_calls, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1;
#pragma unroll
    for (int c = 0; c < kCounters; ++c)
      __hip_atomic_store(call_no + 32 * c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __shared__ float rows_s[kPackItems][32 * kC];
  static_assert(32 * kC == 4 * kPackThreads, "one float4 per thread and item");
  const int nitems = D / kWaveD * kSteps;
  float4 v[kPackItems];
#pragma unroll
  for (int q = 0; q < kPackItems; ++q) {
    const int item = blockIdx.x * kPackItems + q;
    v[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (item < nitems) {
      const int j = item % kSteps, dw = item / kSteps;
      const int n = j / kDB, jd = j % kDB;
      // wave wd of slice sl takes the slice's 32-d blocks wd, wd + WD, wd + 2·WD, …
      const int sl = dw / WD, wd = dw % WD;
      const int64_t k0 = (int64_t)n * D + (int64_t)sl * (WD * kWaveD) + 32 * (jd * WD + wd);
      v[q] = reinterpret_cast<const float4*>(phi + k0 * kC)[threadIdx.x];
    }
  }
#pragma unroll
  for (int q = 0; q < kPackItems; ++q) reinterpret_cast<float4*>(rows_s[q])[threadIdx.x] = v[q];
  __syncthreads();
  const int cg = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = lane & 15, gq = lane >> 4;
  int col;
  bool lo;
  if (cg == 0) {
    col = c;
    lo = false;
  } else if (cg == 1) {
    col = c < 8 ? 16 + c : c - 8;
    lo = c >= 8;
  } else {
    col = 8 + c;
    lo = true;
  }
#pragma unroll
  for (int q = 0; q < kPackItems; ++q) {
    const int item = blockIdx.x * kPackItems + q;
    if (item >= nitems) break;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float f0 = rows_s[q][(8 * gq + e) * kC + col], f1 = rows_s[q][(8 * gq + e + 1) * kC + col];
      uint32_t hw = pack_bf16x2(f0, f1);
      if (lo) hw = pack_bf16x2(f0 - bf16_lo(hw), f1 - bf16_hi(hw));
      w[e / 2] = hw;
    }
    out[(int64_t)item * kPackThreads + threadIdx.x] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ------------------------------------------------------------ main kernel ---
// S workgroups per group, W waves per workgroup: WD along d (D = S·WD·160),
// W/WD along tokens, each with TBW 16-token blocks: M = 16·TBW·W/WD tokens per
// tile.  With four waves a wave holds up to 320 registers of x (VGPRs and
// AGPRs), so a tile can be 64 tokens and φ is read once per 64 tokens.
template <int IO, int S, int W, int WD, int TBW>
__global__ __launch_bounds__(W * 64, 1) void hc_pre_tile_kernel(
    const char* __restrict__ x, const uint4* __restrict__ phip, const float* __restrict__ bias,
    char* __restrict__ h, float* __restrict__ H_pre, float* __restrict__ H_post,
    float* __restrict__ H_res, uint64_t* ctr, uint64_t* rec, int64_t T, int Q, uint32_t tag,
    int iters, float eps, float a_pre, float a_post, float a_res, const float* __restrict__ alpha_dev,
    uint32_t spin_limit, int drop_slice) {
  if (alpha_dev != nullptr) {  // the gate scalars are held on the device (trained α)
    a_pre = alpha_dev[0];
    a_post = alpha_dev[1];
    a_res = alpha_dev[2];
  }
  constexpr int kS = S, kWaves = W, kThreads = W * 64;
  constexpr int WT = kWaves / WD;
  constexpr int M = 16 * TBW * WT;      // tokens per tile
  constexpr int F = M / kS;             // tokens each workgroup finishes
  constexpr int D = kS * WD * kWaveD;
  constexpr int K = kN * D;
  static_assert(M % kS == 0 && F % 4 == 0 && F / 4 <= kWaves, "the last F/4 waves run the Sinkhorn");
  // bytes per element of x and h, and 16-byte words of x per lane and step
  // (fp32 keeps x in full: the collapse needs it exact)
  constexpr int E = IO == kF32 ? 4 : 2;
  constexpr int XW = E / 2;

  // φ ring of each wave (kAhead steps × 3 fragments), in the same LDS as the
  // per-wave partials [col][token] that replace it after the last step
  // (cols 48..51: sums of squares of the four lane groups)
  constexpr int kRingBytes = kWaves * kAhead * kCG * 1024;
  constexpr int kRedBytes = kWaves * TBW * (kCols + 4) * 16 * 4;
  __shared__ __align__(16) char ring_s[kRingBytes > kRedBytes ? kRingBytes : kRedBytes];
  float(*red)[TBW][kCols + 4][16] = reinterpret_cast<float(*)[TBW][kCols + 4][16]>(ring_s);
  __shared__ float gath[kE][M];                       // slice sums: all tokens' pre, ss; finished tokens' rest
  __shared__ __align__(16) float hpre_s[M][kN];
  __shared__ float fin_s[F][kN * kN];                 // res logits of the tokens this workgroup finishes
  __shared__ float bias_s[kC];
  __shared__ int ticket_s;
  __shared__ uint32_t tag_s;

  if (threadIdx.x == 0) {
    // the grid is Q·kS workgroups, Q of each slice: each call adds exactly Q
    // to every slice's counter, so the residues mod Q of one call's tickets
    // are each taken once, whatever the counters held
    static_assert(kS <= kCounters, "a counter per slice");
    const int sl = (int)blockIdx.x % kS;
    const uint64_t v = __hip_atomic_fetch_add(ctr + 32 * sl, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // v mod Q in 32-bit arithmetic: (hi·2³² + lo) mod q, with 2³² mod q =
    // ((2³² − 1) mod q + 1) mod q (products stay below q² < 2³²: Q is at
    // most the CU count)
    const uint32_t q = (uint32_t)Q, hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
    const uint32_t p32 = (0xFFFFFFFFu % q + 1u) % q;
    ticket_s = (int)(((hi % q) * p32 + lo % q) % q) * kS + sl;
  } else if (threadIdx.x == kWave) {
    // process seed + this call's number, read by another wave so that its
    // round trip overlaps the ticket's
    const uint64_t cn =
        __hip_atomic_load(ctr + 32 * ((int)blockIdx.x % kS) + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tag_s = (tag + (uint32_t)cn) | 0x80000000u;
  }
  if (threadIdx.x < kC) bias_s[threadIdx.x] = bias[threadIdx.x];
  __syncthreads();
  tag = tag_s;
  const int ticket = ticket_s;
  const int grp = ticket / kS, slice = ticket % kS;
  if (grp >= Q) return;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wd = wave % WD, wt = wave / WD;
  const int row = lane & 15, g = lane >> 4;
  // this wave's 32-d blocks are wd, wd + WD, wd + 2·WD, … of the slice, so that
  // in each step the CU's waves read WD·64 contiguous bytes of every token row
  const int d0 = slice * (WD * kWaveD) + 32 * wd;  // d of this wave's first block
  const int dw = slice * WD + wd;
  const int64_t ntiles = (T + M - 1) / M;
  constexpr float rK = 1.0f / (float)K;

  // φ fragments of this wave: (j, cg) at byte ((dw·kSteps + j)·kCG + cg)·1024 + lane·16
  const __amdgpu_buffer_rsrc_t prs =
      make_rsrc(phip + (int64_t)dw * kSteps * kCG * 64, (uint32_t)(kSteps * kCG * 64 * 16));
  const uint32_t pvoff = (uint32_t)(lane * 16);
  // x: token 16·(wt·TBW + i) + row of the tile, stream n, d0 + 32·WD·jd + 8·g.
  // The token offset stays in the per-lane offset, which the descriptor's
  // range check always covers, so rows past the tile's end read zeros; the
  // offset within the token row, n·D + 32·WD·jd (a constant per step), goes
  // into the scalar offset.
  uint32_t xvoff[TBW];
#pragma unroll
  for (int i = 0; i < TBW; ++i) xvoff[i] = (uint32_t)(((16 * (wt * TBW + i) + row) * K + d0 + 8 * g) * E);

  uint4 xr[kSteps][TBW][XW];
  char* const ring_w = ring_s + wave * (kAhead * kCG * 1024);  // this wave's φ ring
  const uint32_t ring_lane = (uint32_t)(reinterpret_cast<uintptr_t>(ring_w) & 0xFFFFFFFFu) + lane * 16;

  auto tile_rows = [&](int64_t tl) { return (int)(T - tl * M < M ? T - tl * M : M); };
  auto x_rsrc = [&](int64_t tl) { return make_rsrc(x + tl * M * K * E, (uint32_t)tile_rows(tl) * K * E); };
  // step J's loads: x into its registers, then φ into ring slot J mod kAhead
  auto issue = [&](auto jc, __amdgpu_buffer_rsrc_t xrs) {
    constexpr int J = decltype(jc)::value;
    constexpr int n = J / kDB, jd = J % kDB;
#pragma unroll
    for (int i = 0; i < TBW; ++i)
#pragma unroll
      for (int w = 0; w < XW; ++w) xr[J][i][w] = ld16(xrs, xvoff[i] + 16 * w, (uint32_t)((n * D + 32 * WD * jd) * E));
#pragma unroll
    for (int cg = 0; cg < kCG; ++cg)
      dma16(prs, ring_w + ((J % kAhead) * kCG + cg) * 1024, pvoff, (uint32_t)((J * kCG + cg) * 1024));
  };
  static_assert(kAhead == kDB, "the collapse of d block j frees the registers of the next tile's step j");

  // the first tile's first steps; every later tile's are issued by the collapse
  // of the tile before it
  if (grp < ntiles) {
    const __amdgpu_buffer_rsrc_t xrs = x_rsrc(grp);
    each([&](auto jc) { issue(jc, xrs); __builtin_amdgcn_sched_barrier(0); },
         std::make_integer_sequence<int, kAhead>{});
  }
  for (int64_t tl = grp; tl < ntiles; tl += Q) {
    const int64_t t0 = tl * M;
    const int rows = tile_rows(tl);
    const __amdgpu_buffer_rsrc_t xrs = x_rsrc(tl);

    f32x4_t acc[TBW][kCG];
    float ss[TBW];
#pragma unroll
    for (int i = 0; i < TBW; ++i) {
      ss[i] = 0.f;
#pragma unroll
      for (int cg = 0; cg < kCG; ++cg) acc[i][cg] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    each(
        [&](auto jc) {
          constexpr int J = decltype(jc)::value;
          // loads complete in issue order: step J's are done once no more than
          // the later steps' loads are outstanding (h stores issued between a
          // tile's first steps only make this wait longer)
          constexpr int later = (kSteps - 1 - J < kAhead - 1 ? kSteps - 1 - J : kAhead - 1) * (TBW * XW + kCG);
          wait_vmcnt<later>();
          u32x4_t b0, b1, b2;
          lds_read3<(J % kAhead) * kCG * 1024>(ring_lane, b0, b1, b2);
          const uint4 bf[kCG] = {make_uint4(b0.x, b0.y, b0.z, b0.w), make_uint4(b1.x, b1.y, b1.z, b1.w),
                                 make_uint4(b2.x, b2.y, b2.z, b2.w)};
#pragma unroll
          for (int i = 0; i < TBW; ++i) {
            if constexpr (IO == kF32) {
              // x = hi + lo to about 16 mantissa bits (both parts exact in
              // bf16): hi meets every column group, lo the groups with φ's
              // high parts (x·lo·φ_lo is below fp32 rounding)
              float v[8];
              const uint4 a0 = xr[J][i][0], a1 = xr[J][i][1];
              v[0] = __uint_as_float(a0.x); v[1] = __uint_as_float(a0.y);
              v[2] = __uint_as_float(a0.z); v[3] = __uint_as_float(a0.w);
              v[4] = __uint_as_float(a1.x); v[5] = __uint_as_float(a1.y);
              v[6] = __uint_as_float(a1.z); v[7] = __uint_as_float(a1.w);
              const uint4 ahi = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
              const uint4 alo = pack_bf16x8_rest(v, ahi);
#pragma unroll
              for (int cg = 0; cg < kCG; ++cg) acc[i][cg] = mfma(ahi, bf[cg], acc[i][cg]);
              acc[i][0] = mfma(alo, bf[0], acc[i][0]);
              acc[i][1] = mfma(alo, bf[1], acc[i][1]);
#pragma unroll
              for (int e = 0; e < 8; ++e) ss[i] = __builtin_fmaf(v[e], v[e], ss[i]);
            } else {
              const uint4 a = xr[J][i][0];
#pragma unroll
              for (int cg = 0; cg < kCG; ++cg) acc[i][cg] = mfma(a, bf[cg], acc[i][cg]);
              ss[i] = dot2(a.x, ss[i]);
              ss[i] = dot2(a.y, ss[i]);
              ss[i] = dot2(a.z, ss[i]);
              ss[i] = dot2(a.w, ss[i]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (J + kAhead < kSteps) issue(std::integral_constant<int, J + kAhead>{}, xrs);
          __builtin_amdgcn_sched_barrier(0);
        },
        std::make_integer_sequence<int, kSteps>{});
    __syncthreads();  // every wave is past its ring before the partials overwrite it

    // the rest of the tile works from indices recomputed here (see opaque_zero)
    const int tid = (int)threadIdx.x + opaque_zero();
    const int lane2 = tid & 63, row2 = lane2 & 15, g2 = lane2 >> 4;

    // this wave's partials: D layout of the MFMA result, lane (c, g) holds
    // tokens 4g..4g+3 of column c of its group
#pragma unroll
    for (int i = 0; i < TBW; ++i) {
#pragma unroll
      for (int cg = 0; cg < kCG; ++cg)
#pragma unroll
        for (int q = 0; q < 4; ++q) red[wave][i][cg * 16 + row2][4 * g2 + q] = acc[i][cg][q];
      red[wave][i][kCols + g2][row2] = ss[i];
    }
    __syncthreads();

    // publish: entry e of token t summed over the waves of its token block in
    // a fixed order (hi and lo parts of a column added per wave); all of an
    // item's LDS reads are issued before the first add
    uint64_t* mine = rec + (tl * kS + slice) * (int64_t)(kE * M);
    for (int u = tid; u < kE * M; u += kThreads) {
      const int e = u / M, t = u % M;
      const int b = t >> 4, tt = t & 15, wt2 = b / TBW, i = b % TBW;
      float v = 0.f;
      if (e < kC) {
        float va[WD], vb[WD];
#pragma unroll
        for (int w = 0; w < WD; ++w) {
          va[w] = red[wt2 * WD + w][i][e][tt];
          vb[w] = red[wt2 * WD + w][i][kC + e][tt];
        }
#pragma unroll
        for (int w = 0; w < WD; ++w) v += va[w] + vb[w];
      } else {
        float va[WD][4];
#pragma unroll
        for (int w = 0; w < WD; ++w)
#pragma unroll
          for (int q = 0; q < 4; ++q) va[w][q] = red[wt2 * WD + w][i][kCols + q][tt];
#pragma unroll
        for (int w = 0; w < WD; ++w) v += (va[w][0] + va[w][1]) + (va[w][2] + va[w][3]);
      }
      if (t < rows && slice != drop_slice) put(mine + u, entry(v, tag));
    }

    // gather: (a) pre[4] and the sum of squares of every token, (b) post and
    // res of the tokens this workgroup finishes; slices summed in order
    const uint64_t* tile_rec = rec + tl * kS * (int64_t)(kE * M);
    constexpr int kA = 5 * M, kB = (kC - kN) * F;
    for (int u = tid; u < kA + kB; u += kThreads) {
      int e, t;
      if (u < kA) {
        e = u / M;
        t = u % M;
        if (e == kN) e = kC;  // the sum of squares
      } else {
        e = kN + (u - kA) / F;
        t = slice * F + (u - kA) % F;
      }
      float v = 0.f;
      if (t < rows) {
        uint64_t r[kS];
        uint32_t spins = 0;
        bool ok;
        do {
          ok = true;
#pragma unroll
          for (int sl = 0; sl < kS; ++sl) {
            r[sl] = get(tile_rec + (int64_t)sl * kE * M + e * M + t);
            ok = ok && tagged(r[sl], tag);
          }
          if (!ok) __builtin_amdgcn_s_sleep(2);
        } while (!ok && ++spins < spin_limit);
        // a member that never published poisons the tile's values (NaN)
        v = ok ? 0.f : __builtin_nanf("");
#pragma unroll
        for (int sl = 0; sl < kS; ++sl) v += __uint_as_float((uint32_t)r[sl]);
      }
      gath[e][t] = v;
    }
    __syncthreads();

    // rstd and H_pre of every token (H_pre written by the finishing slice);
    // for the finished tokens also H_post and the res logits
    for (int u = tid; u < M * kN + (kN * kN + kN) * F; u += kThreads) {
      if (u < M * kN) {
        const int t = u >> 2, n = u & 3;
        float hp = 0.f;
        if (t < rows) {
          const float rstd = __builtin_amdgcn_rsqf(gath[kC][t] * rK + eps);
          hp = fast_sigmoid(a_pre * (rstd * gath[n][t]) + bias_s[n]);
          if (t / F == slice) H_pre[(t0 + t) * kN + n] = hp;
        }
        hpre_s[t][n] = hp;
      } else if (u < M * kN + kN * kN * F) {
        const int v = u - M * kN;
        const int f = v >> 4, c = v & 15;
        const int t = slice * F + f;
        if (t < rows) {
          const float rstd = __builtin_amdgcn_rsqf(gath[kC][t] * rK + eps);
          fin_s[f][c] = a_res * (rstd * gath[2 * kN + c][t]) + bias_s[2 * kN + c];
        }
      } else {
        const int v = u - M * kN - kN * kN * F;
        const int f = v >> 2, n = v & 3;
        const int t = slice * F + f;
        if (t < rows) {
          const float rstd = __builtin_amdgcn_rsqf(gath[kC][t] * rK + eps);
          H_post[(t0 + t) * kN + n] = 2.0f * fast_sigmoid(a_post * (rstd * gath[kN + n][t]) + bias_s[kN + n]);
        }
      }
    }
    __syncthreads();

    // collapse from registers, h[t][d] = Σ_n H_pre[t][n]·x[t][n][d], one d
    // block at a time; the registers of block jd then take the next tile's
    // step jd (whose φ goes to the ring, free since the publish)
    const int64_t tn = tl + Q;
    const bool more = tn < ntiles;
    const __amdgpu_buffer_rsrc_t xrs_next = x_rsrc(more ? tn : tl);
    const __amdgpu_buffer_rsrc_t hrs = make_rsrc(h + t0 * D * E, (uint32_t)rows * D * E);
    // LDS reads before the first DMA of the next tile is issued (the compiler
    // waits for every pending LDS DMA before an LDS read)
    float hv[TBW][kN];
#pragma unroll
    for (int i = 0; i < TBW; ++i) {
      const float4 hw = *reinterpret_cast<const float4*>(&hpre_s[16 * (wt * TBW + i) + row2][0]);
      hv[i][0] = hw.x;
      hv[i][1] = hw.y;
      hv[i][2] = hw.z;
      hv[i][3] = hw.w;
    }
    constexpr int kSkWaves = (F + 3) / 4;
    const int sk_u = (wave - (kWaves - kSkWaves)) * 4 + (lane2 >> 4);
    const int sk_i = (lane2 >> 2) & 3, sk_j = lane2 & 3;
    const bool sk_live = wave >= kWaves - kSkWaves && sk_u < F && slice * F + sk_u < rows;
    float sk_m = sk_live ? fin_s[sk_u][sk_i * kN + sk_j] : 0.f;
    each(
        [&](auto jc) {
          constexpr int JD = decltype(jc)::value;
#pragma unroll
          for (int i = 0; i < TBW; ++i) {
            const int t = 16 * (wt * TBW + i) + row2;
            const float* hvi = hv[i];
            float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            const uint32_t hoff = (uint32_t)((t * D + slice * (WD * kWaveD) + 32 * (JD * WD + wd) + 8 * g2) * E);
            if constexpr (IO == kF32) {
#pragma unroll
              for (int n = 0; n < kN; ++n) {
                const uint4 a0 = xr[n * kDB + JD][i][0], a1 = xr[n * kDB + JD][i][1];
                o[0] += hvi[n] * __uint_as_float(a0.x);
                o[1] += hvi[n] * __uint_as_float(a0.y);
                o[2] += hvi[n] * __uint_as_float(a0.z);
                o[3] += hvi[n] * __uint_as_float(a0.w);
                o[4] += hvi[n] * __uint_as_float(a1.x);
                o[5] += hvi[n] * __uint_as_float(a1.y);
                o[6] += hvi[n] * __uint_as_float(a1.z);
                o[7] += hvi[n] * __uint_as_float(a1.w);
              }
              st16(hrs, hoff, make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                                         __float_as_uint(o[3])));
              st16(hrs, hoff + 16, make_uint4(__float_as_uint(o[4]), __float_as_uint(o[5]),
                                              __float_as_uint(o[6]), __float_as_uint(o[7])));
            } else {
#pragma unroll
              for (int n = 0; n < kN; ++n) {
                const uint4 a = xr[n * kDB + JD][i][0];
                o[0] += hvi[n] * bf16_lo(a.x);
                o[1] += hvi[n] * bf16_hi(a.x);
                o[2] += hvi[n] * bf16_lo(a.y);
                o[3] += hvi[n] * bf16_hi(a.y);
                o[4] += hvi[n] * bf16_lo(a.z);
                o[5] += hvi[n] * bf16_hi(a.z);
                o[6] += hvi[n] * bf16_lo(a.w);
                o[7] += hvi[n] * bf16_hi(a.w);
              }
              st16(hrs, hoff,
                   make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                              pack_bf16x2(o[6], o[7])));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if (more) issue(jc, xrs_next);
          __builtin_amdgcn_sched_barrier(0);
        },
        std::make_integer_sequence<int, kDB>{});

    // Sinkhorn of the finished tokens, one H_res entry per lane: lane 16u + 4i
    // + jj of the last F/4 waves holds row i, column jj of token u; row sums
    // over the lane quad, column sums over the rotations by 4 and 8 of the
    // 16-lane row; while the next tile's first loads are in flight
    if (wave >= kWaves - kSkWaves) {
      float m = sk_m;
      float mx = fmaxf(m, dpp<0xB1>(m));   // quad_perm(1,0,3,2)
      mx = fmaxf(mx, dpp<0x4E>(mx));       // quad_perm(2,3,0,1)
      m = expf(m - mx);
      for (int it = 0; it < iters; ++it) {
        float r = m + dpp<0xB1>(m);
        r += dpp<0x4E>(r);
        m *= __builtin_amdgcn_rcpf(r);
        float c = m + dpp<0x124>(m);  // row_ror:4
        c += dpp<0x128>(c);           // row_ror:8
        m *= __builtin_amdgcn_rcpf(c);
      }
      if (sk_live) H_res[((t0 + slice * F + sk_u) * kN + sk_i) * kN + sk_j] = m;
    }
    // no barrier here: the next LDS writes (the partials, after the next
    // tile's steps) follow a barrier every wave reaches after this point
  }
}

}  // namespace tile

// ------------------------------------------------------------------ host ---

namespace {

// Failure injection for tests (mhc_test_exchange_fault): off unless set.
struct ExchangeFault {
  uint32_t spin_limit = tile::kSpinLimit;
  int drop_slice = -1;
};
ExchangeFault g_fault;

// One instantiation of the kernel: S slices, W waves, WD along d, TBW blocks.
struct TileConfig {
  int s = 0, w = 0, wd = 0, tbw = 0;  // s = 0: not eligible
  int64_t m = 0;
};

static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

TileConfig pick_tile(const mhc_desc& d) {
  TileConfig best;
  if (d.N != 4 || (d.io != kBF16 && d.io != kF32) || (d.D != 5120 && d.D != 2560)) return best;
  static const TileConfig kBf16[] = {
      // D = 5120: 8 slices × 4 waves × 64 tokens; 4 × 8 waves × 32; 4 × 8 × 16
      {8, 4, 4, 4, 64}, {4, 8, 8, 2, 32}, {4, 8, 8, 1, 16},
      // D = 2560: 4 slices × 4 waves × 64 tokens; 4 × 8 waves (4 along d) × 32
      {4, 4, 4, 4, 64}, {4, 8, 4, 1, 32}};
  // fp32 x takes twice the registers: 32-token tiles, 8 slices at D = 5120,
  // 4 at D = 2560
  static const TileConfig kF32Cands[] = {{8, 4, 4, 2, 32}, {4, 4, 4, 2, 32}};
  const TileConfig* cands = d.io == kF32 ? kF32Cands : kBf16;
  const int ncands = d.io == kF32 ? 2 : 5;
  const int cus = device_cu_count();
  // the one that leaves each CU the least work over the call (tiles per
  // group × tile size / slices); ties: the larger tile, which reads φ less
  int64_t best_work = -1;
  for (int ci = 0; ci < ncands; ++ci) {
    const TileConfig& c = cands[ci];
    if (c.s * c.wd * tile::kWaveD != d.D) continue;
    const int64_t q = cus / c.s;
    if (q < 1) continue;
    const int64_t ntiles = (d.T + c.m - 1) / c.m;
    const int64_t work = (ntiles + q - 1) / q * c.m / c.s;
    if (best_work < 0 || work < best_work) {
      best_work = work;
      best = c;
    }
  }
  return best;
}

size_t phi_pack_bytes(const mhc_desc& d) {
  return align256((size_t)(d.D / tile::kWaveD) * tile::kSteps * tile::kCG * 64 * sizeof(uint4));
}

}  // namespace

bool pre_tile_eligible(const mhc_desc& d) { return pick_tile(d).s != 0; }

void set_exchange_fault(int drop_slice, uint32_t spin_limit) {
  g_fault.drop_slice = drop_slice;
  g_fault.spin_limit = drop_slice >= 0 ? spin_limit : tile::kSpinLimit;
}

size_t pre_tile_workspace_bytes(const mhc_desc& d) {
  const TileConfig c = pick_tile(d);
  if (c.s == 0) return 0;
  const size_t ntiles = (size_t)((d.T + c.m - 1) / c.m);
  return tile::kHeader + phi_pack_bytes(d) + align256(ntiles * c.s * tile::kE * (size_t)c.m * sizeof(uint64_t));
}

hipError_t launch_pre_tile(const mhc_desc& d, const void* x, const float* phi, const float* bias, void* h,
                           float* H_pre, float* H_post, float* H_res, void* ws, hipStream_t s) {
  const TileConfig c = pick_tile(d);
  if (c.s == 0) return hipErrorInvalidValue;
  const int Q = device_cu_count() / c.s;
  char* w = static_cast<char*>(ws);
  uint64_t* ctr = reinterpret_cast<uint64_t*>(w);
  uint4* phip = reinterpret_cast<uint4*>(w + tile::kHeader);
  uint64_t* rec = reinterpret_cast<uint64_t*>(w + tile::kHeader + phi_pack_bytes(d));
  const int nitems = d.D / tile::kWaveD * tile::kSteps;
  MHC_LAUNCH(tile::phi_pack_tile_kernel, dim3((unsigned)((nitems + tile::kPackItems - 1) / tile::kPackItems)),
                     dim3(tile::kPackThreads), 0, s, phi, phip, d.D, c.wd, ctr + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t tag = process_tag_seed();
  const dim3 grid((unsigned)(Q * c.s)), block((unsigned)(c.w * 64));
  const char* xp = static_cast<const char*>(x);
  char* hp = static_cast<char*>(h);
#define MHC_TILE_ARGS                                                                                    \
  grid, block, 0, s, xp, phip, bias, hp, H_pre, H_post, H_res, ctr, rec, (int64_t)d.T, Q, tag, d.sinkhorn_iters, \
      d.eps, d.alpha_pre, d.alpha_post, d.alpha_res, d.alpha, g_fault.spin_limit, g_fault.drop_slice
  if (d.io == kF32) {
    if (c.s == 8) MHC_LAUNCH((tile::hc_pre_tile_kernel<kF32, 8, 4, 4, 2>), MHC_TILE_ARGS);
    else MHC_LAUNCH((tile::hc_pre_tile_kernel<kF32, 4, 4, 4, 2>), MHC_TILE_ARGS);
  } else if (c.s == 8) MHC_LAUNCH((tile::hc_pre_tile_kernel<kBF16, 8, 4, 4, 4>), MHC_TILE_ARGS);
  else if (c.w == 4) MHC_LAUNCH((tile::hc_pre_tile_kernel<kBF16, 4, 4, 4, 4>), MHC_TILE_ARGS);
  else if (c.wd == 8 && c.tbw == 2) MHC_LAUNCH((tile::hc_pre_tile_kernel<kBF16, 4, 8, 8, 2>), MHC_TILE_ARGS);
  else if (c.wd == 8) MHC_LAUNCH((tile::hc_pre_tile_kernel<kBF16, 4, 8, 8, 1>), MHC_TILE_ARGS);
  else MHC_LAUNCH((tile::hc_pre_tile_kernel<kBF16, 4, 8, 4, 1>), MHC_TILE_ARGS);
#undef MHC_TILE_ARGS
  return hipGetLastError();
}

}  // namespace mhc
