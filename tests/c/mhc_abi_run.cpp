// Drives the mHC C ABI from host code alone (no Python, no torch): reads the
// inputs a test wrote, runs mhc_pre, mhc_post, mhc_post_bwd and mhc_pre_bwd on
// its own device buffers and stream, then the backward again as mhc_post_bwd
// without dx + mhc_pre_bwd_mix, checks a few argument errors, and writes every
// output back for the test to compare with the Python binding's.
//
// Input file (native byte order): int64 T; int32 N, D, io, iters; float eps,
// alpha_pre, alpha_post, alpha_res; then x[T·N·D], y[T·D] (I/O dtype),
// phi[N·D·C], bias[C] (fp32), dh[T·D], dx_next[T·N·D] (I/O dtype).
// Output file: h, H_pre, H_post, H_res, x_next, dx, dy, dH_post, dH_res,
// dphi, dbias, dalpha, then the mixing pair's dx, in that order, raw.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "mhc.h"

namespace {

[[noreturn]] void die(const char* what) {
  std::fprintf(stderr, "mhc_abi_run: %s\n", what);
  std::exit(1);
}

void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "mhc_abi_run: %s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

void mhc_ok(mhc_status s, const char* what) {
  if (s != MHC_OK) {
    std::fprintf(stderr, "mhc_abi_run: %s: %s\n", what, mhc_status_string(s));
    std::exit(1);
  }
}

struct Buf {
  void* d = nullptr;
  size_t n = 0;
  explicit Buf(size_t bytes) : n(bytes) { hip_ok(hipMalloc(&d, bytes < 256 ? 256 : bytes), "hipMalloc"); }
  ~Buf() { (void)hipFree(d); }
  Buf(const Buf&) = delete;
  Buf& operator=(const Buf&) = delete;
};

void read_into(FILE* f, Buf& b) {
  std::vector<char> h(b.n);
  if (b.n && std::fread(h.data(), 1, b.n, f) != b.n) die("short input file");
  hip_ok(hipMemcpy(b.d, h.data(), b.n, hipMemcpyHostToDevice), "hipMemcpy to device");
}

void write_from(FILE* f, const Buf& b) {
  std::vector<char> h(b.n);
  hip_ok(hipMemcpy(h.data(), b.d, b.n, hipMemcpyDeviceToHost), "hipMemcpy to host");
  if (b.n && std::fwrite(h.data(), 1, b.n, f) != b.n) die("short write");
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3) die("usage: mhc_abi_run INPUT OUTPUT");
  if (mhc_abi_version() != MHC_ABI_VERSION) die("library and header ABI versions differ");
  FILE* in = std::fopen(argv[1], "rb");
  if (!in) die("cannot open input");
  mhc_desc d{};
  int32_t hdr[4];
  float sc[4];
  if (std::fread(&d.T, 8, 1, in) != 1 || std::fread(hdr, 4, 4, in) != 4 || std::fread(sc, 4, 4, in) != 4)
    die("short header");
  d.N = hdr[0];
  d.D = hdr[1];
  d.io = hdr[2];
  d.sinkhorn_iters = hdr[3];
  d.eps = sc[0];
  d.alpha_pre = sc[1];
  d.alpha_post = sc[2];
  d.alpha_res = sc[3];
  const size_t T = (size_t)d.T, N = (size_t)d.N, D = (size_t)d.D, C = N * N + 2 * N;
  const size_t e = d.io == MHC_BF16 ? 2 : 4;
  Buf x(T * N * D * e), y(T * D * e), phi(N * D * C * 4), bias(C * 4), dh(T * D * e), dxn(T * N * D * e);
  read_into(in, x);
  read_into(in, y);
  read_into(in, phi);
  read_into(in, bias);
  read_into(in, dh);
  read_into(in, dxn);
  std::fclose(in);

  Buf h(T * D * e), Hp(T * N * 4), Hq(T * N * 4), Hr(T * N * N * 4), xn(T * N * D * e);
  Buf dx(T * N * D * e), dy(T * D * e), dHq(T * N * 4), dHr(T * N * N * 4), dphi(N * D * C * 4),
      dbias(C * 4), dalpha(4 * 4);
  const size_t wp = mhc_pre_workspace_bytes(&d), wb = mhc_pre_bwd_workspace_bytes(&d);
  Buf ws_pre(wp), ws_bwd(wb);
  hipStream_t s;
  hip_ok(hipStreamCreate(&s), "hipStreamCreate");

  // argument errors are reported before anything runs
  if (mhc_pre(&d, nullptr, (float*)phi.d, (float*)bias.d, h.d, (float*)Hp.d, (float*)Hq.d, (float*)Hr.d,
              ws_pre.d, wp, s) != MHC_ERR_INVALID_ARG)
    die("null x accepted");
  mhc_desc bad = d;
  bad.N = 3;
  if (mhc_post(&bad, x.d, y.d, (float*)Hq.d, (float*)Hr.d, xn.d, s) != MHC_ERR_UNSUPPORTED)
    die("N = 3 accepted");
  if (wb > 0 && mhc_pre_bwd(&d, dh.d, x.d, (float*)phi.d, (float*)bias.d, (float*)dHq.d, (float*)dHr.d, dx.d,
                            (float*)dphi.d, (float*)dbias.d, (float*)dalpha.d, ws_bwd.d, wb - 1, s) !=
                     MHC_ERR_INVALID_ARG)
    die("short workspace accepted");

  mhc_ok(mhc_pre(&d, x.d, (float*)phi.d, (float*)bias.d, h.d, (float*)Hp.d, (float*)Hq.d, (float*)Hr.d,
                 ws_pre.d, wp, s),
         "mhc_pre");
  mhc_ok(mhc_post(&d, x.d, y.d, (float*)Hq.d, (float*)Hr.d, xn.d, s), "mhc_post");
  mhc_ok(mhc_post_bwd(&d, dxn.d, x.d, y.d, (float*)Hq.d, (float*)Hr.d, dx.d, dy.d, (float*)dHq.d,
                      (float*)dHr.d, s),
         "mhc_post_bwd");
  mhc_ok(mhc_pre_bwd(&d, dh.d, x.d, (float*)phi.d, (float*)bias.d, (float*)dHq.d, (float*)dHr.d, dx.d,
                     (float*)dphi.d, (float*)dbias.d, (float*)dalpha.d, ws_bwd.d, wb, s),
         "mhc_pre_bwd");
  // the same backward with hc_post's share of dx formed inside the hc_pre backward
  Buf dx2(T * N * D * e), dy2(T * D * e), dHq2(T * N * 4), dHr2(T * N * N * 4), dphi2(N * D * C * 4),
      dbias2(C * 4);
  mhc_ok(mhc_post_bwd(&d, dxn.d, x.d, y.d, (float*)Hq.d, (float*)Hr.d, nullptr, dy2.d, (float*)dHq2.d,
                      (float*)dHr2.d, s),
         "mhc_post_bwd without dx");
  mhc_ok(mhc_pre_bwd_mix(&d, dh.d, x.d, (float*)phi.d, (float*)bias.d, (float*)dHq2.d, (float*)dHr2.d, dxn.d,
                         (float*)Hr.d, dx2.d, (float*)dphi2.d, (float*)dbias2.d, nullptr, ws_bwd.d, wb, s),
         "mhc_pre_bwd_mix");
  hip_ok(hipStreamSynchronize(s), "hipStreamSynchronize");
  hip_ok(hipStreamDestroy(s), "hipStreamDestroy");

  FILE* out = std::fopen(argv[2], "wb");
  if (!out) die("cannot open output");
  for (const Buf* b : {&h, &Hp, &Hq, &Hr, &xn, &dx, &dy, &dHq, &dHr, &dphi, &dbias}) write_from(out, *b);
  Buf* da = &dalpha;
  da->n = 3 * 4;
  write_from(out, *da);
  write_from(out, dx2);
  std::fclose(out);
  return 0;
}
