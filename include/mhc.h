/*
 * mhc.h — C ABI of the MI355X (gfx950) mHC hot path: hc_pre / hc_post and
 * their backward.
 *
 * What the calls compute (cited by page title and section):
 *
 *   hc_pre   — openPangu 2.0 analysis, §5.3 "mHC" formula block: per token,
 *              x̄ = RMSNorm(x) over the flattened N·D state, logits
 *              ℓ = α_g·(x̄·φ) + b with columns [pre N | post N | res N²],
 *              H_pre = sigmoid(ℓ_pre), H_post = 2·sigmoid(ℓ_post),
 *              H_res = Sinkhorn(exp(reshape(ℓ_res, N, N))) (row-normalise then
 *              column-normalise, `sinkhorn_iters` rounds; 20 in the model table),
 *              and the collapsed sublayer input h = Σ_n H_pre[n]·x[n].
 *   hc_post  — same section (roles of the maps) and the Ascend mHC Triton
 *              article's definition paragraph: x_next[n] = Σ_m H_res[n,m]·x[m]
 *              + H_post[n]·y.
 *   stabilised write-back — the sandwich norm and block post-norm of
 *              openPangu's variant (§5.4); see mhc_post_stable.
 *   backward — the exact derivative of the above; hc_pre's backward recomputes
 *              norm, logits and Sinkhorn from x (the Ascend article's
 *              intra-layer recompute paragraph keeps only the hc_pre input and
 *              the sublayer outputs).
 *
 * Conventions for every call:
 *   - Tensors are device pointers (hipMalloc'd or equivalent), row-major and
 *     contiguous, owned by the caller.  x, y, h, x_next, dh, dx_next, dx, dy
 *     use the I/O dtype `desc->io` (fp32, or bf16 stored as raw 16-bit
 *     words); φ, bias, H_*, dH_*, dφ, dbias, dα are always fp32.
 *   - Layouts: x[T][N][D], y[T][D], h[T][D], x_next[T][N][D], φ[N·D][C] with
 *     C = N²+2N, bias[C], H_pre[T][N], H_post[T][N], H_res[T][N][N] (row =
 *     destination stream).
 *   - Alignment: every pointer 16-byte aligned.
 *   - Work is enqueued on `stream` and runs asynchronously; the library never
 *     allocates, frees or synchronises.  Its only global state is an atomic
 *     per-call counter (calls are thread-safe), besides the per-thread switch
 *     of mhc_trace_kernel_events and the test switch of
 *     mhc_test_exchange_fault.  A workspace must not be in
 *     use by two calls at once.  Outputs are overwritten, except `dx` of mhc_pre_bwd,
 *     which is read-modify-write.
 *   - Errors: argument checks are synchronous and return a status without
 *     launching anything.  A failed launch returns MHC_ERR_HIP.  Device faults
 *     surface at the caller's next synchronisation, as in HIP.
 *   - Aliasing: outputs must not alias inputs (x_next ≠ x, y; dx ≠ dx_next).
 *   - Results are bitwise reproducible for the same inputs, shape and device
 *     (reductions have a fixed order; atomics only order or hand out work,
 *     they never accumulate values).
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MHC_ABI_VERSION 5

typedef enum mhc_dtype { MHC_F32 = 0, MHC_BF16 = 1 } mhc_dtype;

typedef enum mhc_status {
  MHC_OK = 0,
  MHC_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, workspace too small */
  MHC_ERR_UNSUPPORTED = 2, /* N not in {1,2,4,8}, D not a multiple of 8, too many rounds */
  MHC_ERR_HIP = 3,         /* the HIP runtime rejected a launch */
  MHC_ERR_TOO_LARGE = 4    /* mhc_pre_noalloc: the call needs more than MHC_NOALLOC_SCRATCH_BYTES */
} mhc_status;

/* Problem descriptor.  T = tokens (batch × sequence; T = 0 is an empty batch:
 * the token outputs are empty, nothing is launched except the zero fill of
 * the parameter gradients that mhc_pre_bwd, mhc_pre_bwd_mix and
 * mhc_post_stable_bwd write, whose pointers must be valid as usual; the
 * pointers of the empty token tensors are not looked at), N streams, D hidden size
 * (multiple of 8), io = mhc_dtype, sinkhorn_iters ≥ 1 (≤ 64 for mhc_pre_bwd),
 * eps ≥ 0 inside the RMS square root, alpha_* the per-group gate scalars
 * multiplying the normalised projection before the bias is added.  `alpha`,
 * if non-NULL, is a device pointer to the three gate scalars (pre, post, res;
 * fp32, 4-byte aligned) that the kernels read instead of alpha_*: a trained α
 * then stays on the device (no host round trip per step, and a captured graph
 * follows its updates).  Leave it NULL (zero-initialise the struct) to use
 * the scalars. */
typedef struct mhc_desc {
  int64_t T;
  int32_t N;
  int32_t D;
  int32_t io;
  int32_t sinkhorn_iters;
  float eps;
  float alpha_pre;
  float alpha_post;
  float alpha_res;
  const float* alpha;
} mhc_desc;

/* Bytes of device workspace mhc_pre needs (0 if none).  Never fails; returns 0
 * for an invalid descriptor. */
size_t mhc_pre_workspace_bytes(const mhc_desc* desc);

/* hc_pre forward.  Reads x once, writes h[T][D] (I/O dtype) and the fp32
 * coefficients H_pre, H_post, H_res.  `workspace` (may be NULL when
 * mhc_pre_workspace_bytes is 0) is scratch owned by the caller, at least
 * that many bytes, 256-byte aligned; its contents on entry are ignored.  For
 * bf16, N = 4, D = 5120 or 2560 the call first packs φ into the workspace (as
 * bf16 high and low parts, so the projection keeps fp32 accuracy on the
 * matrix cores) and then splits each token's reduction across a group of
 * workgroups that exchange partial sums through the workspace, tagged per
 * call, so two calls that share a workspace must not overlap in time (on one
 * stream they never do).  Those workgroups wait for each other with bounded
 * waits; should one never arrive (e.g. far too few free compute units), the
 * affected tokens get NaN in h and in the coefficients rather than a hang or
 * silently wrong values.  The tag is a number each call takes from a
 * device-wide counter, so the call can be captured in a HIP graph with any
 * workspace, never cleared: every replay tags its records afresh. */
mhc_status mhc_pre(const mhc_desc* desc, const void* x, const float* phi, const float* bias,
                   void* h, float* H_pre, float* H_post, float* H_res,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* hc_post forward: x_next = H_res·x + H_post ⊗ y (single read of x and y, single
 * write of x_next). */
mhc_status mhc_post(const mhc_desc* desc, const void* x, const void* y, const float* H_post,
                    const float* H_res, void* x_next, hipStream_t stream);

/* hc_post backward.  Given dx_next, writes
 *   dx[m]       = Σ_n H_res[n,m]·dx_next[n]        (I/O dtype, overwritten)
 *   dy          = Σ_n H_post[n]·dx_next[n]         (I/O dtype)
 *   dH_post[n]  = <dx_next[n], y>,  dH_res[n,m] = <dx_next[n], x[m]>   (fp32)
 * Must run before mhc_pre_bwd, which adds hc_pre's contribution into dx.
 * dx may be NULL: nothing is written for it, and the caller passes dx_next
 * and H_res to mhc_pre_bwd_mix instead, which forms the same term inside the
 * hc_pre backward (the state gradient then crosses HBM once instead of being
 * written here and read back there). */
mhc_status mhc_post_bwd(const mhc_desc* desc, const void* dx_next, const void* x, const void* y,
                        const float* H_post, const float* H_res, void* dx, void* dy,
                        float* dH_post, float* dH_res, hipStream_t stream);

/* Bytes of device workspace mhc_pre_bwd needs; 0 for an invalid descriptor. */
size_t mhc_pre_bwd_workspace_bytes(const mhc_desc* desc);

/* hc_pre backward with recompute from x.  Inputs: dh[T][D] (gradient of h),
 * x, φ, bias, and dH_post / dH_res from mhc_post_bwd.  Outputs:
 *   dx (in/out, I/O dtype): on entry hc_post's contribution, on exit the total;
 *   dphi[N·D][C], dbias[C] (fp32, overwritten);
 *   dalpha[3] (fp32: d/dα_pre, d/dα_post, d/dα_res) or NULL to skip.
 * `workspace` must hold mhc_pre_bwd_workspace_bytes(desc) bytes, 256-byte
 * aligned; its contents on entry are ignored. */
mhc_status mhc_pre_bwd(const mhc_desc* desc, const void* dh, const void* x, const float* phi,
                       const float* bias, const float* dH_post, const float* dH_res, void* dx,
                       float* dphi, float* dbias, float* dalpha, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* mhc_pre_bwd with hc_post's share of the state gradient formed inside it:
 *   dx = Σ_n H_res[n,m]·dx_next[n] + (the hc_pre part written by mhc_pre_bwd)
 * (I/O dtype, overwritten).  For a block x → hc_pre → f → hc_post → x_next
 * this is the state gradient mhc_post_bwd + mhc_pre_bwd produce together,
 * with mhc_post_bwd called with dx = NULL; the H_res term is rounded to the
 * I/O dtype as mhc_post_bwd rounds its dx, so every output equals that of the
 * two calls bit for bit.
 * dx_next and H_res are the arguments mhc_post_bwd took.  dx may be dx_next
 * itself (the gradient is then formed in place), but must not overlap it
 * otherwise, nor x or dh.  Same workspace as mhc_pre_bwd. */
mhc_status mhc_pre_bwd_mix(const mhc_desc* desc, const void* dh, const void* x, const float* phi,
                           const float* bias, const float* dH_post, const float* dH_res,
                           const void* dx_next, const float* H_res, void* dx, float* dphi, float* dbias,
                           float* dalpha, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char* mhc_status_string(mhc_status status);

/* Bytes of device workspace mhc_post_pre needs (the same as mhc_pre's for
 * the same descriptor). */
size_t mhc_post_pre_workspace_bytes(const mhc_desc* desc);

/* hc_post of one layer followed by hc_pre of the next layer (openPangu 2.0
 * analysis §11.3 fuses the write-back, the next RMSNorm and H_pre).  Computes
 * x_next = H_res_in·x + H_post_in ⊗ y ([T][N][D], I/O dtype; the mhc_post
 * contract) and then, on x_next as stored, hc_pre of the next layer with its
 * phi, bias and the descriptor's Sinkhorn rounds, eps and gate scalars: h,
 * H_pre, H_post, H_res (the mhc_pre contract).  The results equal mhc_post
 * followed by mhc_pre bit for bit (the call runs the two kernels; a single
 * pass that keeps x_next on chip measured slower than the pair).  Outputs must
 * not alias inputs; the workspace rules of mhc_pre apply. */
mhc_status mhc_post_pre(const mhc_desc* desc, const void* x, const void* y, const float* H_post_in,
                        const float* H_res_in, const float* phi, const float* bias, void* x_next,
                        void* h, float* H_pre, float* H_post, float* H_res, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* openPangu's stabilised write-back (openPangu 2.0 analysis, §5.4, first two
 * items), per token:
 *   ŷ      = y_weight ⊙ y · (mean_d y² + eps)^(-1/2)   sandwich norm of the
 *            sublayer output before H_post writes it back (ŷ = y if y_weight
 *            is NULL)
 *   z      = H_res·x + H_post ⊗ ŷ                        (as mhc_post)
 *   x_next = out_weight ⊙ z · (mean z² + eps)^(-1/2)     block post-norm over
 *            the token's flattened N·D state (x_next = z if out_weight is NULL)
 * y_weight[D] and out_weight[N·D] are fp32; eps is desc->eps, the hc_pre norm's.
 * With both weights NULL this is mhc_post.  With a weight, N·⌈D/5120⌉ must be
 * at most 4 (D ≤ 5120 at N = 4, 10240 at N = 2, 20480 at N = 1), else
 * MHC_ERR_UNSUPPORTED.  The rest of the mhc_post contract applies. */
mhc_status mhc_post_stable(const mhc_desc* desc, const void* x, const void* y, const float* y_weight,
                           const float* H_post, const float* H_res, const float* out_weight,
                           void* x_next, hipStream_t stream);

/* Bytes of device workspace mhc_post_stable_bwd needs for the given weights
 * (nonzero flags: that weight is present); 0 for an invalid descriptor or
 * when neither is. */
size_t mhc_post_stable_bwd_workspace_bytes(const mhc_desc* desc, int with_y_weight, int with_out_weight);

/* Backward of mhc_post_stable, recomputing ŷ, z and both norms from x and y.
 * Writes dx (I/O dtype, overwritten: mhc_pre_bwd then adds hc_pre's part), dy
 * (I/O dtype), dH_post, dH_res (fp32), and the weight gradients summed over
 * the tokens: dy_weight[D] (required if and only if y_weight is given) and
 * dout_weight[N·D] (likewise for out_weight), fp32, overwritten.  The
 * workspace holds mhc_post_stable_bwd_workspace_bytes bytes, 256-byte
 * aligned; its contents on entry are ignored.  With both weights NULL this is
 * mhc_post_bwd (no workspace).  Shape limits as for mhc_post_stable. */
mhc_status mhc_post_stable_bwd(const mhc_desc* desc, const void* dx_next, const void* x, const void* y,
                               const float* y_weight, const float* H_post, const float* H_res,
                               const float* out_weight, void* dx, void* dy, float* dy_weight,
                               float* dout_weight, float* dH_post, float* dH_res, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Size of the static scratch buffer behind mhc_pre_noalloc, in bytes: one
 * such buffer per GPU the library runs on, held until the process ends. */
#define MHC_NOALLOC_SCRATCH_BYTES (16u << 20)

/* mhc_pre for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace mhc_pre takes from its caller is the library's static scratch
 * buffer of the current device instead, and the call makes no allocation of
 * any kind.  Arguments, layouts, results (bit for bit) and errors as for
 * mhc_pre; in addition MHC_ERR_TOO_LARGE, with nothing launched, when
 * mhc_pre_workspace_bytes(desc) exceeds MHC_NOALLOC_SCRATCH_BYTES (on a
 * 256-CU MI355X every T up to 9,216 fits for bf16, N = 4, D = 5120, up to
 * 9,248 for fp32 at D = 5120, and up to 19,712 at D = 2560 for either; the
 * other paths need at most 2 MB).  The first call on a
 * device looks up the buffer's device address (MHC_ERR_HIP if that fails).
 * Every call on one GPU shares that GPU's buffer, which keeps the last
 * call's contents (nothing in it needs clearing): calls on one stream are
 * safe, calls that overlap in time on one GPU (two streams, two host threads)
 * race and must not be made. */
mhc_status mhc_pre_noalloc(const mhc_desc* desc, const void* x, const float* phi, const float* bias,
                           void* h, float* H_pre, float* H_post, float* H_res, hipStream_t stream);

/* MHC_ABI_VERSION of the built library. */
int mhc_abi_version(void);

/* Kernel-level timing, for benchmarks and profiling (off by default; not part
 * of the method).  While `events` is non-NULL, every mhc_* call made on the
 * calling host thread records events[2k] on its stream immediately before its
 * k-th kernel launch and events[2k + 1] immediately after it, for k counted
 * from this call up to `capacity` launches (later launches are not recorded);
 * names[k] (if `names` is non-NULL) is set to a static string naming the
 * kernel, and *count (if non-NULL) to the number of launches recorded so far.
 * The events are the caller's (created with hipEventCreate, with timing) and
 * must outlive the tracing; hipEventElapsedTime(events[2k], events[2k + 1])
 * is then the k-th kernel's time on the device.  Calling it again restarts
 * the count; mhc_trace_kernel_events(NULL, NULL, 0, NULL) stops.  The state is
 * per host thread.  MHC_ERR_INVALID_ARG for a negative capacity, or a zero
 * one with events. */
mhc_status mhc_trace_kernel_events(hipEvent_t* events, const char** names, int capacity, int* count);

/* Failure injection for tests of the split-K hc_pre's bounded waits (not part
 * of the method; off by default).  While drop_slice >= 0, workgroup
 * `drop_slice` of every group of the split-K kernel (bf16, N = 4, D = 5120 or
 * 2560, more tokens than the few-token path takes) publishes no exchange
 * records, and every wait for records gives up after `spin_limit` polls.  The
 * other members then write NaN for the tokens of every tile (h, H_pre,
 * H_post, H_res): the failure those waits exist for, with every kernel ending
 * normally.  drop_slice = -1 turns it off (spin_limit is then ignored).
 * Process-wide and not synchronised: set it only while no other host thread
 * launches mhc_pre / mhc_post_pre.  MHC_ERR_INVALID_ARG for drop_slice < -1,
 * or for spin_limit 0 with drop_slice >= 0. */
mhc_status mhc_test_exchange_fault(int drop_slice, unsigned spin_limit);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */
