"""fp64 CPU oracle for the mHC hot path (hc_pre / hc_post and their backward).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, constants or helpers with the HIP
library and imports nothing from it.

Sources (cited by page title and section; a reader has the pages):

* [openPangu] "openPangu 2.0 — architecture, training and Ascend systems
  analysis" (technical-report notes), §5.3 "mHC": the formula block
  x̄ = RMSNorm(h̄); [r_pre, r_post, r_res] = x̄·W_mHC; H_pre = sigmoid(r_pre);
  H_post = 2·sigmoid(r_post); H_res = Sinkhorn(reshape(r_res, 4, 4)), and the
  sentence giving the roles of the three maps and the 20 Sinkhorn–Knopp rounds.
  The model table (§01, "mHC streams / Sinkhorn" row) fixes N = 4 and 20 rounds.
* [Ascend-mHC] the Ascend training team's article on the mHC Triton operator
  (jinguxun.com), paragraph defining H_res / H_pre / H_post: H_res is
  non-negative with unit row and column sums; H_pre in (0, 1); H_post in
  (0, 2); H_pre collapses N streams to one, H_post expands one to N, H_res
  mixes N to N.  Its recompute paragraph keeps only the hc_pre input and the
  sublayer outputs, so the backward recomputes hc_pre from x.

Readings where the pages are silent (each also listed in the design doc):

1. ℓ = α_g·(x̄·φ) + b with one gate scalar α per group (pre, post, res) and a
   bias b.  With α = 1, b = 0 this is the pages' formula.
2. Logit columns are ordered [pre 0..N-1 | post N..2N-1 | res 2N..2N+N²-1];
   the res block is reshaped row-major to N×N, row = destination stream.
3. hc_post applies H_res from the left: x_next[n] = Σ_m H_res[n,m]·x[m]
   + H_post[n]·y.  The collapse uses raw x: h = Σ_n H_pre[n]·x[n].
4. RMSNorm is over the flattened N·D vector of a token, mean of squares,
   eps inside the square root, unit weight.
5. Sinkhorn starts from exp(ℓ_res); one round = divide every row by its sum,
   then every column by its sum; the result is the matrix after the last
   column step.  The oracle runs the rounds as written (not the limit).
6. The backward is the exact derivative of 1–5 (the pages give no backward).
7. openPangu's stabilised variant ([openPangu] §5.4, first item) normalises
   the sublayer output before H_post writes it back ("sandwich"
   normalisation): ŷ = γ ⊙ y · (mean_d y² + eps)^(-1/2), an RMSNorm over the
   D features of each token with a learnable weight γ[D]; then
   x_next = H_res·x + H_post ⊗ ŷ.  Same eps as the hc_pre norm.
8. The block-level post-norm of the same list (second item: after the first
   layer and every fifth layer) is an RMSNorm of each token's whole N-stream
   state, over the flattened N·D vector like the hc_pre norm, with a learnable
   weight w[N·D]: x_next ← w ⊙ z · (mean_k z² + eps)^(-1/2), z the write-back
   result.  It is applied to the state the write-back produces.
9. A learnable weight w[N·D] on the hc_pre RMSNorm, x̄ = w ⊙ x·rstd, enters
   only the logits (h collapses the raw streams).

Everything is computed in float64 from the exact input values (bf16 inputs
arrive already upcast).  Shapes: x[T,N,D], y[T,D], phi[N·D, N²+2N],
bias[N²+2N]; T tokens, N streams, D hidden.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "n_logits",
    "rms_rstd",
    "project",
    "split_logits",
    "gates",
    "sinkhorn",
    "sinkhorn_trace",
    "sinkhorn_bwd",
    "hc_pre",
    "hc_post",
    "hc_post_bwd",
    "hc_pre_bwd",
    "sandwich_norm",
    "hc_post_sandwich",
    "hc_post_sandwich_bwd",
    "rms_norm",
    "rms_norm_bwd",
    "hc_post_stable",
    "hc_post_stable_bwd",
    "hc_pre_weighted",
    "hc_pre_weighted_bwd",
]


def n_logits(N: int) -> int:
    """Number of projection outputs per token: N pre + N post + N² res logits
    ([openPangu] §5.3: [r_pre, r_post, r_res] with r_res reshaped to N×N)."""
    return N * N + 2 * N


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def rms_rstd(x: np.ndarray, eps: float) -> np.ndarray:
    """Reciprocal RMS of each token's flattened N·D state.

    [openPangu] §5.3, x̄ = RMSNorm(h̄): rstd_t = (mean_k x_{t,k}² + eps)^(-1/2),
    so that x̄_t = rstd_t · x_t (unit weight).  Returns shape [T].
    """
    x = _f64(x)
    T = x.shape[0]
    flat = x.reshape(T, int(np.prod(x.shape[1:])))  # explicit width: T may be 0
    return 1.0 / np.sqrt(np.mean(flat * flat, axis=1) + eps)


def project(x: np.ndarray, phi: np.ndarray, eps: float):
    """x̄·W_mHC of [openPangu] §5.3.

    Returns (rstd[T], raw[T,C], q[T,C]) with raw = x_flat·φ and q = rstd·raw,
    which equals RMSNorm(x)·φ because the unit-weight norm is a per-token scale.
    """
    x = _f64(x)
    T = x.shape[0]
    rstd = rms_rstd(x, eps)
    raw = x.reshape(T, int(np.prod(x.shape[1:]))) @ _f64(phi)
    return rstd, raw, rstd[:, None] * raw


def _alpha_vector(N: int, alphas) -> np.ndarray:
    a_pre, a_post, a_res = (float(a) for a in alphas)
    return np.concatenate([np.full(N, a_pre), np.full(N, a_post), np.full(N * N, a_res)])


def split_logits(q: np.ndarray, bias: np.ndarray, alphas, N: int):
    """ℓ = α_g ⊙ q + b, split into (ℓ_pre[T,N], ℓ_post[T,N], ℓ_res[T,N,N]).

    Column order [pre | post | res] and the row-major N×N reshape follow the
    bracket [r_pre, r_post, r_res] and reshape(r_res, 4, 4) of [openPangu] §5.3.
    """
    logits = _alpha_vector(N, alphas)[None, :] * _f64(q) + _f64(bias)[None, :]
    T = logits.shape[0]
    return logits[:, :N], logits[:, N:2 * N], logits[:, 2 * N:].reshape(T, N, N)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def gates(l_pre: np.ndarray, l_post: np.ndarray):
    """H_pre = sigmoid(r_pre) in (0,1), H_post = 2·sigmoid(r_post) in (0,2)
    ([openPangu] §5.3; ranges from [Ascend-mHC], definition paragraph)."""
    return _sigmoid(_f64(l_pre)), 2.0 * _sigmoid(_f64(l_post))


def sinkhorn_trace(M0: np.ndarray, iters: int):
    """Sinkhorn–Knopp rounds on positive matrices M0[..., N, N].

    One round divides each row by its sum, then each column by its sum
    ([openPangu] §5.3: 20 Sinkhorn–Knopp rounds onto the doubly-stochastic
    set).  Returns the final matrix and the list of every step's input and
    divisor, which the backward walks in reverse:
    trace = [(kind, X_in, sums, Y_out), ...] with kind 'row' or 'col'.
    """
    M = _f64(M0)
    trace = []
    for _ in range(iters):
        r = M.sum(axis=-1, keepdims=True)
        Y = M / r
        trace.append(("row", M, r, Y))
        M = Y
        c = M.sum(axis=-2, keepdims=True)
        Y = M / c
        trace.append(("col", M, c, Y))
        M = Y
    return M, trace


def sinkhorn(M0: np.ndarray, iters: int) -> np.ndarray:
    """Final matrix of :func:`sinkhorn_trace`."""
    return sinkhorn_trace(M0, iters)[0]


def sinkhorn_bwd(trace, dH: np.ndarray) -> np.ndarray:
    """Gradient w.r.t. the Sinkhorn input M0, given dL/dH_res.

    Each step is Y = X / s with s the row (or column) sums of X, so
    dX = (dY − Σ_along(dY ⊙ Y)) / s, summed along the same axis; applied to
    the recorded steps in reverse order.
    """
    g = _f64(dH)
    for kind, _X, s, Y in reversed(trace):
        axis = -1 if kind == "row" else -2
        g = (g - np.sum(g * Y, axis=axis, keepdims=True)) / s
    return g


def hc_pre(x, phi, bias, alphas=(0.01, 0.01, 0.01), eps: float = 1e-6, iters: int = 20):
    """hc_pre: coefficients and the collapsed layer input.

    Steps in the order of [openPangu] §5.3: RMSNorm, projection, the two sigmoid
    gates and Sinkhorn(exp(ℓ_res)); then h = Σ_n H_pre[n]·x[n] on the raw
    streams (H_pre chooses which streams the sublayer reads, §5.3 and
    [Ascend-mHC] definition paragraph).

    Returns dict(h[T,D], H_pre[T,N], H_post[T,N], H_res[T,N,N], rstd, raw, logits).
    """
    x = _f64(x)
    T, N, D = x.shape
    rstd, raw, q = project(x, phi, eps)
    l_pre, l_post, l_res = split_logits(q, bias, alphas, N)
    H_pre, H_post = gates(l_pre, l_post)
    H_res = sinkhorn(np.exp(l_res), iters)
    h = np.einsum("tn,tnd->td", H_pre, x)
    return {
        "h": h,
        "H_pre": H_pre,
        "H_post": H_post,
        "H_res": H_res,
        "rstd": rstd,
        "raw": raw,
        "l_pre": l_pre,
        "l_post": l_post,
        "l_res": l_res,
    }


def hc_post(x, y, H_post, H_res) -> np.ndarray:
    """hc_post: x_next[n] = Σ_m H_res[n,m]·x[m] + H_post[n]·y.

    H_res mixes the N streams on the residual path and H_post writes the
    sublayer output back to the streams ([openPangu] §5.3 roles sentence;
    [Ascend-mHC] definition paragraph).  Returns x_next[T,N,D].
    """
    x = _f64(x)
    return np.einsum("tnm,tmd->tnd", _f64(H_res), x) + _f64(H_post)[:, :, None] * _f64(y)[:, None, :]


def hc_post_bwd(dx_next, x, y, H_post, H_res):
    """Exact derivative of :func:`hc_post`.

    Returns (dx[T,N,D], dy[T,D], dH_post[T,N], dH_res[T,N,N]) with
    dx[m] = Σ_n H_res[n,m]·dx_next[n], dy = Σ_n H_post[n]·dx_next[n],
    dH_res[n,m] = <dx_next[n], x[m]>, dH_post[n] = <dx_next[n], y>.
    """
    g = _f64(dx_next)
    x = _f64(x)
    y = _f64(y)
    dx = np.einsum("tnm,tnd->tmd", _f64(H_res), g)
    dy = np.einsum("tn,tnd->td", _f64(H_post), g)
    dH_post = np.einsum("tnd,td->tn", g, y)
    dH_res = np.einsum("tnd,tmd->tnm", g, x)
    return dx, dy, dH_post, dH_res


def hc_pre_bwd(dh, x, phi, bias, dH_post, dH_res, alphas=(0.01, 0.01, 0.01),
               eps: float = 1e-6, iters: int = 20):
    """Exact derivative of :func:`hc_pre`, recomputing the forward from x.

    The recompute follows the intra-layer recompute paragraph of
    [Ascend-mHC]: only x (the hc_pre input) is kept; norm, logits and the
    Sinkhorn rounds are rebuilt here.  Inputs dH_post and dH_res are the
    gradients reaching the coefficients from hc_post.

    Returns dict(dx[T,N,D] (hc_pre's contribution only), dphi[K,C],
    dbias[C], dalpha[3], dlogits[T,C]).
    """
    x = _f64(x)
    T, N, D = x.shape
    K = N * D
    phi = _f64(phi)
    a_vec = _alpha_vector(N, alphas)

    rstd, raw, q = project(x, phi, eps)
    l_pre, l_post, l_res = split_logits(q, bias, alphas, N)
    H_pre, H_post = gates(l_pre, l_post)
    M0 = np.exp(l_res)
    _, trace = sinkhorn_trace(M0, iters)

    dh = _f64(dh)
    # h = Σ_n H_pre[n] x[n]
    dH_pre = np.einsum("td,tnd->tn", dh, x)
    dx = H_pre[:, :, None] * dh[:, None, :]

    s_pre = H_pre
    s_post = H_post / 2.0
    dl_pre = dH_pre * s_pre * (1.0 - s_pre)
    dl_post = _f64(dH_post) * 2.0 * s_post * (1.0 - s_post)
    dl_res = sinkhorn_bwd(trace, dH_res) * M0           # d exp(ℓ) = exp(ℓ) dℓ

    dlogits = np.concatenate([dl_pre, dl_post, dl_res.reshape(T, N * N)], axis=1)
    dq = dlogits * a_vec[None, :]
    dbias = dlogits.sum(axis=0)
    groups = [slice(0, N), slice(N, 2 * N), slice(2 * N, 2 * N + N * N)]
    dalpha = np.array([np.sum(dlogits[:, g] * q[:, g]) for g in groups])

    # q = rstd·raw, raw = x_flat·φ, rstd = (Σ x²/K + eps)^(-1/2)
    xf = x.reshape(T, K)
    draw = rstd[:, None] * dq                            # dL/draw
    drstd = np.sum(dq * raw, axis=1)                     # dL/drstd
    dx_flat = draw @ phi.T - (drstd * rstd ** 3 / K)[:, None] * xf
    dx = dx + dx_flat.reshape(T, N, D)
    dphi = xf.T @ draw
    return {"dx": dx, "dphi": dphi, "dbias": dbias, "dalpha": dalpha, "dlogits": dlogits}


def sandwich_norm(y, gamma, eps: float = 1e-6):
    """ŷ = γ ⊙ y · r, r = (mean_d y² + eps)^(-1/2) per token ([openPangu] §5.4,
    sandwich normalisation of the sublayer output; reading 7).  Returns
    (ŷ[T,D], r[T])."""
    y = _f64(y)
    r = 1.0 / np.sqrt(np.mean(y * y, axis=1) + eps)
    return _f64(gamma)[None, :] * y * r[:, None], r


def hc_post_sandwich(x, y, gamma, H_post, H_res, eps: float = 1e-6) -> np.ndarray:
    """hc_post with the sublayer output normalised before the write-back:
    x_next = H_res·x + H_post ⊗ sandwich_norm(y)."""
    y_hat, _ = sandwich_norm(y, gamma, eps)
    return hc_post(x, y_hat, H_post, H_res)


def hc_post_sandwich_bwd(dx_next, x, y, gamma, H_post, H_res, eps: float = 1e-6):
    """Exact derivative of :func:`hc_post_sandwich`.

    With g = dL/dŷ = Σ_n H_post[n]·dx_next[n] and D features:
    dγ = Σ_t g ⊙ y·r, dy = r·(γ ⊙ g) − (r³/D)·y·Σ_d(γ ⊙ g ⊙ y);
    dx, dH_res as in :func:`hc_post_bwd`, dH_post[n] = <dx_next[n], ŷ>.
    Returns (dx, dy, dgamma[D], dH_post, dH_res).
    """
    y = _f64(y)
    gamma = _f64(gamma)
    T, D = y.shape
    y_hat, r = sandwich_norm(y, gamma, eps)
    dx, g, dH_post, dH_res = hc_post_bwd(dx_next, x, y_hat, H_post, H_res)
    dgamma = np.sum(g * y * r[:, None], axis=0)
    gg = gamma[None, :] * g
    s = np.sum(gg * y, axis=1)
    dy = r[:, None] * gg - (r ** 3 / D)[:, None] * y * s[:, None]
    return dx, dy, dgamma, dH_post, dH_res


def rms_norm(v, weight, eps: float = 1e-6):
    """Row-wise RMSNorm with a learnable weight: out = w ⊙ v · r,
    r = (mean over the row of v² + eps)^(-1/2).  v[T,F], weight[F].  Returns
    (out[T,F], r[T]).  Readings 7 and 8 use it over D (sublayer output) and
    over N·D (the whole state)."""
    v = _f64(v)
    r = 1.0 / np.sqrt(np.mean(v * v, axis=1) + eps)
    return _f64(weight)[None, :] * v * r[:, None], r


def rms_norm_bwd(dout, v, weight, eps: float = 1e-6):
    """Exact derivative of :func:`rms_norm`: with u = w ⊙ dout and F features,
    dv = r·u − (r³/F)·v·Σ(u ⊙ v) and dw = Σ_t dout ⊙ v·r.  Returns (dv, dw)."""
    v = _f64(v)
    dout = _f64(dout)
    F = v.shape[1]
    _, r = rms_norm(v, weight, eps)
    u = _f64(weight)[None, :] * dout
    s = np.sum(u * v, axis=1)
    dv = r[:, None] * u - (r ** 3 / F)[:, None] * v * s[:, None]
    dw = np.sum(dout * v * r[:, None], axis=0)
    return dv, dw


def hc_post_stable(x, y, H_post, H_res, y_weight=None, out_weight=None, eps: float = 1e-6):
    """The stabilised write-back of [openPangu] §5.4 (readings 7 and 8):
    ŷ = rms_norm(y, y_weight) (sandwich norm; ŷ = y when y_weight is None),
    z = H_res·x + H_post ⊗ ŷ, x_next = rms_norm(z over N·D, out_weight) (block
    post-norm; x_next = z when out_weight is None).  Returns x_next[T,N,D]."""
    x = _f64(x)
    T, N, D = x.shape
    y_hat = _f64(y) if y_weight is None else rms_norm(y, y_weight, eps)[0]
    z = hc_post(x, y_hat, H_post, H_res)
    if out_weight is None:
        return z
    return rms_norm(z.reshape(T, N * D), out_weight, eps)[0].reshape(T, N, D)


def hc_post_stable_bwd(dx_next, x, y, H_post, H_res, y_weight=None, out_weight=None,
                       eps: float = 1e-6):
    """Exact derivative of :func:`hc_post_stable`, by the chain rule through
    its three steps.  Returns dict(dx, dy, dH_post, dH_res, dy_weight,
    dout_weight); a weight's gradient is None when the weight is None."""
    x = _f64(x)
    T, N, D = x.shape
    y = _f64(y)
    y_hat = y if y_weight is None else rms_norm(y, y_weight, eps)[0]
    g = _f64(dx_next)
    dout_weight = None
    if out_weight is not None:
        z = hc_post(x, y_hat, H_post, H_res)
        dz, dout_weight = rms_norm_bwd(g.reshape(T, N * D), z.reshape(T, N * D), out_weight, eps)
        g = dz.reshape(T, N, D)
    dx, dy_hat, dH_post, dH_res = hc_post_bwd(g, x, y_hat, H_post, H_res)
    dy_weight = None
    dy = dy_hat
    if y_weight is not None:
        dy, dy_weight = rms_norm_bwd(dy_hat, y, y_weight, eps)
    return {"dx": dx, "dy": dy, "dH_post": dH_post, "dH_res": dH_res,
            "dy_weight": dy_weight, "dout_weight": dout_weight}


def hc_pre_weighted(x, norm_weight, phi, bias, alphas=(0.01, 0.01, 0.01), eps: float = 1e-6,
                    iters: int = 20):
    """hc_pre with a learnable weight on its RMSNorm (reading 9):
    x̄ = w ⊙ x·rstd over the flattened N·D state, ℓ = α_g·(x̄·φ) + b, then the
    gates, Sinkhorn and the collapse h = Σ_n H_pre[n]·x[n] of raw x as in
    :func:`hc_pre`.  Returns the same dict as :func:`hc_pre`."""
    x = _f64(x)
    T, N, D = x.shape
    xbar, rstd = rms_norm(x.reshape(T, N * D), norm_weight, eps)
    q = xbar @ _f64(phi)
    l_pre, l_post, l_res = split_logits(q, bias, alphas, N)
    H_pre, H_post = gates(l_pre, l_post)
    H_res = sinkhorn(np.exp(l_res), iters)
    h = np.einsum("tn,tnd->td", H_pre, x)
    return {"h": h, "H_pre": H_pre, "H_post": H_post, "H_res": H_res, "rstd": rstd,
            "l_pre": l_pre, "l_post": l_post, "l_res": l_res}


def hc_pre_weighted_bwd(dh, x, norm_weight, phi, bias, dH_post, dH_res,
                        alphas=(0.01, 0.01, 0.01), eps: float = 1e-6, iters: int = 20):
    """Exact derivative of :func:`hc_pre_weighted`, recomputing from x.
    Returns dict(dx (hc_pre's part), dphi, dbias, dalpha, dnorm_weight)."""
    x = _f64(x)
    T, N, D = x.shape
    K = N * D
    phi = _f64(phi)
    xf = x.reshape(T, K)
    xbar, _ = rms_norm(xf, norm_weight, eps)
    q = xbar @ phi
    l_pre, l_post, l_res = split_logits(q, bias, alphas, N)
    H_pre, H_post = gates(l_pre, l_post)
    M0 = np.exp(l_res)
    _, trace = sinkhorn_trace(M0, iters)

    dh = _f64(dh)
    dH_pre = np.einsum("td,tnd->tn", dh, x)
    dx = H_pre[:, :, None] * dh[:, None, :]
    s_post = H_post / 2.0
    dl_pre = dH_pre * H_pre * (1.0 - H_pre)
    dl_post = _f64(dH_post) * 2.0 * s_post * (1.0 - s_post)
    dl_res = sinkhorn_bwd(trace, dH_res) * M0
    dlogits = np.concatenate([dl_pre, dl_post, dl_res.reshape(T, N * N)], axis=1)
    dq = dlogits * _alpha_vector(N, alphas)[None, :]
    groups = [slice(0, N), slice(N, 2 * N), slice(2 * N, 2 * N + N * N)]
    dalpha = np.array([np.sum(dlogits[:, g] * q[:, g]) for g in groups])
    dphi = xbar.T @ dq
    dxf, dw = rms_norm_bwd(dq @ phi.T, xf, norm_weight, eps)
    return {"dx": dx + dxf.reshape(T, N, D), "dphi": dphi, "dbias": dlogits.sum(axis=0),
            "dalpha": dalpha, "dnorm_weight": dw}
