"""Pins for the fp64 oracle's forward: closed forms, invariants, special cases.

Each test checks the oracle against something other than itself — a value the
mathematics fixes, a library routine, a hand-unrolled scalar computation, or a
property the pages state (openPangu 2.0 analysis §5.3; Ascend mHC Triton article,
definition paragraph).  Together they are chosen so that a dropped term, a
wrong sign, index or reshape, or a transposed operand fails at least one.
"""

import math

import numpy as np
import pytest

from oracle import mhc_oracle as O
from residual_stream_amd.inputs import make_inputs


def _cfg_logits(T=64, N=4, D=256, seed=0, alpha=0.01):
    inp = make_inputs(T, N, D, seed=seed, alpha=alpha)
    _, _, q = O.project(inp.x, inp.phi, inp.eps)
    return inp, O.split_logits(q, inp.bias, inp.alphas, N)


# ---------------------------------------------------------------- RMSNorm ---

@pytest.mark.parametrize("c", [1.0, -3.5, 1e-4, 0.0])
def test_rstd_constant_vector_closed_form(c):
    # x = c·1 → mean(x²) = c², rstd = 1/sqrt(c² + eps).  c = 1e-4 makes eps dominate.
    eps = 1e-6
    x = np.full((1, 4, 8), c)
    assert O.rms_rstd(x, eps)[0] == pytest.approx(1.0 / math.sqrt(c * c + eps), rel=1e-14)


def test_rstd_matches_library_norm():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 4, 32)) * rng.uniform(0.1, 10, size=(5, 1, 1))
    K = 4 * 32
    ref = 1.0 / np.sqrt(np.linalg.norm(x.reshape(5, K), axis=1) ** 2 / K + 1e-6)
    np.testing.assert_allclose(O.rms_rstd(x, 1e-6), ref, rtol=1e-13)


def test_projection_against_fsum():
    inp = make_inputs(6, 4, 16, seed=1)
    rstd, raw, q = O.project(inp.x, inp.phi, inp.eps)
    xf = inp.x.astype(np.float64).reshape(6, -1)
    phi = inp.phi.astype(np.float64)
    for t in (0, 3, 5):
        ss = math.fsum(v * v for v in xf[t])
        r = 1.0 / math.sqrt(ss / xf.shape[1] + inp.eps)
        assert rstd[t] == pytest.approx(r, rel=1e-14)
        for c in (0, 7, 23):
            p = math.fsum(xf[t, k] * phi[k, c] for k in range(xf.shape[1]))
            assert raw[t, c] == pytest.approx(p, rel=1e-12, abs=1e-14)
            assert q[t, c] == pytest.approx(r * p, rel=1e-12, abs=1e-14)


# ------------------------------------------------------------------ gates ---

def test_gates_at_zero_logit():
    H_pre, H_post = O.gates(np.zeros((1, 4)), np.zeros((1, 4)))
    assert np.all(H_pre == 0.5)
    assert np.all(H_post == 1.0)


def test_gate_ranges_on_workload_and_extremes():
    _, (lp, lq, _) = _cfg_logits(alpha=1.0)
    H_pre, H_post = O.gates(lp, lq)
    assert np.all((H_pre > 0) & (H_pre < 1))
    assert np.all((H_post > 0) & (H_post < 2))
    a, b = O.gates(np.array([[-30.0, 30.0]]), np.array([[-30.0, 30.0]]))
    assert 0 < a[0, 0] < 1e-12 and 1 - 1e-12 < a[0, 1] <= 1
    assert 0 < b[0, 0] < 1e-12 and 2 - 1e-12 < b[0, 1] <= 2


def test_logit_column_order_pre_post_res():
    # Bias alone drives the logits (phi = 0): +10 on the pre block, -10 on the
    # post block, a single large res logit at (row 0, col 1) of the row-major
    # reshape.  A swapped block order or a column-major reshape fails here.
    N = 4
    C = O.n_logits(N)
    bias = np.zeros(C)
    bias[:N] = 10.0
    bias[N:2 * N] = -10.0
    bias[2 * N + 0 * N + 1] = 10.0
    x = np.ones((1, N, 8))
    out = O.hc_pre(x, np.zeros((N * 8, C)), bias, alphas=(1, 1, 1), iters=50)
    assert np.all(out["H_pre"] > 0.9999)
    assert np.all(out["H_post"] < 1e-3)
    H = out["H_res"][0]
    # the large entry stays at (0, 1); the other rows share columns 0, 2, 3
    assert H[0, 1] > 0.95
    assert abs(H[1, 0] - 1.0 / 3.0) < 0.02
    np.testing.assert_allclose(H[1:, [0, 2, 3]], 1.0 / 3.0, atol=0.02)


# --------------------------------------------------------------- Sinkhorn ---

def _sinkhorn_2x2_unrolled(a, b, c, d, iters):
    """Scalar hand-unrolled Sinkhorn on [[a, b], [c, d]]: rows, then columns."""
    for _ in range(iters):
        r0 = a + b
        r1 = c + d
        a, b = a / r0, b / r0
        c, d = c / r1, d / r1
        c0 = a + c
        c1 = b + d
        a, c = a / c0, c / c0
        b, d = b / c1, d / c1
    return a, b, c, d


@pytest.mark.parametrize("iters", [1, 2, 20])
def test_sinkhorn_n2_hand_unrolled(iters):
    rng = np.random.default_rng(7)
    L = rng.standard_normal((16, 2, 2)) * 1.5
    M0 = np.exp(L)
    H = O.sinkhorn(M0, iters)
    for t in range(16):
        ref = _sinkhorn_2x2_unrolled(*M0[t].ravel(), iters)
        np.testing.assert_allclose(H[t].ravel(), ref, rtol=1e-14, atol=0)


def test_sinkhorn_n2_converged_closed_form():
    # The doubly-stochastic scaling of a positive 2x2 [[a,b],[c,d]] is
    # [[p,1-p],[1-p,p]] with p/(1-p) = sqrt(ad/bc) (cross ratio is preserved).
    rng = np.random.default_rng(8)
    M0 = np.exp(rng.standard_normal((8, 2, 2)) * 0.3)
    H = O.sinkhorn(M0, 20)
    a, b, c, d = (M0[:, i, j] for i, j in ((0, 0), (0, 1), (1, 0), (1, 1)))
    p = np.sqrt(a * d) / (np.sqrt(a * d) + np.sqrt(b * c))
    np.testing.assert_allclose(H[:, 0, 0], p, atol=1e-12)
    np.testing.assert_allclose(H[:, 0, 1], 1 - p, atol=1e-12)


def test_sinkhorn_n1_is_one():
    H = O.sinkhorn(np.exp(np.array([[[3.7]], [[-2.0]]])), 20)
    assert np.all(H == 1.0)


def test_sinkhorn_separable_gives_uniform_after_one_round():
    rng = np.random.default_rng(9)
    a = rng.standard_normal((3, 4, 1))
    b = rng.standard_normal((3, 1, 4))
    H = O.sinkhorn(np.exp(a + b), 1)
    np.testing.assert_allclose(H, 0.25, atol=1e-15)


def test_sinkhorn_row_offset_invariance():
    rng = np.random.default_rng(10)
    L = rng.standard_normal((5, 4, 4))
    off = rng.standard_normal((5, 4, 1)) * 3
    np.testing.assert_allclose(O.sinkhorn(np.exp(L + off), 20), O.sinkhorn(np.exp(L), 20),
                               rtol=0, atol=1e-15)


def test_sinkhorn_permutation_equivariance():
    rng = np.random.default_rng(11)
    L = rng.standard_normal((4, 4))
    P = np.eye(4)[[2, 0, 3, 1]]
    H = O.sinkhorn(np.exp(L)[None], 20)[0]
    HP = O.sinkhorn(np.exp(P @ L @ P.T)[None], 20)[0]
    np.testing.assert_allclose(HP, P @ H @ P.T, atol=1e-15)


def test_sinkhorn_doubly_stochastic_at_workload_logits():
    # The pages' constraint: non-negative entries, row and column sums 1.
    for alpha in (0.01,):
        _, (_, _, l_res) = _cfg_logits(alpha=alpha)
        H = O.sinkhorn(np.exp(l_res), 20)
        assert np.all(H >= 0)
        np.testing.assert_allclose(H.sum(-1), 1.0, atol=1e-6)
        np.testing.assert_allclose(H.sum(-2), 1.0, atol=1e-6)
        # norm preserving: spectral norm of a doubly-stochastic matrix is 1
        np.testing.assert_allclose(np.linalg.norm(H, ord=2, axis=(-2, -1)), 1.0, atol=1e-6)


def test_sinkhorn_last_step_is_a_column_step():
    # Large logits and a single round: the column sums are exact, the row sums
    # are not.  A column-first round would give the opposite.
    rng = np.random.default_rng(12)
    H = O.sinkhorn(np.exp(rng.standard_normal((16, 4, 4)) * 3), 1)
    np.testing.assert_allclose(H.sum(-2), 1.0, atol=1e-14)
    assert np.max(np.abs(H.sum(-1) - 1)) > 1e-2


# ------------------------------------------------------ collapse and mix ---

def test_post_identity_and_zero_gate_returns_x():
    inp = make_inputs(8, 4, 32, seed=2)
    H_res = np.broadcast_to(np.eye(4), (8, 4, 4))
    xn = O.hc_post(inp.x, inp.y, np.zeros((8, 4)), H_res)
    assert np.array_equal(xn, inp.x.astype(np.float64))


def test_post_permutation_permutes_streams():
    inp = make_inputs(8, 4, 32, seed=2)
    perm = [3, 0, 1, 2]
    P = np.eye(4)[perm]
    xn = O.hc_post(inp.x, inp.y, np.zeros((8, 4)), np.broadcast_to(P, (8, 4, 4)))
    assert np.array_equal(xn, inp.x.astype(np.float64)[:, perm, :])


def test_post_writes_y_through_h_post():
    inp = make_inputs(4, 2, 16, seed=5)
    Hp = np.array([[0.5, 1.5]] * 4)
    xn = O.hc_post(inp.x, inp.y, Hp, np.broadcast_to(np.eye(2), (4, 2, 2)))
    x = inp.x.astype(np.float64)
    y = inp.y.astype(np.float64)
    np.testing.assert_array_equal(xn[:, 0], x[:, 0] + 0.5 * y)
    np.testing.assert_array_equal(xn[:, 1], x[:, 1] + 1.5 * y)


def test_n1_closed_form():
    # N = 1: H_res = [[1]], h = sigmoid(l_pre)·x, x_next = x + 2·sigmoid(l_post)·y,
    # with l = alpha·rstd·(x·phi) + b computed by hand.
    rng = np.random.default_rng(4)
    T, D = 3, 8
    x = rng.standard_normal((T, 1, D)) * 2.0
    y = rng.standard_normal((T, D))
    phi = rng.standard_normal((D, 3))
    b = rng.standard_normal(3)
    al = (0.7, -1.3, 2.0)
    out = O.hc_pre(x, phi, b, alphas=al, eps=1e-6, iters=20)
    for t in range(T):
        xt = x[t, 0]
        r = 1.0 / math.sqrt(sum(v * v for v in xt) / D + 1e-6)
        lp = al[0] * r * float(xt @ phi[:, 0]) + b[0]
        lq = al[1] * r * float(xt @ phi[:, 1]) + b[1]
        sp = 1.0 / (1.0 + math.exp(-lp))
        sq = 1.0 / (1.0 + math.exp(-lq))
        np.testing.assert_allclose(out["h"][t], sp * xt, rtol=1e-13)
        assert out["H_res"][t, 0, 0] == 1.0
        xn = O.hc_post(x[t:t + 1], y[t:t + 1], out["H_post"][t:t + 1], out["H_res"][t:t + 1])
        np.testing.assert_allclose(xn[0, 0], xt + 2 * sq * y[t], rtol=1e-13)


def test_collapse_uses_raw_streams():
    # One-hot H_pre (via bias) must return the raw stream, not its normalised copy.
    N, D = 4, 8
    C = O.n_logits(N)
    b = np.zeros(C)
    b[:N] = [-40, 40, -40, -40]
    x = np.random.default_rng(6).standard_normal((2, N, D)) * 5
    out = O.hc_pre(x, np.zeros((N * D, C)), b, alphas=(1, 1, 1))
    np.testing.assert_allclose(out["h"], x[:, 1, :], rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("iters,scale", [(20, None), (1, 3.0)])
def test_stream_sum_conservation(iters, scale):
    # Column sums of H_res are 1 after the final column step, so
    # Σ_n x_next[n] = Σ_m x[m] + (Σ_n H_post[n])·y.  With a single round and
    # large logits the row sums are far from 1: a transposed mix fails here.
    inp = make_inputs(16, 4, 64, seed=3)
    bias = inp.bias.astype(np.float64)
    if scale is not None:
        bias = np.random.default_rng(13).standard_normal(bias.shape) * scale
    out = O.hc_pre(inp.x, inp.phi, bias, inp.alphas, inp.eps, iters)
    xn = O.hc_post(inp.x, inp.y, out["H_post"], out["H_res"])
    lhs = xn.sum(axis=1)
    rhs = inp.x.astype(np.float64).sum(axis=1) + out["H_post"].sum(axis=1)[:, None] * inp.y
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)


def test_mix_is_non_expanding():
    inp, (_, _, l_res) = _cfg_logits()
    H = O.sinkhorn(np.exp(l_res), 20)
    mixed = np.einsum("tnm,tmd->tnd", H, inp.x.astype(np.float64))
    lhs = np.linalg.norm(mixed.reshape(inp.T, -1), axis=1)
    rhs = np.linalg.norm(inp.x.astype(np.float64).reshape(inp.T, -1), axis=1)
    assert np.all(lhs <= rhs * (1 + 1e-6))


def test_hc_pre_h_matches_explicit_loop():
    inp = make_inputs(3, 4, 8, seed=14)
    out = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas)
    x = inp.x.astype(np.float64)
    for t in range(3):
        for d in range(8):
            ref = math.fsum(out["H_pre"][t, n] * x[t, n, d] for n in range(4))
            assert out["h"][t, d] == pytest.approx(ref, rel=1e-14, abs=1e-15)


@pytest.mark.parametrize("iters", [1, 3])
def test_large_logit_inputs_separate_round_counts(iters):
    # The GPU tests of the Sinkhorn round count use bias std 3 at alpha = 1:
    # there one or three rounds differ from twenty, and from the same number of
    # column-first rounds, by far more than the bf16 gate (2e-2), so a wrong
    # count or order fails them.
    inp = make_inputs(64, 4, 256, io="bf16", seed=11, alpha=1.0, iters=iters, bias_std=3.0)
    _, _, q = O.project(inp.x, inp.phi, inp.eps)
    _, _, l_res = O.split_logits(q, inp.bias, inp.alphas, 4)
    M0 = np.exp(l_res)
    few = O.sinkhorn(M0, iters)
    ref = O.sinkhorn(M0, 20)
    col_first = np.swapaxes(O.sinkhorn(np.swapaxes(M0, -1, -2), iters), -1, -2)
    assert np.max(np.abs(few - ref)) / np.max(np.abs(ref)) > 0.1
    assert np.max(np.abs(few - col_first)) / np.max(np.abs(few)) > 0.1
    np.testing.assert_array_equal(few, O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas, inp.eps, iters)["H_res"])


def test_empty_batch():
    # no tokens: every token output is empty and the parameter gradients,
    # sums over the tokens, are exactly zero
    inp = make_inputs(0, 4, 64, io="f32", seed=0, grads=True)
    pre = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
    assert pre["h"].shape == (0, 64) and pre["H_pre"].shape == (0, 4) and pre["H_res"].shape == (0, 4, 4)
    assert O.hc_post(inp.x, inp.y, pre["H_post"], pre["H_res"]).shape == (0, 4, 64)
    dx, dy, dHp, dHr = O.hc_post_bwd(inp.dx_next, inp.x, inp.y, pre["H_post"], pre["H_res"])
    assert dx.shape == (0, 4, 64) and dy.shape == (0, 64)
    g = O.hc_pre_bwd(inp.dh, inp.x, inp.phi, inp.bias, dHp, dHr, inp.alphas, inp.eps, inp.iters)
    assert g["dx"].shape == (0, 4, 64)
    for k in ("dphi", "dbias", "dalpha"):
        assert np.all(g[k] == 0.0), k
    assert g["dphi"].shape == inp.phi.shape and g["dbias"].shape == inp.bias.shape
