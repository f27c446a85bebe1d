"""Pins for the oracle's stabilised write-back and weighted norm ([openPangu]
§5.4: sandwich norm of the sublayer output, block post-norm of the state, and
a learnable weight on the hc_pre norm): closed forms, reductions to the
unweighted calls, scale invariance of an RMS norm and the orthogonality of its
gradient, and fp64 central finite differences of every input of the backward."""

import numpy as np
import pytest

from oracle import mhc_oracle as O


def _case(T=4, N=4, D=16, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, N, D))
    y = rng.standard_normal((T, D)) * 3.0
    gamma = rng.uniform(0.5, 1.5, D)
    Hp = rng.uniform(0.0, 2.0, (T, N))
    Hr = rng.uniform(0.0, 1.0, (T, N, N))
    g = rng.standard_normal((T, N, D))
    return x, y, gamma, Hp, Hr, g


def test_constant_vector_closed_form():
    c, eps, D = -2.5, 1e-3, 12
    y = np.full((1, D), c)
    gamma = np.linspace(0.5, 2.0, D)
    y_hat, r = O.sandwich_norm(y, gamma, eps)
    assert np.allclose(y_hat[0], gamma * c / np.sqrt(c * c + eps), rtol=1e-15, atol=0)
    assert np.isclose(r[0], 1.0 / np.sqrt(c * c + eps), rtol=1e-15)


def test_unit_weight_gives_unit_rms_up_to_eps():
    _, y, _, _, _, _ = _case()
    eps = 1e-2
    y_hat, _ = O.sandwich_norm(y, np.ones(y.shape[1]), eps)
    ms = np.mean(y * y, axis=1)
    assert np.allclose(np.mean(y_hat * y_hat, axis=1), ms / (ms + eps), rtol=1e-13)


def test_scale_invariance_and_orthogonal_gradient():
    x, y, gamma, Hp, Hr, g = _case(seed=3)
    a, _ = O.sandwich_norm(y, gamma, eps=0.0)
    b, _ = O.sandwich_norm(7.0 * y, gamma, eps=0.0)
    assert np.allclose(a, b, rtol=1e-13, atol=0)
    # ŷ(s·y) = ŷ(y) for every s > 0, so dL/dy is orthogonal to y, token by token
    _, dy, _, _, _ = O.hc_post_sandwich_bwd(g, x, y, gamma, Hp, Hr, eps=0.0)
    dots = np.sum(dy * y, axis=1)
    assert np.all(np.abs(dots) <= 1e-12 * np.linalg.norm(dy, axis=1) * np.linalg.norm(y, axis=1))


def test_no_write_back_leaves_the_mix():
    x, y, gamma, Hp, Hr, _ = _case(seed=4)
    xn = O.hc_post_sandwich(x, y, gamma, np.zeros_like(Hp), Hr)
    assert np.allclose(xn, np.einsum("tnm,tmd->tnd", Hr, x), rtol=0, atol=0)


def _fd(fun, arr, idx, h=1e-6):
    old = arr[idx]
    arr[idx] = old + h
    lp = fun()
    arr[idx] = old - h
    lm = fun()
    arr[idx] = old
    return (lp - lm) / (2 * h)


@pytest.mark.parametrize("eps", [1e-6, 0.5])
def test_backward_finite_differences(eps):
    x, y, gamma, Hp, Hr, g = _case(seed=5)
    loss = lambda: float(np.sum(g * O.hc_post_sandwich(x, y, gamma, Hp, Hr, eps)))
    dx, dy, dgamma, dHp, dHr = O.hc_post_sandwich_bwd(g, x, y, gamma, Hp, Hr, eps)
    rng = np.random.default_rng(9)
    for arr, grad in ((x, dx), (y, dy), (gamma, dgamma), (Hp, dHp), (Hr, dHr)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            num = _fd(loss, arr, idx)
            assert abs(num - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (arr.shape, idx, num, grad[idx])


# ---- block post-norm and the full stabilised write-back ([openPangu] §5.4) ----

def test_rms_norm_constant_row_closed_form():
    c, eps, F = 3.0, 0.25, 10
    w = np.linspace(-1.0, 1.0, F)
    out, r = O.rms_norm(np.full((1, F), c), w, eps)
    assert np.allclose(out[0], w * c / np.sqrt(c * c + eps), rtol=1e-15, atol=1e-300)
    assert np.isclose(r[0], 1.0 / np.sqrt(c * c + eps), rtol=1e-15)


def test_stable_without_weights_is_hc_post():
    x, y, _, Hp, Hr, g = _case(seed=6)
    assert np.array_equal(O.hc_post_stable(x, y, Hp, Hr), O.hc_post(x, y, Hp, Hr))
    got = O.hc_post_stable_bwd(g, x, y, Hp, Hr)
    ref = O.hc_post_bwd(g, x, y, Hp, Hr)
    for a, b in zip((got["dx"], got["dy"], got["dH_post"], got["dH_res"]), ref):
        assert np.array_equal(a, b)
    assert got["dy_weight"] is None and got["dout_weight"] is None


def test_stable_sandwich_only_is_hc_post_sandwich():
    x, y, gamma, Hp, Hr, g = _case(seed=7)
    assert np.allclose(O.hc_post_stable(x, y, Hp, Hr, y_weight=gamma),
                       O.hc_post_sandwich(x, y, gamma, Hp, Hr), rtol=1e-14, atol=0)
    got = O.hc_post_stable_bwd(g, x, y, Hp, Hr, y_weight=gamma)
    dx, dy, dgamma, dHp, dHr = O.hc_post_sandwich_bwd(g, x, y, gamma, Hp, Hr)
    for a, b in ((got["dx"], dx), (got["dy"], dy), (got["dy_weight"], dgamma),
                 (got["dH_post"], dHp), (got["dH_res"], dHr)):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_post_norm_unit_weight_gives_unit_rms_per_token():
    x, y, gamma, Hp, Hr, _ = _case(seed=8)
    T, N, D = x.shape
    xn = O.hc_post_stable(x, y, Hp, Hr, y_weight=gamma, out_weight=np.ones(N * D), eps=0.0)
    assert np.allclose(np.mean(xn.reshape(T, -1) ** 2, axis=1), 1.0, rtol=1e-13)
    # without the sandwich norm z is linear in (x, y), so scaling both leaves x_next unchanged
    a = O.hc_post_stable(x, y, Hp, Hr, out_weight=np.ones(N * D), eps=0.0)
    b = O.hc_post_stable(5 * x, 5 * y, Hp, Hr, out_weight=np.ones(N * D), eps=0.0)
    assert np.allclose(a, b, rtol=1e-12, atol=0)


@pytest.mark.parametrize("sw,pn", [(False, True), (True, True)])
def test_stable_backward_finite_differences(sw, pn):
    x, y, gamma, Hp, Hr, g = _case(seed=10)
    T, N, D = x.shape
    wy = gamma if sw else None
    wx = np.random.default_rng(11).uniform(0.5, 1.5, N * D) if pn else None
    eps = 1e-3
    loss = lambda: float(np.sum(g * O.hc_post_stable(x, y, Hp, Hr, wy, wx, eps)))
    got = O.hc_post_stable_bwd(g, x, y, Hp, Hr, wy, wx, eps)
    pairs = [(x, got["dx"]), (y, got["dy"]), (Hp, got["dH_post"]), (Hr, got["dH_res"])]
    if sw:
        pairs.append((wy, got["dy_weight"]))
    if pn:
        pairs.append((wx, got["dout_weight"]))
    rng = np.random.default_rng(12)
    for arr, grad in pairs:
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            num = _fd(loss, arr, idx)
            assert abs(num - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (arr.shape, idx, num, grad[idx])


# ---- learnable weight on the hc_pre norm ----

def _pre_case(T=3, N=4, D=8, seed=0):
    rng = np.random.default_rng(seed)
    C = N * N + 2 * N
    x = rng.standard_normal((T, N, D))
    w = rng.uniform(0.5, 1.5, N * D)
    phi = rng.standard_normal((N * D, C)) * 0.5
    bias = rng.standard_normal(C) * 0.1
    return x, w, phi, bias, (0.7, 0.9, 1.1)


def test_weighted_pre_unit_weight_is_hc_pre():
    x, _, phi, bias, al = _pre_case(seed=1)
    T, N, D = x.shape
    a = O.hc_pre_weighted(x, np.ones(N * D), phi, bias, al, 1e-6, 20)
    b = O.hc_pre(x, phi, bias, al, 1e-6, 20)
    for k in ("h", "H_pre", "H_post", "H_res"):
        assert np.allclose(a[k], b[k], rtol=1e-13, atol=1e-15), k


def test_weighted_pre_equals_weight_folded_into_phi():
    # x̄ = w ⊙ x·rstd, so x̄·φ = rstd·x·(diag(w)·φ): the weight folds into φ's rows
    x, w, phi, bias, al = _pre_case(seed=2)
    a = O.hc_pre_weighted(x, w, phi, bias, al, 1e-6, 20)
    b = O.hc_pre(x, w[:, None] * phi, bias, al, 1e-6, 20)
    for k in ("h", "H_pre", "H_post", "H_res"):
        assert np.allclose(a[k], b[k], rtol=1e-12, atol=1e-15), k


def test_weighted_pre_backward_finite_differences():
    x, w, phi, bias, al = _pre_case(seed=3)
    T, N, D = x.shape
    rng = np.random.default_rng(4)
    dh = rng.standard_normal((T, D))
    dHq = rng.standard_normal((T, N))
    dHr = rng.standard_normal((T, N, N))

    def loss():
        r = O.hc_pre_weighted(x, w, phi, bias, al, 1e-3, 6)
        return float(np.sum(dh * r["h"]) + np.sum(dHq * r["H_post"]) + np.sum(dHr * r["H_res"]))

    got = O.hc_pre_weighted_bwd(dh, x, w, phi, bias, dHq, dHr, al, 1e-3, 6)
    for arr, grad in ((x, got["dx"]), (w, got["dnorm_weight"]), (phi, got["dphi"]), (bias, got["dbias"])):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in arr.shape)
            num = _fd(loss, arr, idx)
            assert abs(num - grad[idx]) <= 1e-6 * max(1.0, abs(grad[idx])), (arr.shape, idx, num, grad[idx])
