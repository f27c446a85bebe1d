"""Pins for the oracle's sandwich-normalised write-back ([openPangu] §5.4,
first item): closed forms, the scale invariance of an RMS norm and the
orthogonality of its gradient that follows, and fp64 central finite
differences of every input of the backward."""

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
