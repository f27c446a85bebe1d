"""Pins for the oracle's backward: fp64 central finite differences and exact identities.

The loss is L = <dh, h> + <dx_next, x_next> with (h, H_pre, H_post, H_res) =
hc_pre(x, phi, bias) and x_next = hc_post(x, y, H_post, H_res), the chain the
library runs (hc_post's backward feeds dH_post, dH_res into hc_pre's backward,
and the two dx contributions add).  Finite differences use a T = 4, D = 16
slice, as the fp64 checks of the backward ask.
"""

import numpy as np
import pytest

from oracle import mhc_oracle as O
from residual_stream_amd.inputs import make_inputs


def _loss(x, y, phi, bias, alphas, dh, dxn, eps, iters):
    out = O.hc_pre(x, phi, bias, alphas, eps, iters)
    xn = O.hc_post(x, y, out["H_post"], out["H_res"])
    return float(np.sum(dh * out["h"]) + np.sum(dxn * xn))


def _analytic(x, y, phi, bias, alphas, dh, dxn, eps, iters):
    out = O.hc_pre(x, phi, bias, alphas, eps, iters)
    dx_post, dy, dHp, dHr = O.hc_post_bwd(dxn, x, y, out["H_post"], out["H_res"])
    g = O.hc_pre_bwd(dh, x, phi, bias, dHp, dHr, alphas, eps, iters)
    return {"x": dx_post + g["dx"], "y": dy, "phi": g["dphi"], "bias": g["dbias"],
            "alphas": g["dalpha"]}


def _fd(fun, arr, idx_list, h=1e-6):
    out = []
    for idx in idx_list:
        old = arr[idx]
        arr[idx] = old + h
        lp = fun()
        arr[idx] = old - h
        lm = fun()
        arr[idx] = old
        out.append((lp - lm) / (2 * h))
    return np.array(out)


@pytest.mark.parametrize("N,alpha,bias_scale", [(4, 1.0, 1.0), (4, 0.01, None), (2, 0.5, 2.0),
                                                (1, 1.0, 1.0)])
def test_backward_matches_central_differences(N, alpha, bias_scale):
    T, D = 4, 16
    inp = make_inputs(T, N, D, seed=21, alpha=alpha, grads=True)
    x = inp.x.astype(np.float64)
    y = inp.y.astype(np.float64)
    phi = inp.phi.astype(np.float64)
    bias = inp.bias.astype(np.float64)
    if bias_scale is not None:
        bias = np.random.default_rng(22).standard_normal(bias.shape) * bias_scale
    alphas = np.array(inp.alphas, dtype=np.float64)
    dh = inp.dh.astype(np.float64)
    dxn = inp.dx_next.astype(np.float64)
    eps, iters = inp.eps, inp.iters

    def f():
        return _loss(x, y, phi, bias, tuple(alphas), dh, dxn, eps, iters)

    g = _analytic(x, y, phi, bias, tuple(alphas), dh, dxn, eps, iters)
    rng = np.random.default_rng(23)
    for name, arr in (("x", x), ("y", y), ("phi", phi), ("bias", bias), ("alphas", alphas)):
        flat_n = arr.size
        picks = range(flat_n) if flat_n <= 64 else rng.choice(flat_n, 64, replace=False)
        idx = [np.unravel_index(int(i), arr.shape) for i in picks]
        num = _fd(f, arr, idx)
        ana = np.array([g[name][i] for i in idx])
        scale = max(1.0, np.max(np.abs(ana)))
        np.testing.assert_allclose(ana, num, rtol=0, atol=2e-7 * scale, err_msg=name)


def test_res_logit_gradient_rows_sum_to_zero():
    # Adding a constant to a row of the res logits leaves H_res unchanged
    # (row normalisation comes first), so each row of dℓ_res sums to zero.
    inp = make_inputs(8, 4, 32, seed=24, alpha=1.0, grads=True)
    out = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas)
    _, _, dHp, dHr = O.hc_post_bwd(inp.dx_next, inp.x, inp.y, out["H_post"], out["H_res"])
    g = O.hc_pre_bwd(inp.dh, inp.x, inp.phi, inp.bias, dHp, dHr, inp.alphas)
    dres = g["dlogits"][:, 8:].reshape(8, 4, 4)
    np.testing.assert_allclose(dres.sum(-1), 0.0, atol=1e-13)


def test_uniform_upstream_gradient_passes_through_mix():
    # All dx_next[n] = g → dx[m] = Σ_n H_res[n,m]·g = g, because column sums are 1.
    inp = make_inputs(8, 4, 32, seed=25)
    out = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas)
    g = np.random.default_rng(26).standard_normal((8, 1, 32))
    dxn = np.broadcast_to(g, (8, 4, 32))
    dx, _, _, _ = O.hc_post_bwd(dxn, inp.x, inp.y, out["H_post"], out["H_res"])
    np.testing.assert_allclose(dx, np.broadcast_to(g, dx.shape), atol=1e-14)


def test_post_bwd_explicit_loops():
    inp = make_inputs(2, 3, 5, seed=27, grads=True)
    rng = np.random.default_rng(28)
    Hp = rng.uniform(0, 2, (2, 3))
    Hr = rng.uniform(0, 1, (2, 3, 3))
    x, y = inp.x.astype(np.float64), inp.y.astype(np.float64)
    g = rng.standard_normal((2, 3, 5))
    dx, dy, dHp, dHr = O.hc_post_bwd(g, x, y, Hp, Hr)
    for t in range(2):
        for n in range(3):
            assert dHp[t, n] == pytest.approx(sum(g[t, n, d] * y[t, d] for d in range(5)), rel=1e-13)
            for m in range(3):
                assert dHr[t, n, m] == pytest.approx(sum(g[t, n, d] * x[t, m, d] for d in range(5)),
                                                     rel=1e-13)
        for d in range(5):
            assert dy[t, d] == pytest.approx(sum(Hp[t, n] * g[t, n, d] for n in range(3)), rel=1e-13)
            for m in range(3):
                assert dx[t, m, d] == pytest.approx(sum(Hr[t, n, m] * g[t, n, d] for n in range(3)),
                                                    rel=1e-13)
