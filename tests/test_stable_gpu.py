"""mhc_post_stable / mhc_post_stable_bwd (openPangu's stabilised write-back:
sandwich norm of the sublayer output, block post-norm of the state) through
the C ABI against the fp64 oracle, on seeded inputs only: the activations of
``make_inputs``, the coefficients of ``make_coefficients`` and the weights of
``make_norm_weights``.  Shapes cover one to four chunks per thread, ragged
rows (D not a multiple of the 512 elements a wave covers), the smallest D,
workgroups that walk several tokens, and the full 4096-token Pro shape."""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

from oracle import mhc_oracle as O
from residual_stream_amd import mhc
from residual_stream_amd.inputs import make_coefficients, make_inputs, make_norm_weights

from mhc_testlib import TOL, assert_close, dev, host

pytestmark = pytest.mark.gpu

FLAGS = [(True, False), (False, True), (True, True)]
FLAG_IDS = ["sandwich", "postnorm", "both"]

# (io, N, D, T): one chunk per thread at N = 4 (D ≤ 5120), two at N = 2,
# four at N = 1; D = 40 and 5000 leave lanes idle; D = 8 is the smallest row
# bf16 N = 4 with D a multiple of 640 (5120, 2560) takes the backward with
# ten elements a thread when the post-norm is on; 4864 takes the general one
SHAPES = [("bf16", 4, 5120, 37), ("bf16", 4, 2560, 130), ("bf16", 4, 4864, 21), ("f32", 4, 5120, 33),
          ("f32", 4, 40, 9), ("bf16", 2, 10240, 7), ("f32", 1, 20480, 5), ("f32", 2, 5000, 11), ("bf16", 1, 8, 3)]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _case(io, N, D, T, seed):
    inp = make_inputs(T, N, D, io=io, seed=seed, grads=True)
    Hq, Hr = make_coefficients(T, N, seed=seed + 1)
    wy, wx = make_norm_weights(N, D, seed=seed + 2)
    return inp, Hq, Hr, wy, wx


def _gpu(inp, Hq, Hr, wy, wx, sw, pn, bwd=True):
    io = inp.io
    x, y = dev(inp.x, io), dev(inp.y, io)
    Hq_d, Hr_d = dev(Hq), dev(Hr)
    kw = dict(y_weight=dev(wy) if sw else None, out_weight=dev(wx) if pn else None, eps=inp.eps)
    xn = mhc.mhc_post_stable(x, y, Hq_d, Hr_d, **kw)
    grads = None
    if bwd:
        grads = mhc.mhc_post_stable_bwd(dev(inp.dx_next, io), x, y, Hq_d, Hr_d, **kw)
    torch.cuda.synchronize()
    return xn, grads


def _oracle_fwd(inp, Hq, Hr, wy, wx, sw, pn, sel=slice(None)):
    return O.hc_post_stable(inp.x[sel], inp.y[sel], Hq[sel], Hr[sel], wy if sw else None,
                            wx if pn else None, inp.eps)


def _oracle_bwd(inp, Hq, Hr, wy, wx, sw, pn, sel=slice(None)):
    return O.hc_post_stable_bwd(inp.dx_next[sel], inp.x[sel], inp.y[sel], Hq[sel], Hr[sel],
                                wy if sw else None, wx if pn else None, inp.eps)


def _check_grads(grads, ref, tol, sw, pn):
    dx, dy, dHq, dHr, dwy, dwx = grads
    assert_close("dx", host(dx), ref["dx"], tol)
    assert_close("dy", host(dy), ref["dy"], tol)
    assert_close("dH_post", host(dHq), ref["dH_post"], tol)
    assert_close("dH_res", host(dHr), ref["dH_res"], tol)
    if sw:
        assert_close("dy_weight", host(dwy), ref["dy_weight"], tol)
    else:
        assert dwy is None
    if pn:
        assert_close("dout_weight", host(dwx), ref["dout_weight"], tol)
    else:
        assert dwx is None


@pytest.mark.parametrize("sw,pn", FLAGS, ids=FLAG_IDS)
@pytest.mark.parametrize("io,N,D,T", SHAPES)
def test_forward_and_backward_match_oracle(io, N, D, T, sw, pn):
    _say(f"[stable] {io} N={N} D={D} T={T} sandwich={sw} postnorm={pn}")
    inp, Hq, Hr, wy, wx = _case(io, N, D, T, seed=N * 1000 + T)
    xn, grads = _gpu(inp, Hq, Hr, wy, wx, sw, pn)
    tol = TOL[io]
    assert_close("x_next", host(xn), _oracle_fwd(inp, Hq, Hr, wy, wx, sw, pn), tol)
    _check_grads(grads, _oracle_bwd(inp, Hq, Hr, wy, wx, sw, pn), tol, sw, pn)


@pytest.mark.parametrize("D,T", [(5120, 300), (5120, 1500), (2560, 1100)])
@pytest.mark.parametrize("sw,pn", FLAGS, ids=FLAG_IDS)
def test_workgroups_walk_several_tokens(sw, pn, D, T):
    # more tokens than the backward grid holds workgroups (one per compute
    # unit at D = 5120 with the post-norm, two of 256 threads at D = 2560), so
    # each one sums several tokens into its weight rows; ragged, so that some
    # take one token more (300: one or two tokens, so the prefetch of a token
    # two ahead runs out early)
    _say(f"[stable] bf16 N=4 D={D} T={T} sandwich={sw} postnorm={pn}")
    inp, Hq, Hr, wy, wx = _case("bf16", 4, D, T, seed=77)
    xn, grads = _gpu(inp, Hq, Hr, wy, wx, sw, pn)
    tol = TOL["bf16"]
    assert_close("x_next", host(xn), _oracle_fwd(inp, Hq, Hr, wy, wx, sw, pn), tol)
    _check_grads(grads, _oracle_bwd(inp, Hq, Hr, wy, wx, sw, pn), tol, sw, pn)


def test_full_pro_shape_sampled_tokens_and_full_weight_gradients():
    # T = 4096, N = 4, D = 5120, bf16, both norms: per-token outputs on 64
    # sampled tokens, the weight gradients (sums over every token) in full,
    # the oracle run over blocks of tokens
    T, N, D = 4096, 4, 5120
    _say(f"[stable] full shape bf16 T={T} N={N} D={D}, both norms")
    inp, Hq, Hr, wy, wx = _case("bf16", N, D, T, seed=4096)
    xn, grads = _gpu(inp, Hq, Hr, wy, wx, True, True)
    tol = TOL["bf16"]
    idx = np.sort(np.random.default_rng(5).choice(T, 64, replace=False))
    assert_close("x_next", host(xn[idx]), _oracle_fwd(inp, Hq, Hr, wy, wx, True, True, idx), tol)
    ref = _oracle_bwd(inp, Hq, Hr, wy, wx, True, True, idx)
    dx, dy, dHq, dHr, dwy, dwx = grads
    assert_close("dx", host(dx[idx]), ref["dx"], tol)
    assert_close("dy", host(dy[idx]), ref["dy"], tol)
    assert_close("dH_post", host(dHq[idx]), ref["dH_post"], tol)
    assert_close("dH_res", host(dHr[idx]), ref["dH_res"], tol)
    gwy = np.zeros(D)
    gwx = np.zeros(N * D)
    for t0 in range(0, T, 512):
        r = _oracle_bwd(inp, Hq, Hr, wy, wx, True, True, slice(t0, t0 + 512))
        gwy += r["dy_weight"]
        gwx += r["dout_weight"]
    assert_close("dy_weight", host(dwy), gwy, tol)
    assert_close("dout_weight", host(dwx), gwx, tol)


def test_no_weights_is_mhc_post_bit_for_bit():
    _say("[stable] no weights == mhc_post / mhc_post_bwd")
    inp, Hq, Hr, wy, wx = _case("bf16", 4, 5120, 21, seed=3)
    x, y, Hq_d, Hr_d = dev(inp.x, "bf16"), dev(inp.y, "bf16"), dev(Hq), dev(Hr)
    dxn = dev(inp.dx_next, "bf16")
    a = mhc.mhc_post_stable(x, y, Hq_d, Hr_d)
    b = mhc.mhc_post(x, y, Hq_d, Hr_d)
    ga = mhc.mhc_post_stable_bwd(dxn, x, y, Hq_d, Hr_d)
    gb = mhc.mhc_post_bwd(dxn, x, y, Hq_d, Hr_d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for u, v in zip(ga[:4], gb):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)
    assert ga[4] is None and ga[5] is None


def test_backward_is_deterministic():
    _say("[stable] two backward calls, same bits")
    inp, Hq, Hr, wy, wx = _case("bf16", 4, 5120, 700, seed=8)
    _, g1 = _gpu(inp, Hq, Hr, wy, wx, True, True)
    _, g2 = _gpu(inp, Hq, Hr, wy, wx, True, True)
    for u, v in zip(g1, g2):
        assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_argument_errors():
    inp, Hq, Hr, wy, wx = _case("bf16", 4, 256, 5, seed=1)
    x, y, Hq_d, Hr_d = dev(inp.x, "bf16"), dev(inp.y, "bf16"), dev(Hq), dev(Hr)
    dxn = dev(inp.dx_next, "bf16")
    # a weight gradient must be given exactly when its weight is (the
    # binding refuses the call before the library sees it)
    T, N, D = x.shape
    f32 = dict(dtype=torch.float32, device="cuda")
    out = (torch.empty_like(x), torch.empty_like(y), torch.empty((T, N), **f32),
           torch.empty((T, N, N), **f32), None, None)
    with pytest.raises(ValueError, match="dy_weight"):
        mhc.mhc_post_stable_bwd(dxn, x, y, Hq_d, Hr_d, y_weight=dev(wy), out=out)
    # ... and the library refuses it too, called through the C ABI directly
    lib, wy_d = mhc.load(), dev(wy)
    d = mhc.desc_for(x)
    ws = torch.empty(mhc.workspace_bytes("post_stable_bwd", T, N, D, mhc.MHC_BF16, y_weight=True) + 256,
                     dtype=torch.uint8, device="cuda")
    st = lib.mhc_post_stable_bwd(ctypes.byref(d), dxn.data_ptr(), x.data_ptr(), y.data_ptr(), wy_d.data_ptr(),
                                 Hq_d.data_ptr(), Hr_d.data_ptr(), None, out[0].data_ptr(), out[1].data_ptr(),
                                 None, None, out[2].data_ptr(), out[3].data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == mhc.MHC_ERR_INVALID_ARG
    # too small a workspace
    with pytest.raises(mhc.MhcError):
        mhc.mhc_post_stable_bwd(dxn, x, y, Hq_d, Hr_d, y_weight=dev(wy),
                                workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    # x_next may not alias x
    with pytest.raises(mhc.MhcError):
        mhc.mhc_post_stable(x, y, Hq_d, Hr_d, y_weight=dev(wy), out=x)
    # eight streams with a norm are outside the supported shapes
    big = make_inputs(3, 8, 64, io="f32", seed=2)
    Hq8, Hr8 = make_coefficients(3, 8, seed=3)
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_post_stable(dev(big.x, "f32"), dev(big.y, "f32"), dev(Hq8), dev(Hr8),
                            y_weight=dev(np.ones(64, np.float32)))
    assert e.value.status == mhc.MHC_ERR_UNSUPPORTED
