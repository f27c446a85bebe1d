"""mhc_post_bwd without dx + mhc_pre_bwd_mix (hc_post's share of the state
gradient formed inside the hc_pre backward) through the C ABI: against the
fp64 oracle (the total dx = H_resᵀ·dx_next + the hc_pre part), against the
two-call path mhc_post_bwd → mhc_pre_bwd (bit for bit: the mix is rounded as
mhc_post_bwd rounds its dx, on the matrix-core path inside the dx pass, on
other shapes by a separate kernel), and on its argument checks.  Inputs: the seeded
``make_inputs`` instances."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from residual_stream_amd import mhc
from residual_stream_amd.inputs import make_inputs

from mhc_testlib import TOL, assert_close, tol_of, dev, gpu_forward, host, oracle_backward

pytestmark = pytest.mark.gpu

# (io, N, D, T, fused): the bf16 matrix-core dx pass mixes in its own
# registers (fused); the fp32 tiled passes and the per-token kernels take the
# mix as a separate kernel first.  T = 37 and 70 leave ragged last tiles.
CASES = [("bf16", 4, 5120, 37, True), ("bf16", 4, 2560, 70, True), ("bf16", 4, 256, 19, True),
         ("f32", 4, 2560, 33, False), ("f32", 4, 5120, 17, False), ("bf16", 2, 512, 20, False),
         ("f32", 8, 64, 5, False), ("bf16", 1, 72, 9, False)]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _run(inp):
    x, y = dev(inp.x, inp.io), dev(inp.y, inp.io)
    phi, bias = dev(inp.phi), dev(inp.bias)
    dxn, dh = dev(inp.dx_next, inp.io), dev(inp.dh, inp.io)
    fwd = gpu_forward(inp)
    kw = dict(iters=inp.iters, eps=inp.eps, alphas=inp.alphas)
    # the two calls
    dx2, dy2, dHp2, dHr2 = mhc.mhc_post_bwd(dxn, x, y, fwd["H_post"], fwd["H_res"])
    two = mhc.mhc_pre_bwd(dh, x, phi, bias, dHp2, dHr2, dx2, **kw)
    # the mixing pair
    none, dy, dHp, dHr = mhc.mhc_post_bwd(dxn, x, y, fwd["H_post"], fwd["H_res"], want_dx=False)
    mix = mhc.mhc_pre_bwd_mix(dh, x, phi, bias, dHp, dHr, dxn, fwd["H_res"], **kw)
    torch.cuda.synchronize()
    assert none is None
    return (dy2, dHp2, dHr2, two), (dy, dHp, dHr, mix)


@pytest.mark.parametrize("io,N,D,T,fused", CASES)
def test_mix_matches_oracle_and_the_two_calls(io, N, D, T, fused):
    _say(f"[mix] {io} N={N} D={D} T={T} fused={fused}")
    inp = make_inputs(T, N, D, io=io, seed=500 + T, alpha=0.3, grads=True)
    (dy2, dHp2, dHr2, two), (dy, dHp, dHr, mix) = _run(inp)
    # post backward without dx: the other outputs are those of the full call
    for name, a, b in (("dy", dy, dy2), ("dH_post", dHp, dHp2), ("dH_res", dHr, dHr2)):
        assert torch.equal(_bits(a), _bits(b)), name
    # dφ, dbias, dα do not depend on dx: the same bits as mhc_pre_bwd
    for name, a, b in zip(("dphi", "dbias", "dalpha"), mix[1:], two[1:]):
        assert torch.equal(a, b), name
    # the total state gradient against the oracle
    ref = oracle_backward(inp)
    for name, got in (("dx", mix[0]), ("dphi", mix[1]), ("dbias", mix[2])):
        assert_close(name, host(got), ref[name], tol_of(name, io))
    assert torch.equal(_bits(mix[0]), _bits(two[0])), f"dx differs from the two calls (fused={fused})"


def test_mix_full_shape_sampled_tokens():
    # T = 4096, N = 4, D = 5120, bf16: dx on 48 sampled tokens against the
    # oracle run on those tokens only (the backward is token-local apart from
    # dφ / dbias / dα, which equal mhc_pre_bwd's bits), the rest of the tile
    # layout exercised at full size
    T, N, D = 4096, 4, 5120
    _say(f"[mix] full shape bf16 T={T}")
    inp = make_inputs(T, N, D, io="bf16", seed=4242, grads=True)
    (_, _, _, two), (_, _, _, mix) = _run(inp)
    for name, a, b in zip(("dphi", "dbias", "dalpha"), mix[1:], two[1:]):
        assert torch.equal(a, b), name
    idx = np.sort(np.random.default_rng(9).choice(T, 48, replace=False))
    ref = oracle_backward(inp, tokens=idx)
    assert_close("dx", host(mix[0][idx]), ref["dx"], TOL["bf16"])
    assert torch.equal(_bits(mix[0]), _bits(two[0]))


@pytest.mark.parametrize("io,N,D,T", [("bf16", 4, 5120, 37), ("f32", 4, 2560, 20), ("bf16", 2, 512, 9)])
def test_mix_in_place_equals_out_of_place(io, N, D, T):
    # dx may be dx_next's own buffer: the same bits as a separate output
    _say(f"[mix] in place {io} N={N} D={D} T={T}")
    inp = make_inputs(T, N, D, io=io, seed=700 + T, grads=True)
    x, y = dev(inp.x, io), dev(inp.y, io)
    phi, bias = dev(inp.phi), dev(inp.bias)
    dxn, dh = dev(inp.dx_next, io), dev(inp.dh, io)
    fwd = gpu_forward(inp)
    kw = dict(iters=inp.iters, eps=inp.eps, alphas=inp.alphas)
    _, _, dHp, dHr = mhc.mhc_post_bwd(dxn, x, y, fwd["H_post"], fwd["H_res"], want_dx=False)
    sep = mhc.mhc_pre_bwd_mix(dh, x, phi, bias, dHp, dHr, dxn, fwd["H_res"], **kw)
    C = N * N + 2 * N
    f32 = dict(dtype=torch.float32, device="cuda")
    out = (dxn, torch.empty((N * D, C), **f32), torch.empty((C,), **f32), torch.empty((4,), **f32))
    inpl = mhc.mhc_pre_bwd_mix(dh, x, phi, bias, dHp, dHr, dxn, fwd["H_res"], out=out, **kw)
    torch.cuda.synchronize()
    assert inpl[0].data_ptr() == dxn.data_ptr()
    for name, u, v in zip(("dx", "dphi", "dbias", "dalpha"), sep, inpl):
        assert torch.equal(_bits(u), _bits(v)), name


def test_mix_argument_errors():
    inp = make_inputs(5, 4, 256, io="bf16", seed=3, grads=True)
    x, y = dev(inp.x, "bf16"), dev(inp.y, "bf16")
    phi, bias = dev(inp.phi), dev(inp.bias)
    dxn, dh = dev(inp.dx_next, "bf16"), dev(inp.dh, "bf16")
    fwd = gpu_forward(inp)
    _, _, dHp, dHr = mhc.mhc_post_bwd(dxn, x, y, fwd["H_post"], fwd["H_res"], want_dx=False)
    T, N, D = x.shape
    C = N * N + 2 * N
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = lambda dx: (dx, torch.empty((N * D, C), **f32), torch.empty((C,), **f32), torch.empty((4,), **f32))
    # dx may not overlap x, nor dx_next other than by being it
    with pytest.raises(mhc.MhcError):
        mhc.mhc_pre_bwd_mix(dh, x, phi, bias, dHp, dHr, dxn, fwd["H_res"], out=outs(x))
    n = dxn.numel()
    buf = torch.empty(n + 8, dtype=dxn.dtype, device="cuda")
    a, b = buf[:n].view_as(dxn), buf[8:].view_as(dxn)
    b.copy_(dxn)
    with pytest.raises(mhc.MhcError):
        mhc.mhc_pre_bwd_mix(dh, x, phi, bias, dHp, dHr, b, fwd["H_res"], out=outs(a))
    # too small a workspace
    with pytest.raises(mhc.MhcError):
        mhc.mhc_pre_bwd_mix(dh, x, phi, bias, dHp, dHr, dxn, fwd["H_res"],
                            workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
