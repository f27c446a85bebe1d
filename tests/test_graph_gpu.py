"""A whole mHC step (hc_pre, hc_post and both backwards, or the stabilised
write-back and its backward) captured once in a HIP graph and replayed with
new input contents: every replay must equal the same calls made eagerly on
the same inputs, bit for bit.  Eager calls and synchronisations run between
the replays, so state left behind by one replay (workspace records, exchange
tags) meets the next one."""

from __future__ import annotations

import sys

import pytest
import torch

from residual_stream_amd import mhc
from residual_stream_amd.inputs import make_coefficients, make_inputs, make_norm_weights

from mhc_testlib import dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _bitwise(name, a, b):
    assert a.shape == b.shape, (name, a.shape, b.shape)
    assert torch.equal(_bits(a), _bits(b)), f"{name}: replay differs from the eager call"


def _load(bufs, src, io):
    for name in ("x", "y", "dh", "dx_next"):
        bufs[name].copy_(dev(getattr(src, name), io))


# (io, N, D, T): the split-K hc_pre and the tiled hc_pre backward at bf16
# N = 4, D = 5120; the fp32 tiled backward at D = 2560; the generic kernels at N = 2
STEP_CASES = [("bf16", 4, 5120, 300), ("f32", 4, 2560, 70), ("bf16", 2, 512, 33)]


@pytest.mark.parametrize("mix", [False, True], ids=["two_call_bwd", "mix_bwd"])
@pytest.mark.parametrize("io,N,D,T", STEP_CASES)
def test_training_step_graph_replays_match_eager(io, N, D, T, mix):
    # mix: mhc_post_bwd without dx, then mhc_pre_bwd_mix (the backward pair
    # the benchmark's step uses); else mhc_post_bwd then mhc_pre_bwd
    _say(f"[graph] step {io} N={N} D={D} T={T} mix={mix}")
    sets = [make_inputs(T, N, D, io=io, seed=100 + s, alpha=0.3, grads=True) for s in range(3)]
    s0 = sets[0]
    kw = dict(iters=s0.iters, eps=s0.eps, alphas=s0.alphas)
    bufs = {name: dev(getattr(s0, name), io) for name in ("x", "y", "dh", "dx_next")}
    phi, bias = dev(s0.phi), dev(s0.bias)
    x, y, dh, dxn = bufs["x"], bufs["y"], bufs["dh"], bufs["dx_next"]
    f32 = dict(dtype=torch.float32, device="cuda")
    K, C = N * D, N * N + 2 * N
    pre_out = (torch.empty_like(y), torch.empty((T, N), **f32), torch.empty((T, N), **f32),
               torch.empty((T, N, N), **f32))
    xn = torch.empty_like(x)
    pb_out = (torch.empty_like(x), torch.empty_like(y), torch.empty((T, N), **f32),
              torch.empty((T, N, N), **f32))
    qb_out = (torch.empty((K, C), **f32), torch.empty((C,), **f32), torch.empty((4,), **f32))
    ws_pre = torch.empty(max(mhc.workspace_bytes("pre", T, N, D, mhc._io_of(x)), 1), dtype=torch.uint8,
                         device="cuda")
    ws_bwd = torch.empty(max(mhc.workspace_bytes("pre_bwd", T, N, D, mhc._io_of(x)), 1), dtype=torch.uint8,
                         device="cuda")

    def backward(Hq, Hr, pb, qb, ws):
        if mix:
            mhc.mhc_post_bwd(dxn, x, y, Hq, Hr, out=(None,) + tuple(pb[1:]))
            return mhc.mhc_pre_bwd_mix(dh, x, phi, bias, pb[2], pb[3], dxn, Hr, out=(pb[0],) + tuple(qb),
                                       workspace=ws, **kw)
        mhc.mhc_post_bwd(dxn, x, y, Hq, Hr, out=pb)
        return mhc.mhc_pre_bwd(dh, x, phi, bias, pb[2], pb[3], pb[0], out=qb, workspace=ws, **kw)

    def step():
        ws_pre.zero_()
        h, Hp, Hq, Hr = mhc.mhc_pre(x, phi, bias, out=pre_out, workspace=ws_pre, **kw)
        mhc.mhc_post(x, y, Hq, Hr, out=xn)
        backward(Hq, Hr, pb_out, qb_out, ws_bwd)

    step()  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        _load(bufs, sets[rep % 3], io)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (*pre_out, xn, *pb_out, *qb_out)]
        # the same calls, eagerly, into fresh outputs
        h, Hp, Hq, Hr = mhc.mhc_pre(x, phi, bias, **kw)
        xn_e = mhc.mhc_post(x, y, Hq, Hr)
        pb = tuple(torch.empty_like(t) for t in pb_out)
        qb = tuple(torch.empty_like(t) for t in qb_out)
        _, dphi, dbias, dal = backward(Hq, Hr, pb, qb, torch.empty_like(ws_bwd))
        dx, dy, dHq, dHr = pb
        torch.cuda.synchronize()
        ref = (h, Hp, Hq, Hr, xn_e, dx, dy, dHq, dHr, dphi, dbias)
        names = ("h", "H_pre", "H_post", "H_res", "x_next", "dx", "dy", "dH_post", "dH_res", "dphi", "dbias")
        for name, a, b in zip(names, got, ref):
            _bitwise(f"replay {rep} {name}", a, b)
        _bitwise(f"replay {rep} dalpha", got[-1][:3], dal)


def test_stabilised_write_back_graph_replays_match_eager():
    T, N, D, io = 200, 4, 5120, "bf16"
    _say(f"[graph] stabilised write-back {io} N={N} D={D} T={T}")
    sets = [make_inputs(T, N, D, io=io, seed=200 + s, grads=True) for s in range(3)]
    Hq, Hr = make_coefficients(T, N, seed=210)
    wy, wx = make_norm_weights(N, D, seed=211)
    Hq, Hr, wy, wx = dev(Hq), dev(Hr), dev(wy), dev(wx)
    bufs = {name: dev(getattr(sets[0], name), io) for name in ("x", "y", "dh", "dx_next")}
    x, y, dxn = bufs["x"], bufs["y"], bufs["dx_next"]
    eps = sets[0].eps
    f32 = dict(dtype=torch.float32, device="cuda")
    xn = torch.empty_like(x)
    out = (torch.empty_like(x), torch.empty_like(y), torch.empty((T, N), **f32), torch.empty((T, N, N), **f32),
           torch.empty((D,), **f32), torch.empty((N * D,), **f32))
    ws = torch.empty(mhc.workspace_bytes("post_stable_bwd", T, N, D, mhc._io_of(x), y_weight=True, out_weight=True),
                     dtype=torch.uint8, device="cuda")
    kw = dict(y_weight=wy, out_weight=wx, eps=eps)

    def step():
        mhc.mhc_post_stable(x, y, Hq, Hr, out=xn, **kw)
        mhc.mhc_post_stable_bwd(dxn, x, y, Hq, Hr, out=out, workspace=ws, **kw)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        _load(bufs, sets[rep % 3], io)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (xn, *out)]
        ref = (mhc.mhc_post_stable(x, y, Hq, Hr, **kw),) + tuple(mhc.mhc_post_stable_bwd(dxn, x, y, Hq, Hr, **kw))
        torch.cuda.synchronize()
        names = ("x_next", "dx", "dy", "dH_post", "dH_res", "dy_weight", "dout_weight")
        for name, a, b in zip(names, got, ref):
            _bitwise(f"replay {rep} {name}", a, b)
