"""mhc_post_pre (hc_post of one layer fused with hc_pre of the next) through
the C ABI: equal bit for bit to mhc_post followed by mhc_pre, and within the
bf16/fp32 tolerance of the fp64 oracle composition (hc_post, rounding of
x_next to the I/O dtype, hc_pre)."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import mhc_oracle as O
from residual_stream_amd import mhc
from residual_stream_amd.inputs import make_coefficients, make_inputs, to_io

from mhc_testlib import assert_close, dev, host, tol_of

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _case(T, N, D, io, seed):
    """Inputs of the fused call, all seeded: the state x, the sublayer output
    y, the previous layer's coefficients H_post / H_res (drawn in their
    ranges), and the next layer's φ and bias (a second draw)."""
    a = make_inputs(T, N, D, io=io, seed=seed, alpha=0.3)
    b = make_inputs(T, N, D, io=io, seed=seed + 1000, alpha=0.3)
    x, y = dev(a.x, io), dev(a.y, io)
    Hq, Hr = make_coefficients(T, N, seed=seed + 2000)
    return a, b, x, y, dev(Hq), dev(Hr)


def _both(a, b, x, y, Hq, Hr):
    kw = dict(iters=b.iters, eps=b.eps, alphas=b.alphas)
    fused = mhc.mhc_post_pre(x, y, Hq, Hr, dev(b.phi), dev(b.bias), **kw)
    xn = mhc.mhc_post(x, y, Hq, Hr)
    sep = (xn,) + tuple(mhc.mhc_pre(xn, dev(b.phi), dev(b.bias), **kw))
    torch.cuda.synchronize()
    return fused, sep


def _bitwise(name, f, s):
    assert torch.equal(f.view(torch.int16) if f.dtype == torch.bfloat16 else f,
                       s.view(torch.int16) if s.dtype == torch.bfloat16 else s), f"{name} differs"


NAMES = ("x_next", "h", "H_pre", "H_post", "H_res")


@pytest.mark.parametrize("T", [1, 5, 37, 130])
@pytest.mark.parametrize("D", [2560, 5120])
def test_fused_equals_post_then_pre_split_k_shapes(T, D):
    _say(f"[post_pre] bf16 N=4 D={D} T={T}")
    fused, sep = _both(*_case(T, 4, D, "bf16", seed=T + D))
    for name, f, s in zip(NAMES, fused, sep):
        _bitwise(name, f, s)


@pytest.mark.parametrize("io,N,T,D", [("bf16", 4, 37, 512), ("f32", 4, 33, 5120), ("bf16", 2, 9, 64),
                                      ("f32", 8, 5, 40)])
def test_fused_equals_post_then_pre_other_shapes(io, N, T, D):
    _say(f"[post_pre] {io} N={N} D={D} T={T} (two-kernel path)")
    fused, sep = _both(*_case(T, N, D, io, seed=3))
    for name, f, s in zip(NAMES, fused, sep):
        _bitwise(name, f, s)


@pytest.mark.parametrize("io,T,D", [("bf16", 130, 5120), ("bf16", 70, 2560), ("f32", 33, 256)])
def test_fused_matches_oracle(io, T, D):
    _say(f"[post_pre] oracle {io} T={T} D={D}")
    a, b, x, y, Hq, Hr = _case(T, 4, D, io, seed=21)
    kw = dict(iters=b.iters, eps=b.eps, alphas=b.alphas)
    xn, h, Hp2, Hq2, Hr2 = mhc.mhc_post_pre(x, y, Hq, Hr, dev(b.phi), dev(b.bias), **kw)
    torch.cuda.synchronize()
    Hq_ref, Hr_ref = make_coefficients(T, 4, seed=21 + 2000)
    ref_xn = O.hc_post(a.x, a.y, Hq_ref, Hr_ref)
    assert_close("x_next", host(xn), ref_xn, tol_of("x_next", io))
    # the next layer reads x_next as stored (rounded to the I/O dtype)
    xn_io = to_io(ref_xn.astype(np.float32), io).astype(np.float64)
    ref = O.hc_pre(xn_io, b.phi, b.bias, b.alphas, b.eps, b.iters)
    for name, got in (("h", h), ("H_pre", Hp2), ("H_post", Hq2), ("H_res", Hr2)):
        assert_close(name, host(got), ref[name], tol_of(name, io))


def test_fused_full_size_equals_post_then_pre():
    _say("[post_pre] bf16 T=4096 N=4 D=5120, all outputs bit for bit")
    fused, sep = _both(*_case(4096, 4, 5120, "bf16", seed=99))
    for name, f, s in zip(NAMES, fused, sep):
        _bitwise(name, f, s)


def test_fused_rejects_aliasing():
    a, b, x, y, Hq, Hr = _case(5, 4, 256, "bf16", seed=1)
    with pytest.raises(mhc.MhcError):
        mhc.mhc_post_pre(x, y, Hq, Hr, dev(b.phi), dev(b.bias),
                         out=(x, torch.empty_like(y), torch.empty_like(Hq), torch.empty_like(Hq),
                              torch.empty_like(Hr)))


def test_graph_replay_with_cleared_workspace_matches_eager():
    # the split-K hc_pre (and the fused call) captured in a graph together with a
    # zero fill of the workspace; replayed with new input contents, every replay
    # must equal the eager call on the same inputs, bit for bit
    _say("[graph] split-K hc_pre and mhc_post_pre under graph replay")
    T, N, D = 300, 4, 5120
    sets = [make_inputs(T, N, D, io="bf16", seed=s, alpha=0.3) for s in (31, 32, 33)]
    Hq0, Hr0 = make_coefficients(T, N, seed=34)
    Hq0, Hr0 = dev(Hq0), dev(Hr0)
    x = dev(sets[0].x, "bf16")
    y = dev(sets[0].y, "bf16")
    phi, bias = dev(sets[0].phi), dev(sets[0].bias)
    kw = dict(iters=sets[0].iters, eps=sets[0].eps, alphas=sets[0].alphas)
    out_pre = (torch.empty((T, D), dtype=torch.bfloat16, device="cuda"), torch.empty((T, N), device="cuda"),
               torch.empty((T, N), device="cuda"), torch.empty((T, N, N), device="cuda"))
    out_pp = (torch.empty_like(x),) + tuple(torch.empty_like(t) for t in out_pre)
    ws = torch.empty(mhc.workspace_bytes("pre", T, N, D, mhc.MHC_BF16), dtype=torch.uint8, device="cuda")
    ws2 = torch.empty_like(ws)
    mhc.mhc_pre(x, phi, bias, out=out_pre, workspace=ws, **kw)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ws.zero_()
        mhc.mhc_pre(x, phi, bias, out=out_pre, workspace=ws, **kw)
        ws2.zero_()
        mhc.mhc_post_pre(x, y, Hq0, Hr0, phi, bias, out=out_pp, workspace=ws2, **kw)
    for rep in range(6):
        src = sets[rep % 3]
        x.copy_(dev(src.x, "bf16"))
        y.copy_(dev(src.y, "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_pre = mhc.mhc_pre(x, phi, bias, **kw)
        ref_pp = mhc.mhc_post_pre(x, y, Hq0, Hr0, phi, bias, **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("h", "H_pre", "H_post", "H_res"), out_pre, ref_pre):
            _bitwise(f"replay {rep} pre {name}", a, b)
        for name, a, b in zip(NAMES, out_pp, ref_pp):
            _bitwise(f"replay {rep} post_pre {name}", a, b)


def test_graph_replay_with_uncleared_caller_workspace_matches_eager():
    # a caller's workspace, never zero-filled, captured with the calls: the
    # exchange tags still change on every replay (the packing kernel of each
    # call advances an epoch in the workspace), so replays on new inputs equal
    # the eager calls bit for bit
    _say("[graph] caller workspace, not cleared")
    T, N, D = 300, 4, 5120
    sets = [make_inputs(T, N, D, io="bf16", seed=s, alpha=1.0) for s in (41, 42, 43)]
    x = dev(sets[0].x, "bf16")
    phi, bias = dev(sets[0].phi), dev(sets[0].bias)
    kw = dict(iters=sets[0].iters, eps=sets[0].eps, alphas=sets[0].alphas)
    out_pre = (torch.empty((T, D), dtype=torch.bfloat16, device="cuda"), torch.empty((T, N), device="cuda"),
               torch.empty((T, N), device="cuda"), torch.empty((T, N, N), device="cuda"))
    ws = torch.full((mhc.workspace_bytes("pre", T, N, D, mhc.MHC_BF16),), 0x5A, dtype=torch.uint8, device="cuda")
    mhc.mhc_pre(x, phi, bias, out=out_pre, workspace=ws, **kw)  # warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mhc.mhc_pre(x, phi, bias, out=out_pre, workspace=ws, **kw)
    for rep in range(6):
        src = sets[rep % 3]
        x.copy_(dev(src.x, "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = mhc.mhc_pre(x, phi, bias, **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("h", "H_pre", "H_post", "H_res"), out_pre, ref):
            _bitwise(f"replay {rep} {name}", a, b)


def test_uncleared_workspaces_over_earlier_calls_records_match_fresh_ones():
    # one buffer, never cleared, serves as the workspace at shifting offsets,
    # so each call finds records, headers and packed φ of earlier calls (on
    # other inputs) at every position of its own workspace; each result must
    # equal that of a call on a zeroed workspace of its own, bit for bit
    _say("[workspace] uncleared buffer at shifting offsets")
    T, N, D = 300, 4, 5120
    sets = [make_inputs(T, N, D, io="bf16", seed=s, alpha=1.0) for s in (51, 52, 53)]
    kw = dict(iters=sets[0].iters, eps=sets[0].eps, alphas=sets[0].alphas)
    need = mhc.workspace_bytes("pre", T, N, D, mhc.MHC_BF16)
    big = torch.full((need + 64 * 256,), 0x5A, dtype=torch.uint8, device="cuda")
    xs = [dev(s.x, "bf16") for s in sets]
    phi, bias = dev(sets[0].phi), dev(sets[0].bias)
    for k, off in enumerate((0, 256, 4096, 0, 512, 256, 8192, 0, 768, 4096, 1024, 0, 16128, 256)):
        x = xs[k % 3]
        got = mhc.mhc_pre(x, phi, bias, workspace=big[off:off + need], **kw)
        ref = mhc.mhc_pre(x, phi, bias, workspace=torch.zeros(need, dtype=torch.uint8, device="cuda"), **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(("h", "H_pre", "H_post", "H_res"), got, ref):
            _bitwise(f"call {k} (offset {off}) {name}", a, b)
