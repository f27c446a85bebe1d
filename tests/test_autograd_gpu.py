"""MHCBlock (torch.autograd wiring of the four C-ABI calls) against the fp64
oracle: x_next, and the gradients of a linear loss with respect to x, φ, b and
α, through a sublayer y = c ⊙ h with a fixed seeded vector c.  The oracle
composes the same steps from the seeded inputs alone (hc_pre, y = c ⊙ h,
hc_post; then hc_post_bwd, dh = c ⊙ dy, hc_pre_bwd), in fp64 without the
rounding of h, y and dh to the I/O dtype that the GPU path stores; that
rounding stays inside the tolerance."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import mhc_oracle as O
from residual_stream_amd.inputs import make_inputs, make_norm_weights

from mhc_testlib import TOL, assert_close, dev, host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


class _Scale(torch.nn.Module):
    """y = h ⊙ c with a fixed per-d vector c (a stand-in sublayer with an exact backward)."""

    def __init__(self, c):
        super().__init__()
        self.register_buffer("c", c)

    def forward(self, h):
        return h * self.c


def _scale_vector(inp):
    return make_norm_weights(inp.N, inp.D, seed=7)[0]  # U(0.5, 1.5)[D]


def _run(inp, recompute):
    from residual_stream_amd.autograd import MHCBlock

    io = inp.io
    c = dev(_scale_vector(inp), io)
    g = dev(inp.dx_next, io)
    block = MHCBlock(_Scale(c), inp.N, inp.D, iters=inp.iters, eps=inp.eps, alpha=inp.alphas,
                     train_alpha=True, recompute=recompute)
    with torch.no_grad():
        block.phi.copy_(dev(inp.phi))
        block.bias.copy_(dev(inp.bias))
    x = dev(inp.x, io).requires_grad_(True)
    xn = block(x)
    (xn.float() * g.float()).sum().backward()
    torch.cuda.synchronize()
    return block, x, xn


@pytest.mark.parametrize("io,T,D", [("bf16", 70, 256), ("f32", 33, 64), ("bf16", 5, 512)])
def test_block_matches_oracle(io, T, D):
    _say(f"[autograd] io={io} T={T} D={D}")
    inp = make_inputs(T, 4, D, io=io, seed=11, alpha=0.3, grads=True)
    block, x, xn = _run(inp, recompute=False)
    c = _scale_vector(inp).astype(np.float64)
    ref = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
    y = ref["h"] * c[None, :]
    tol = TOL[io]
    assert_close("x_next", host(xn), O.hc_post(inp.x, y, ref["H_post"], ref["H_res"]), tol)
    dx_post, dy, dHq, dHr = O.hc_post_bwd(inp.dx_next, inp.x, y, ref["H_post"], ref["H_res"])
    dh = dy * c[None, :]
    pre = O.hc_pre_bwd(dh, inp.x, inp.phi, inp.bias, dHq, dHr, inp.alphas, inp.eps, inp.iters)
    assert_close("dx", host(x.grad), dx_post + pre["dx"], tol)
    assert_close("dphi", host(block.phi.grad), pre["dphi"], tol)
    assert_close("dbias", host(block.bias.grad), pre["dbias"], tol)
    assert_close("dalpha", block.alpha.grad.double().cpu().numpy(), pre["dalpha"], tol)


def test_recompute_gives_identical_gradients():
    _say("[autograd] recompute on/off, bf16 T=70 D=256")
    inp = make_inputs(70, 4, 256, io="bf16", seed=5, alpha=0.3, grads=True)
    a = _run(inp, recompute=False)
    b = _run(inp, recompute=True)
    assert torch.equal(a[2], b[2])
    assert torch.equal(a[1].grad, b[1].grad)
    assert torch.equal(a[0].phi.grad, b[0].phi.grad)
    assert torch.equal(a[0].bias.grad, b[0].bias.grad)
    assert torch.equal(a[0].alpha.grad, b[0].alpha.grad)


def test_batched_state_shape():
    _say("[autograd] [B, S, N, D] input")
    inp = make_inputs(12, 4, 64, io="f32", seed=2)
    from residual_stream_amd.autograd import MHCBlock

    block = MHCBlock(torch.nn.Identity(), 4, 64)
    x = dev(inp.x, "f32").reshape(3, 4, 4, 64)
    out = block(x)
    assert out.shape == x.shape
    flat = block(x.reshape(12, 4, 64))
    assert torch.equal(out.reshape(12, 4, 64), flat)


@pytest.mark.parametrize("io,T,D", [("bf16", 70, 256), ("f32", 33, 64)])
def test_stabilised_block_matches_oracle(io, T, D):
    # openPangu's variant: sandwich norm, block post-norm and a weighted hc_pre
    # norm, all three weights trained; the oracle composes hc_pre_weighted,
    # y = c ⊙ h and hc_post_stable, then their backward passes
    _say(f"[autograd] stabilised block io={io} T={T} D={D}")
    from residual_stream_amd.autograd import MHCBlock

    N = 4
    inp = make_inputs(T, N, D, io=io, seed=13, alpha=0.3, grads=True)
    wy, wx = make_norm_weights(N, D, seed=14)
    wp = make_norm_weights(N, D, seed=15)[1]
    c = _scale_vector(inp)
    block = MHCBlock(_Scale(dev(c, io)), N, D, iters=inp.iters, eps=inp.eps, alpha=inp.alphas,
                     train_alpha=True, sandwich_norm=True, post_norm=True, pre_norm_weight=True)
    with torch.no_grad():
        block.phi.copy_(dev(inp.phi))
        block.bias.copy_(dev(inp.bias))
        block.y_weight.copy_(dev(wy))
        block.out_weight.copy_(dev(wx))
        block.pre_weight.copy_(dev(wp))
    x = dev(inp.x, io).requires_grad_(True)
    xn = block(x)
    (xn.float() * dev(inp.dx_next, io).float()).sum().backward()
    torch.cuda.synchronize()

    c = c.astype(np.float64)
    pre = O.hc_pre_weighted(inp.x, wp, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
    y = pre["h"] * c[None, :]
    tol = TOL[io]
    assert_close("x_next", host(xn),
                 O.hc_post_stable(inp.x, y, pre["H_post"], pre["H_res"], wy, wx, inp.eps), tol)
    post = O.hc_post_stable_bwd(inp.dx_next, inp.x, y, pre["H_post"], pre["H_res"], wy, wx, inp.eps)
    dh = post["dy"] * c[None, :]
    pb = O.hc_pre_weighted_bwd(dh, inp.x, wp, inp.phi, inp.bias, post["dH_post"], post["dH_res"],
                               inp.alphas, inp.eps, inp.iters)
    assert_close("dx", host(x.grad), post["dx"] + pb["dx"], tol)
    assert_close("dphi", host(block.phi.grad), pb["dphi"], tol)
    assert_close("dbias", host(block.bias.grad), pb["dbias"], tol)
    assert_close("dalpha", block.alpha.grad.double().cpu().numpy(), pb["dalpha"], tol)
    assert_close("dy_weight", host(block.y_weight.grad), post["dy_weight"], tol)
    assert_close("dout_weight", host(block.out_weight.grad), post["dout_weight"], tol)
    assert_close("dpre_weight", host(block.pre_weight.grad), pb["dnorm_weight"], tol)


@pytest.mark.parametrize("io,D,L", [("bf16", 2560, 3), ("bf16", 5120, 2), ("f32", 256, 3)])
def test_stack_equals_blocks_one_after_another(io, D, L):
    # the fused boundary (mhc_post_pre) equals hc_post then hc_pre bit for bit,
    # and the stack's backward runs the blocks' kernels in the same order:
    # outputs and every gradient must be identical (bf16 at D = 2560 / 5120 runs
    # the fused split-K kernel; the f32 case its two-kernel fallback)
    _say(f"[autograd] stack of {L} blocks vs blocks in sequence, io={io} D={D}")
    from residual_stream_amd.autograd import MHCBlock, MHCStack

    N, T = 4, 70
    blocks = []
    for li in range(L):
        inp_l = make_inputs(T, N, D, io=io, seed=50 + li, alpha=0.3)
        c = make_norm_weights(N, D, seed=60 + li)[0]
        b = MHCBlock(_Scale(dev(c, io)), N, D, iters=inp_l.iters, eps=inp_l.eps, alpha=inp_l.alphas,
                     train_alpha=True)
        with torch.no_grad():
            b.phi.copy_(dev(inp_l.phi))
            b.bias.copy_(dev(inp_l.bias))
        blocks.append(b)
    inp = make_inputs(T, N, D, io=io, seed=49, grads=True)
    g = dev(inp.dx_next, io).float()
    params = [p for b in blocks for p in (b.phi, b.bias, b.alpha)]

    def run(fn):
        for p in params:
            p.grad = None
        x = dev(inp.x, io).requires_grad_(True)
        out = fn(x)
        (out.float() * g).sum().backward()
        torch.cuda.synchronize()
        return out.detach(), x.grad, [p.grad.clone() for p in params]

    def chain(x):
        for b in blocks:
            x = b(x)
        return x

    a = run(chain)
    s = run(MHCStack(blocks))
    assert torch.equal(a[0], s[0]), "x_L differs"
    assert torch.equal(a[1], s[1]), "dx differs"
    for i, (u, v) in enumerate(zip(a[2], s[2])):
        assert torch.equal(u, v), f"parameter gradient {i} differs"


def test_stack_rejects_stabilised_blocks():
    from residual_stream_amd.autograd import MHCBlock, MHCStack

    b = MHCBlock(torch.nn.Identity(), 4, 64, sandwich_norm=True)
    with pytest.raises(ValueError):
        MHCStack([b, MHCBlock(torch.nn.Identity(), 4, 64)])


def test_block_forward_backward_captured_in_a_graph():
    # forward + backward of a block with a trained α captured in one HIP graph
    # (no host synchronisation anywhere in either direction); every replay on
    # new inputs equals the eager step, outputs and all four gradients
    from residual_stream_amd.autograd import MHCBlock

    _say("[autograd] block forward + backward in a graph")
    T, N, D, io = 130, 4, 5120, "bf16"
    sets = [make_inputs(T, N, D, io=io, seed=60 + k, alpha=0.3, grads=True) for k in range(3)]
    c = dev(_scale_vector(sets[0]), io)
    block = MHCBlock(_Scale(c), N, D, iters=20, eps=1e-6, alpha=(0.3, 0.2, 0.4), train_alpha=True)
    with torch.no_grad():
        block.phi.copy_(dev(sets[0].phi))
        block.bias.copy_(dev(sets[0].bias))
    x_s = dev(sets[0].x, io).requires_grad_(True)
    g_s = dev(sets[0].dx_next, io)
    params = (block.phi, block.bias, block.alpha)

    def step():
        out = block(x_s)
        out.backward(g_s)
        return out

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            for p in params + (x_s,):
                p.grad = None
            step()
    torch.cuda.current_stream().wait_stream(side)
    for p in params + (x_s,):
        p.grad = None
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out_s = step()
    for rep in range(5):
        src = sets[rep % 3]
        with torch.no_grad():
            x_s.copy_(dev(src.x, io))
            g_s.copy_(dev(src.dx_next, io))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [out_s.clone()] + [t.grad.clone() for t in (x_s,) + params]
        # the eager step on the same inputs, into fresh gradients
        saved = [t.grad for t in (x_s,) + params]
        for t in (x_s,) + params:
            t.grad = None
        ref = [step().detach().clone()] + [t.grad.clone() for t in (x_s,) + params]
        torch.cuda.synchronize()
        for t, s_ in zip((x_s,) + params, saved):
            t.grad = s_
        for name, a, b in zip(("x_next", "dx", "dphi", "dbias", "dalpha"), got, ref):
            a_ = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
            b_ = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
            assert torch.equal(a_, b_), f"replay {rep}: {name} differs from the eager step"
