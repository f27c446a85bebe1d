"""The binding on the GPU: argument checks before any launch, gate scalars
held on the device, and kernel-level timing through the C ABI."""

from __future__ import annotations

import sys

import pytest
import torch

from residual_stream_amd import mhc
from residual_stream_amd.inputs import make_inputs

from mhc_testlib import dev, oracle_backward

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_wrong_shapes_and_dtypes_raise_before_launch():
    _say("[binding] argument checks")
    inp = make_inputs(8, 4, 256, io="bf16", seed=1, grads=True)
    x, y = dev(inp.x, "bf16"), dev(inp.y, "bf16")
    phi, bias = dev(inp.phi), dev(inp.bias)
    h, Hp, Hq, Hr = mhc.mhc_pre(x, phi, bias)
    with pytest.raises(ValueError, match="phi has shape"):
        mhc.mhc_pre(x, phi.t().contiguous(), bias)
    with pytest.raises(TypeError, match="y has dtype"):
        mhc.mhc_post(x, y.float(), Hq, Hr)
    with pytest.raises(ValueError, match="x_next has shape"):
        mhc.mhc_post(x, y, Hq, Hr, out=torch.empty((7, 4, 256), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="H_res has shape"):
        mhc.mhc_post(x, y, Hq, Hr[:4].contiguous())
    with pytest.raises(ValueError, match="dH_res has shape"):
        mhc.mhc_pre_bwd(dev(inp.dh, "bf16"), x, phi, bias, Hq, Hr[:, 0].contiguous(), torch.zeros_like(x))
    with pytest.raises(ValueError, match="workspace"):
        mhc.mhc_pre(x, phi, bias, workspace=torch.empty(4096, dtype=torch.uint8))
    torch.cuda.synchronize()


@pytest.mark.parametrize("T,D", [(64, 256), (300, 5120), (37, 2560)])
def test_device_alpha_equals_scalar_alpha(T, D):
    # α read from device memory gives the same bits as α passed as scalars,
    # forward and backward, on every hc_pre path
    _say(f"[binding] device alpha T={T} D={D}")
    inp = make_inputs(T, 4, D, io="bf16", seed=T, alpha=(0.7, 0.4, 1.3), grads=True)
    x, phi, bias = dev(inp.x, "bf16"), dev(inp.phi), dev(inp.bias)
    a_dev = torch.tensor(inp.alphas, dtype=torch.float32, device="cuda")
    ref = mhc.mhc_pre(x, phi, bias, alphas=inp.alphas)
    got = mhc.mhc_pre(x, phi, bias, alphas=a_dev)
    dh = dev(inp.dh, "bf16")
    Hq, Hr = ref[2], ref[3]
    rb = mhc.mhc_pre_bwd(dh, x, phi, bias, Hq, Hr, torch.zeros_like(x), alphas=inp.alphas)
    gb = mhc.mhc_pre_bwd(dh, x, phi, bias, Hq, Hr, torch.zeros_like(x), alphas=a_dev)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(_bits(a), _bits(b))
    for a, b in zip(rb, gb):
        assert torch.equal(_bits(a), _bits(b))


def test_kernel_trace_names_and_times_each_launch():
    _say("[binding] kernel trace")
    inp = make_inputs(4096, 4, 5120, io="bf16", seed=2)
    x, phi, bias = dev(inp.x, "bf16"), dev(inp.phi), dev(inp.bias)
    y = dev(inp.y, "bf16")
    out = mhc.mhc_pre(x, phi, bias)
    with mhc.KernelTrace(8) as tr:
        mhc.mhc_pre(x, phi, bias, out=out)
        mhc.mhc_post(x, y, out[2], out[3])
    torch.cuda.synchronize()
    rec = tr.durations_us()
    assert [n for n, _ in rec][:1] == ["tile::phi_pack_tile_kernel"], rec
    assert "hc_pre_tile_kernel" in rec[1][0] and "hc_post_generic" in rec[2][0], rec
    assert len(rec) == 3 and all(0 < us < 10000 for _, us in rec), rec
    # tracing is off again: further calls record nothing
    mhc.mhc_post(x, y, out[2], out[3])
    torch.cuda.synchronize()
    assert len(tr.durations_us()) == 3


@pytest.mark.parametrize("io,D", [("bf16", 5120), ("f32", 256)])
def test_empty_batch_every_call(io, D):
    """T = 0: every call succeeds without touching the (empty) token tensors,
    returns empty token outputs, and the parameter gradients, sums over no
    tokens, come back as zeros (oracle: the same sums over an empty batch),
    overwriting what the output buffers held."""
    N, C = 4, 24
    inp = make_inputs(0, N, D, io=io, seed=0, grads=True)
    ref = oracle_backward(inp)
    x, y = dev(inp.x, io), dev(inp.y, io)
    phi, bias = dev(inp.phi), dev(inp.bias)
    h, Hp, Hq, Hr = mhc.mhc_pre(x, phi, bias)
    assert h.shape == (0, D) and Hp.shape == (0, N) and Hq.shape == (0, N) and Hr.shape == (0, N, N)
    assert mhc.mhc_pre_noalloc(x, phi, bias)[0].shape == (0, D)
    assert mhc.mhc_post(x, y, Hq, Hr).shape == (0, N, D)
    assert mhc.mhc_post_pre(x, y, Hq, Hr, phi, bias)[0].shape == (0, N, D)
    dxn, dh = dev(inp.dx_next, io), dev(inp.dh, io)
    dx, dy, dHq, dHr = mhc.mhc_post_bwd(dxn, x, y, Hq, Hr)
    assert dx.shape == (0, N, D) and dy.shape == (0, D) and dHq.shape == (0, N) and dHr.shape == (0, N, N)
    nan = float("nan")
    for mix in (False, True):
        outs = (torch.full((N * D, C), nan, device="cuda"), torch.full((C,), nan, device="cuda"),
                torch.full((4,), nan, device="cuda"))
        if mix:
            g = mhc.mhc_pre_bwd_mix(dh, x, phi, bias, dHq, dHr, dxn, Hr, out=(torch.empty_like(x),) + outs)
        else:
            g = mhc.mhc_pre_bwd(dh, x, phi, bias, dHq, dHr, dx, out=outs)
        torch.cuda.synchronize()
        assert g[0].shape == (0, N, D)
        for k, t in zip(("dphi", "dbias", "dalpha"), g[1:]):
            assert torch.equal(t.cpu().double(), torch.from_numpy(ref[k])), (mix, k)
    if io == "bf16":
        wy = torch.ones(D, device="cuda")
        wx = torch.ones(N * D, device="cuda")
        assert mhc.mhc_post_stable(x, y, Hq, Hr, y_weight=wy, out_weight=wx).shape == (0, N, D)
        sb = mhc.mhc_post_stable_bwd(dxn, x, y, Hq, Hr, y_weight=wy, out_weight=wx)
        torch.cuda.synchronize()
        assert sb[0].shape == (0, N, D)
        assert torch.count_nonzero(sb[4]) == 0 and torch.count_nonzero(sb[5]) == 0
