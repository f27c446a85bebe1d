"""The binding has no CPU path: a missing library or host tensors are errors,
raised on the host before anything reaches the GPU, and the autograd modules
go through the same calls."""

from __future__ import annotations

import os

import pytest
import torch

from residual_stream_amd import mhc


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        mhc.load(str(tmp_path / "libmhc.so"))


@pytest.fixture(scope="module")
def built():
    if not os.path.exists(mhc.LIB_PATH):
        pytest.skip("libmhc.so not built (run __graft_entry__.build())")
    mhc.load()


def _cpu_case(T=3, N=4, D=64, dtype=torch.float32):
    C = N * N + 2 * N
    return (torch.zeros(T, N, D, dtype=dtype), torch.zeros(T, D, dtype=dtype), torch.zeros(N * D, C),
            torch.zeros(C), torch.zeros(T, N), torch.zeros(T, N, N))


def test_host_tensors_are_rejected_by_every_call(built):
    x, y, phi, bias, Hq, Hr = _cpu_case()
    calls = [
        lambda: mhc.mhc_pre(x, phi, bias),
        lambda: mhc.mhc_post(x, y, Hq, Hr),
        lambda: mhc.mhc_post_bwd(x, x, y, Hq, Hr),
        lambda: mhc.mhc_pre_bwd(y, x, phi, bias, Hq, Hr, x.clone()),
        lambda: mhc.mhc_post_pre(x, y, Hq, Hr, phi, bias),
        lambda: mhc.mhc_post_stable(x, y, Hq, Hr),
        lambda: mhc.mhc_post_stable_bwd(x, x, y, Hq, Hr),
    ]
    for call in calls:
        with pytest.raises(RuntimeError, match="GPU tensors"):
            call()


def test_unsupported_io_dtype_is_rejected(built):
    x, y, phi, bias, Hq, Hr = _cpu_case(dtype=torch.float16)
    with pytest.raises(TypeError):
        mhc.mhc_post(x, y, Hq, Hr)


def test_descriptor_layout_matches_the_header():
    # int64 T; int32 N, D, io, iters; float eps, three alphas; const float* alpha
    import ctypes
    assert ctypes.sizeof(mhc.MhcDesc) == 48
    assert mhc.MhcDesc.alpha.offset == 40
    d = mhc.make_desc(5, 4, 64, mhc.MHC_BF16, 7, 1e-5, (0.1, 0.2, 0.3))
    assert (d.T, d.N, d.D, d.io, d.sinkhorn_iters) == (5, 4, 64, mhc.MHC_BF16, 7)
    assert d.alpha is None


def test_host_alpha_tensor_is_rejected():
    with pytest.raises(ValueError, match="device alpha"):
        mhc.make_desc(5, 4, 64, mhc.MHC_F32, alphas=torch.ones(3))


def test_argument_checks_name_the_tensor():
    # the shape / dtype / layout checks every call makes before a pointer
    # reaches the C ABI (device = x's; here the host, to run without a GPU)
    cpu = torch.device("cpu")
    sh = mhc._coef_shapes(3, 4, 64)
    assert sh == {"x": (3, 4, 64), "y": (3, 64), "phi": (256, 24), "bias": (24,), "H": (3, 4),
                  "H_res": (3, 4, 4)}
    mhc._expect("y", torch.zeros(3, 64), sh["y"], torch.float32, cpu)  # passes
    with pytest.raises(ValueError, match="y has shape"):
        mhc._expect("y", torch.zeros(3, 65), sh["y"], torch.float32, cpu)
    with pytest.raises(ValueError, match="phi has shape"):
        mhc._expect("phi", torch.zeros(24, 256), sh["phi"], torch.float32, cpu)  # transposed
    with pytest.raises(TypeError, match="dtype"):
        mhc._expect("y", torch.zeros(3, 64, dtype=torch.bfloat16), sh["y"], torch.float32, cpu)
    with pytest.raises(ValueError, match="contiguous"):
        mhc._expect("H_res", torch.zeros(3, 4, 4).transpose(1, 2), sh["H_res"], torch.float32, cpu)
    with pytest.raises(ValueError, match="required"):
        mhc._expect("dy", None, sh["y"], torch.float32, cpu)
    mhc._expect("dx", None, sh["x"], torch.float32, cpu, optional=True)
    with pytest.raises(ValueError, match="expected cuda"):
        mhc._expect("y", torch.zeros(3, 64), sh["y"], torch.float32, torch.device("cuda", 0))


def test_workspace_size_counts_bytes():
    assert mhc._ws_bytes(None) == 0
    with pytest.raises(ValueError):
        mhc._ws_bytes(torch.zeros(10, dtype=torch.float32))  # a host tensor
