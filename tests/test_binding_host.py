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
