"""mhc_pre_noalloc (hc_pre on the library's static scratch buffer, for
callers that cannot allocate) through the C ABI: equal bit for bit to mhc_pre
with a workspace of its own, call after call on the same buffer, each later
call on a smaller input than the one before (so it finds the larger call's
records and packed φ in the buffer), on every hc_pre path (split-K tiles at
both widths, the few-token path, the fp32 matrix-core path), and within the
bf16 tolerance of the fp64 oracle on sampled tokens; too large a call is
refused with MHC_ERR_TOO_LARGE and launches nothing."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import mhc_oracle as O
from residual_stream_amd import mhc
from residual_stream_amd.inputs import make_inputs

from mhc_testlib import assert_close, dev, host, tol_of

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _bitwise(name, a, b):
    a = a.view(torch.int16) if a.dtype == torch.bfloat16 else a
    b = b.view(torch.int16) if b.dtype == torch.bfloat16 else b
    assert torch.equal(a, b), f"{name} differs"


NAMES = ("h", "H_pre", "H_post", "H_res")

# (T, D, io): largest first, then smaller inputs, crossing the kernel paths
CALLS = [(4096, 5120, "bf16"), (1024, 5120, "f32"), (300, 5120, "bf16"), (2048, 2560, "bf16"),
         (37, 2560, "bf16"), (100, 512, "f32"), (17, 5120, "bf16")]


def test_noalloc_equals_mhc_pre_call_after_call():
    for k, (T, D, io) in enumerate(CALLS):
        _say(f"[noalloc] call {k}: T={T} N=4 D={D} io={io}")
        inp = make_inputs(T, 4, D, io=io, seed=900 + k, alpha=1.0)
        x, phi, bias = dev(inp.x, io), dev(inp.phi), dev(inp.bias)
        kw = dict(iters=inp.iters, eps=inp.eps, alphas=inp.alphas)
        assert mhc.workspace_bytes("pre", T, 4, D, mhc.MHC_BF16 if io == "bf16" else mhc.MHC_F32) \
            <= mhc.NOALLOC_SCRATCH_BYTES
        got = mhc.mhc_pre_noalloc(x, phi, bias, **kw)
        ref = mhc.mhc_pre(x, phi, bias, **kw)
        torch.cuda.synchronize()
        for name, a, b in zip(NAMES, got, ref):
            _bitwise(f"call {k} {name}", a, b)
        if k == 1:  # and the oracle, on every token of this one
            r = O.hc_pre(inp.x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
            for name, a in zip(NAMES, got):
                assert_close(name, host(a), r[name], tol_of(name, io), case=f"noalloc T={T} D={D}")


def test_noalloc_refuses_calls_beyond_its_buffer():
    T, D = 9217, 5120  # the first bf16 token count whose workspace exceeds the buffer (256 CUs)
    need = mhc.workspace_bytes("pre", T, 4, D, mhc.MHC_BF16)
    if need <= mhc.NOALLOC_SCRATCH_BYTES:
        pytest.skip("this device's tile choice fits T=9217 in the buffer")
    _say(f"[noalloc] T={T} D={D}: needs {need} bytes, refused")
    x = torch.zeros((T, 4, D), dtype=torch.bfloat16, device="cuda")
    phi = torch.zeros((4 * D, 24), dtype=torch.float32, device="cuda")
    bias = torch.zeros((24,), dtype=torch.float32, device="cuda")
    h = torch.full((T, D), 7.0, dtype=torch.bfloat16, device="cuda")
    Hs = tuple(torch.full(s, 7.0, device="cuda") for s in ((T, 4), (T, 4), (T, 4, 4)))
    with pytest.raises(mhc.MhcError) as e:
        mhc.mhc_pre_noalloc(x, phi, bias, out=(h,) + Hs)
    assert e.value.status == mhc.MHC_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((h == 7.0).all()) and all(bool((t == 7.0).all()) for t in Hs), "a refused call wrote"
