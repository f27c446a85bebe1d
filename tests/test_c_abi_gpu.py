"""The C ABI driven from host code alone: tests/c/mhc_abi_run.cpp (built by
the package build) allocates its own device buffers and stream, runs the
forward and backward calls on inputs this test writes (the backward twice:
mhc_post_bwd + mhc_pre_bwd, and mhc_post_bwd without dx + mhc_pre_bwd_mix),
and must produce the same bits as the Python binding on the same inputs.  It also checks that
argument errors are reported before anything runs."""

from __future__ import annotations

import os
import struct
import subprocess
import sys

import numpy as np
import pytest
import torch

from residual_stream_amd import build, mhc
from residual_stream_amd.inputs import make_inputs

from mhc_testlib import dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _io_bytes(a: np.ndarray, io: str) -> bytes:
    if io == "f32":
        return np.ascontiguousarray(a, dtype=np.float32).tobytes()
    # bf16: the top 16 bits of the (already bf16-valued) float32
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16).tobytes()


@pytest.mark.parametrize("io,T,N,D", [("bf16", 300, 4, 5120), ("f32", 70, 4, 256), ("bf16", 9, 2, 64)])
def test_host_program_matches_binding(io, T, N, D, tmp_path):
    exe = build.ABI_RUN
    assert os.path.exists(exe), f"{exe} is missing: run the package build"
    _say(f"[c-abi] io={io} T={T} N={N} D={D}")
    inp = make_inputs(T, N, D, io=io, seed=T + D, alpha=0.3, grads=True)
    code = 1 if io == "bf16" else 0
    hdr = struct.pack("=q4i4f", T, N, D, code, inp.iters, inp.eps, *inp.alphas)
    blob = hdr + _io_bytes(inp.x, io) + _io_bytes(inp.y, io) + inp.phi.astype(np.float32).tobytes() + \
        inp.bias.astype(np.float32).tobytes() + _io_bytes(inp.dh, io) + _io_bytes(inp.dx_next, io)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    fin.write_bytes(blob)
    r = subprocess.run([exe, str(fin), str(fout)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    x, y = dev(inp.x, io), dev(inp.y, io)
    phi, bias = dev(inp.phi), dev(inp.bias)
    kw = dict(iters=inp.iters, eps=inp.eps, alphas=inp.alphas)
    h, Hp, Hq, Hr = mhc.mhc_pre(x, phi, bias, **kw)
    xn = mhc.mhc_post(x, y, Hq, Hr)
    dx, dy, dHq, dHr = mhc.mhc_post_bwd(dev(inp.dx_next, io), x, y, Hq, Hr)
    dx, dphi, dbias, dalpha = mhc.mhc_pre_bwd(dev(inp.dh, io), x, phi, bias, dHq, dHr, dx, **kw)
    torch.cuda.synchronize()
    ours = [h, Hp, Hq, Hr, xn, dx, dy, dHq, dHr, dphi, dbias, dalpha[:3], dx]
    names = ["h", "H_pre", "H_post", "H_res", "x_next", "dx", "dy", "dH_post", "dH_res", "dphi", "dbias",
             "dalpha", "dx of the mixing pair"]
    data = fout.read_bytes()
    off = 0
    for name, t in zip(names, ours):
        nb = t.numel() * t.element_size()
        got = np.frombuffer(data[off:off + nb], dtype=np.uint8)
        off += nb
        want = t.contiguous().view(torch.uint8).cpu().numpy().reshape(-1)
        assert np.array_equal(got, want), f"{name} differs between the host program and the binding"
    assert off == len(data)
