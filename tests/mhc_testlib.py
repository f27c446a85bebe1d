"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
run the C-ABI path, run the oracle, compare normwise.

The gate is normwise per output tensor, max|gpu - oracle| / max|oracle|.
Beside it every comparison records elementwise statistics (reported, not
gated): the largest absolute error, and the largest and 99th-percentile
relative error over the elements whose reference magnitude is at least 1e-3
of the tensor's largest (relative error is meaningless near zeros).  They are
printed with the test's output and, when the environment variable
MHC_PARITY_STATS names a file, written there as JSON lines at the end of the
session.
"""

from __future__ import annotations

import os
import sys

import numpy as np
import torch

from oracle import mhc_oracle as O
from residual_stream_amd import mhc
from residual_stream_amd.inputs import IO_BF16, MhcInputs

TOL = {"f32": 1e-5, "bf16": 2e-2}
# Outputs stored in the I/O dtype (h, x_next, dx, dy) carry its rounding; the
# fp32 outputs (H_pre, H_post, H_res and the gradients dH_*, dφ, dbias, dα)
# are computed in fp32 from the exactly stored inputs, so their gate stays
# tight for bf16 I/O too.
STORED = frozenset({"h", "x_next", "dx", "dy"})
TOL_FP32_OUT = {"f32": 1e-5, "bf16": 1e-4}


def tol_of(name: str, io: str) -> float:
    """Gate of output `name` for I/O dtype `io`."""
    return TOL[io] if name in STORED else TOL_FP32_OUT[io]


def tdtype(io: str):
    return torch.bfloat16 if io == IO_BF16 else torch.float32


def dev(a: np.ndarray, io: str | None = None, device="cuda") -> torch.Tensor:
    """numpy float32 (holding I/O-dtype values) → device tensor of the I/O dtype (exact)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if io is not None:
        t = t.to(tdtype(io))
    return t.to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if den == 0:
        return float(num)
    return float(num / den)


STATS: list = []  # elementwise statistics of every comparison of this session


def elementwise_stats(got, ref) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    big = np.max(np.abs(ref)) if ref.size else 0.0
    mask = np.abs(ref) >= 1e-3 * big if big > 0 else np.zeros(ref.shape, bool)
    rel = diff[mask] / np.abs(ref[mask]) if mask.any() else np.zeros(1)
    return {"max_abs": float(diff.max()) if diff.size else 0.0,
            "max_rel": float(rel.max()), "p99_rel": float(np.percentile(rel, 99)),
            "n": int(ref.size)}


def assert_close(name, got, ref, tol, case: str = ""):
    err = normwise(got, ref)
    st = elementwise_stats(got, ref)
    st.update(name=name, case=case, normwise=err, tol=tol)
    STATS.append(st)
    print(f"    {name}: normwise {err:.2e} (gate {tol:.0e}); elementwise max abs {st['max_abs']:.2e}, "
          f"max rel {st['max_rel']:.2e}, p99 rel {st['p99_rel']:.2e} over {st['n']}", flush=True)
    sys.stdout.flush()
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert err <= tol, f"{name}: normwise error {err:.3e} > {tol:.1e}"
    return err


def write_stats():
    path = os.environ.get("MHC_PARITY_STATS")
    if not path or not STATS:
        return
    import json
    with open(path, "a") as f:
        for st in STATS:
            f.write(json.dumps(st) + "\n")


def gpu_forward(inp: MhcInputs, stream=None):
    x = dev(inp.x, inp.io)
    y = dev(inp.y, inp.io)
    phi = dev(inp.phi)
    bias = dev(inp.bias)
    kw = dict(iters=inp.iters, eps=inp.eps, alphas=inp.alphas, stream=stream)
    h, Hp, Hq, Hr = mhc.mhc_pre(x, phi, bias, **kw)
    xn = mhc.mhc_post(x, y, Hq, Hr, stream=stream)
    return {"h": h, "H_pre": Hp, "H_post": Hq, "H_res": Hr, "x_next": xn}


def gpu_backward(inp: MhcInputs, fwd=None):
    x = dev(inp.x, inp.io)
    y = dev(inp.y, inp.io)
    phi = dev(inp.phi)
    bias = dev(inp.bias)
    if fwd is None:
        fwd = gpu_forward(inp)
    dxn = dev(inp.dx_next, inp.io)
    dh = dev(inp.dh, inp.io)
    dx, dy, dHp, dHr = mhc.mhc_post_bwd(dxn, x, y, fwd["H_post"], fwd["H_res"])
    dx, dphi, dbias, dalpha = mhc.mhc_pre_bwd(dh, x, phi, bias, dHp, dHr, dx, iters=inp.iters,
                                              eps=inp.eps, alphas=inp.alphas)
    return {"dx": dx, "dy": dy, "dH_post": dHp, "dH_res": dHr, "dphi": dphi, "dbias": dbias,
            "dalpha": dalpha}


def oracle_forward(inp: MhcInputs, tokens=None):
    sel = slice(None) if tokens is None else tokens
    x = inp.x[sel]
    out = O.hc_pre(x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
    out["x_next"] = O.hc_post(x, inp.y[sel], out["H_post"], out["H_res"])
    return out


def oracle_backward(inp: MhcInputs, tokens=None):
    sel = slice(None) if tokens is None else tokens
    x, y = inp.x[sel], inp.y[sel]
    pre = O.hc_pre(x, inp.phi, inp.bias, inp.alphas, inp.eps, inp.iters)
    dx, dy, dHp, dHr = O.hc_post_bwd(inp.dx_next[sel], x, y, pre["H_post"], pre["H_res"])
    g = O.hc_pre_bwd(inp.dh[sel], x, inp.phi, inp.bias, dHp, dHr, inp.alphas, inp.eps, inp.iters)
    return {"dx": dx + g["dx"], "dy": dy, "dH_post": dHp, "dH_res": dHr, "dphi": g["dphi"],
            "dbias": g["dbias"], "dalpha": g["dalpha"]}
