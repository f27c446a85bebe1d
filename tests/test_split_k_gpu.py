"""The split-K hc_pre and the tiled hc_pre backward against the fp64 oracle,
where their own structure can go wrong.

The split-K forward (bf16 or fp32, N = 4, D = 5120 or 2560) cuts each token's
reduction into S slices of d (S = 8 or 4); a group of S workgroups walks the
tiles grp, grp + Q, grp + 2Q, ... (M = 16, 32 or 64 tokens each, 32 for fp32, Q = compute
units / S), holds the tile's x on chip from the projection to the collapse,
and workgroup `slice` of the group runs the gates and Sinkhorn of tokens
slice·M/S .. (slice+1)·M/S − 1 of each tile.  A token's coefficients sent to
the wrong token, a tile's records mixed with another's, or a finishing share
written to the wrong rows only shows where the projection matters: at alpha
= 1 (at the workloads' alpha = 0.01 the logits are almost the bias, the same
for every token).  So these cases run at alpha = 1, at full size, with
sampled tokens that cover a whole tile at both ends of a group and every
token one workgroup finishes, on both sides of a ragged end.

The Sinkhorn round count and order (openPangu 2.0 analysis, §5.3: rows then
columns, 20 rounds in the model) are pinned with large logits (bias standard
deviation 3), where one or three rounds are far from converged, so that a
wrong count or a column-first round moves H_res by much more than the gate.
"""

from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest
import torch

from oracle import mhc_oracle as O
from residual_stream_amd import mhc
from residual_stream_amd.inputs import make_coefficients, make_inputs, to_io

from mhc_testlib import (TOL, assert_close, tol_of, dev, gpu_backward, gpu_forward, host,
                         oracle_backward, oracle_forward)

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

FWD_KEYS = ("h", "H_pre", "H_post", "H_res", "x_next")
BWD_KEYS = ("dx", "dy", "dH_post", "dH_res", "dphi", "dbias", "dalpha")
TILE = 16  # tokens per tile of the tiled backward
SLICE_D_PER_WAVE = 160  # d per wave of the split-K forward


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def tile_config(T, D, io="bf16"):
    """(S, M, Q): the split-K forward's slices per group, tile size and number
    of groups for T tokens of width D, chosen as the library chooses them
    (the candidate that leaves each compute unit the least work; fp32 x takes
    twice the registers, so its tiles are 32 tokens)."""
    cus = _cus()
    best = None
    cands = ((8, 4, 32), (4, 4, 32)) if io == "f32" else ((8, 4, 64), (4, 8, 32), (4, 8, 16), (4, 4, 64),
                                                          (4, 4, 32))
    for s_, wd, m in cands:
        if s_ * wd * SLICE_D_PER_WAVE != D:
            continue
        q = cus // s_
        ntiles = (T + m - 1) // m
        work = (ntiles + q - 1) // q * m // s_
        if best is None or work < best[0]:
            best = (work, s_, m, q)
    return best[1:]


def split_k_tokens(T, D, grp=3, slice_=5, extra=24, seed=0, io="bf16"):
    """Tokens that exercise the split-K kernel's structure: all tokens of the
    first and the last tile of group `grp`, every token workgroup (grp,
    slice_) finishes in each of its tiles, the last two tokens and a random
    handful."""
    S, M, Q = tile_config(T, D, io)
    share = M // S
    ntiles = (T + M - 1) // M
    grp = min(grp, Q - 1, ntiles - 1)
    slice_ = slice_ % S
    nloc = (ntiles - grp + Q - 1) // Q
    toks = set()
    for tile in (grp, grp + (nloc - 1) * Q):
        toks.update(range(tile * M, min(T, tile * M + M)))
    for p in range(nloc):
        for u in range(share):
            toks.add((grp + p * Q) * M + slice_ * share + u)
    toks.update((0, T - 2, T - 1))
    rng = np.random.default_rng(seed)
    toks.update(rng.choice(T, extra, replace=False).tolist())
    return np.array(sorted(t for t in toks if 0 <= t < T))


def check_forward(inp, tokens=None, tag=""):
    _say(f"[fwd] {tag} T={inp.T} N={inp.N} D={inp.D} io={inp.io} alpha={inp.alphas[0]} "
         f"iters={inp.iters} tokens={'all' if tokens is None else len(tokens)}")
    g = gpu_forward(inp)
    torch.cuda.synchronize()
    r = oracle_forward(inp, tokens)
    for k in FWD_KEYS:
        got = host(g[k])
        if tokens is not None:
            got = got[tokens]
        assert_close(k, got, r[k], tol_of(k, inp.io), case=f"{tag} T={inp.T} D={inp.D}")


# -------------------------------------------- split-K forward, alpha = 1 ---

@pytest.mark.parametrize("T,D,io", [(4096, 5120, "bf16"), (4093, 5120, "bf16"), (2048, 2560, "bf16"),
                                    (4096, 2560, "bf16"), (4093, 2560, "bf16"),
                                    (1024, 5120, "f32"), (1021, 5120, "f32"), (2048, 2560, "f32"),
                                    (2045, 2560, "f32"), (4096, 5120, "f32")])
def test_split_k_forward_alpha1_full_size(T, D, io):
    inp = make_inputs(T, 4, D, io=io, seed=T + D, alpha=1.0)
    check_forward(inp, tokens=split_k_tokens(T, D, seed=T, io=io), tag="split-K alpha=1")


def test_split_k_forward_alpha1_other_group():
    # the last group and slice, so that the sampled batch is not one position only
    inp = make_inputs(4096, 4, 5120, io="bf16", seed=77, alpha=1.0)
    check_forward(inp, tokens=split_k_tokens(4096, 5120, grp=10_000, slice_=15, seed=1),
                  tag="split-K alpha=1, last group")


@pytest.mark.parametrize("iters", [1, 3, 64])
@pytest.mark.parametrize("T,D,io", [(65, 5120, "bf16"), (300, 5120, "bf16"), (300, 2560, "bf16"),
                                    (65, 5120, "f32"), (300, 2560, "f32")])
def test_split_k_sinkhorn_rounds(iters, T, D, io):
    inp = make_inputs(T, 4, D, io=io, seed=iters + T + D, alpha=1.0, iters=iters, bias_std=3.0)
    check_forward(inp, tag=f"split-K rounds={iters}")


# ------------------------------------- a group member that never publishes ---

@pytest.mark.parametrize("T,D,drop", [(300, 5120, 3), (300, 2560, 0)])
def test_lost_group_member_poisons_every_tile(T, D, drop):
    """Forced from the host (mhc_test_exchange_fault): workgroup `drop` of
    every group publishes no records and each record wait gives up after 64
    polls.  Every token then comes out as NaN, a loud failure, and the kernels
    end normally.  The next call, with the fault off, is right again: its
    records carry a new tag, so the partial records the faulty call left in
    the same workspace cannot match."""
    _say(f"[fault] drop slice {drop}, T={T} D={D}")
    lib = mhc.load()
    inp = make_inputs(T, 4, D, io="bf16", seed=T + D + drop, alpha=1.0)
    x, phi, bias = dev(inp.x, "bf16"), dev(inp.phi), dev(inp.bias)
    desc = mhc.desc_for(x, inp.iters, inp.eps, inp.alphas)
    ws = torch.empty(lib.mhc_pre_workspace_bytes(ctypes.byref(desc)), dtype=torch.uint8, device="cuda")
    assert lib.mhc_test_exchange_fault(drop, 64) == 0
    try:
        bad = mhc.mhc_pre(x, phi, bias, iters=inp.iters, eps=inp.eps, alphas=inp.alphas, workspace=ws)
        torch.cuda.synchronize()
    finally:
        assert lib.mhc_test_exchange_fault(-1, 0) == 0
    for name, t in zip(("h", "H_pre", "H_post", "H_res"), bad):
        assert torch.isnan(t.float()).all(), name
    good = mhc.mhc_pre(x, phi, bias, iters=inp.iters, eps=inp.eps, alphas=inp.alphas, workspace=ws)
    torch.cuda.synchronize()
    r = oracle_forward(inp)
    for name, t in zip(("h", "H_pre", "H_post", "H_res"), good):
        assert_close(name, host(t), r[name], tol_of(name, "bf16"), case=f"after the fault, T={T} D={D}")


def test_fault_switch_rejects_bad_arguments():
    lib = mhc.load()
    assert lib.mhc_test_exchange_fault(-2, 64) == mhc.MHC_ERR_INVALID_ARG
    assert lib.mhc_test_exchange_fault(0, 0) == mhc.MHC_ERR_INVALID_ARG
    assert lib.mhc_test_exchange_fault(-1, 0) == 0


# ------------------------ hc_post + next hc_pre in one call, alpha = 1 ---

@pytest.mark.parametrize("T,D", [(4096, 5120), (4093, 2560)])
def test_fused_post_pre_alpha1_full_size(T, D):
    _say(f"[post_pre] oracle composition, alpha=1, T={T} D={D}")
    a = make_inputs(T, 4, D, io="bf16", seed=T + 5, alpha=1.0)
    b = make_inputs(T, 4, D, io="bf16", seed=T + 1005, alpha=1.0)
    Hq_ref, Hr_ref = make_coefficients(T, 4, seed=T + 2005)
    x, y = dev(a.x, "bf16"), dev(a.y, "bf16")
    kw = dict(iters=b.iters, eps=b.eps, alphas=b.alphas)
    xn, h, Hp, Hq, Hr = mhc.mhc_post_pre(x, y, dev(Hq_ref), dev(Hr_ref), dev(b.phi), dev(b.bias), **kw)
    torch.cuda.synchronize()
    tk = split_k_tokens(T, D, seed=T + 5)
    ref_xn = O.hc_post(a.x[tk], a.y[tk], Hq_ref[tk], Hr_ref[tk])
    case = f"post_pre alpha=1 T={T} D={D}"
    assert_close("x_next", host(xn)[tk], ref_xn, TOL["bf16"], case=case)
    # the next layer reads the state as stored (rounded to bf16)
    xn_io = to_io(ref_xn.astype(np.float32), "bf16").astype(np.float64)
    ref = O.hc_pre(xn_io, b.phi, b.bias, b.alphas, b.eps, b.iters)
    for name, got in (("h", h), ("H_pre", Hp), ("H_post", Hq), ("H_res", Hr)):
        assert_close(name, host(got)[tk], ref[name], tol_of(name, "bf16"), case=case)


# ----------------------------------------- tiled backward, alpha = 1 ---

def _bwd_tokens(T, seed=0):
    # both sides of every 16-token tile edge at the start and the end, and of
    # the token splits' edges (multiples of 16 near T/12·k), plus random ones
    rng = np.random.default_rng(seed)
    toks = set(range(0, 33)) | set(range(T - 33, T))
    for k in range(1, 12):
        c = (T * k // 12) // TILE * TILE
        toks.update((c - 1, c, c + 1))
    toks.update(rng.choice(T, 40, replace=False).tolist())
    return np.array(sorted(t for t in toks if 0 <= t < T))


def check_backward(inp, tokens=None, tag=""):
    _say(f"[bwd] {tag} T={inp.T} N={inp.N} D={inp.D} io={inp.io} alpha={inp.alphas[0]} iters={inp.iters}")
    g = gpu_backward(inp)
    torch.cuda.synchronize()
    r = oracle_backward(inp)
    for k in BWD_KEYS:
        got, ref = host(g[k]), r[k]
        if tokens is not None and k not in ("dphi", "dbias", "dalpha"):
            got, ref = got[tokens], ref[tokens]
        assert_close(k, got, ref, tol_of(k, inp.io), case=f"{tag} T={inp.T} D={inp.D}")


def test_tiled_backward_alpha1_full_size_bf16():
    # B=1, S=4096, N=4, D=5120, bf16 I/O at alpha = 1: dx, dy, dH_* on sampled
    # tokens, the whole dphi, dbias and dalpha against the full fp64 oracle
    inp = make_inputs(4096, 4, 5120, io="bf16", seed=3, alpha=1.0, grads=True)
    check_backward(inp, tokens=_bwd_tokens(4096), tag="tiled bwd alpha=1")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("iters", [1, 3, 64])
@pytest.mark.parametrize("T,D", [(70, 256), (37, 2560)])
def test_tiled_backward_sinkhorn_rounds(io, iters, T, D):
    inp = make_inputs(T, 4, D, io=io, seed=iters * 7 + T, alpha=1.0, iters=iters, bias_std=3.0, grads=True)
    check_backward(inp, tag=f"tiled bwd rounds={iters}")
