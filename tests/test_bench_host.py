"""Host-side checks of bench.py: the one-GPU rule, and the algorithmic byte
counts the roofline divides by (every tensor read or written once)."""

from __future__ import annotations

import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_pro_shape():
    b = _bench()
    T, N, D = 4096, 4, 5120
    e, K, C = 2, N * D, N * N + 2 * N
    ab = b.algo_bytes(T, N, D, "bf16")
    phi = K * C * 4 + C * 4
    coef = (N + N * N) * 4
    # hc_pre: x in, h out, H_pre/H_post/H_res out; φ and b once
    assert ab["mhc_pre"] == T * (K * e + D * e + C * 4) + phi
    # hc_post: x, y, H in; x_next out
    assert ab["mhc_post"] == T * (2 * K * e + D * e + coef)
    # hc_post backward: dx_next, x, y, H in; dx, dy, dH out (without dx: one K·e less each way)
    assert ab["mhc_post_bwd"] == T * (3 * K * e + 2 * D * e + 2 * coef)
    assert ab["mhc_post_bwd"] - ab["mhc_post_bwd_nodx"] == T * K * e
    # hc_pre backward: dh, x, dx (or dx_next) in, dx out, dH in; φ read and dφ written once;
    # the mixing call also reads H_res
    assert ab["mhc_pre_bwd"] == T * (D * e + 3 * K * e + coef) + 2 * phi
    assert ab["mhc_pre_bwd_mix"] - ab["mhc_pre_bwd"] == T * N * N * 4
    # the step with the mixing backward moves one state-sized tensor less than with two calls
    two = ab["mhc_pre"] + ab["mhc_post"] + ab["mhc_post_bwd"] + ab["mhc_pre_bwd"]
    mix = ab["mhc_pre"] + ab["mhc_post"] + ab["mhc_post_bwd_nodx"] + ab["mhc_pre_bwd_mix"]
    assert two - mix == T * K * e - T * N * N * 4


def test_kernel_names_as_the_library_reports_them():
    b = _bench()
    assert b.short_name("(tile::hc_pre_tile_kernel<8, 4, 4, 4>)") == "hc_pre_tile_kernel<8, 4, 4, 4>"
    assert b.short_name("tile::phi_pack_tile_kernel") == "phi_pack_tile_kernel"
    assert b.short_name("(hc_post_bwd_generic<N, IO, true>)") == "hc_post_bwd_generic<N, IO, true>"
    assert b.short_name("bwd_dx_kernel<true>") == "bwd_dx_kernel<true>"


def test_kernel_bytes_add_up_to_the_calls():
    # the kernels of each call together move the call's algorithmic bytes
    # (φ packing reads φ and writes its copy; the backward's φ read is
    # counted in the projection and in the dx pass, its dφ in the final sum)
    b = _bench()
    T, N, D = 4096, 4, 5120
    K, C = N * D, N * N + 2 * N
    phi = K * C * 4
    for io in ("bf16", "f32"):
        ab = b.algo_bytes(T, N, D, io)
        kb = lambda n: b.kernel_bytes(n, T, N, D, io)  # noqa: E731
        assert kb("hc_pre_tile_kernel<8, 4, 4, 4>") == ab["mhc_pre"]
        assert kb("hc_pre_mfma_kernel<IO, TM>") == ab["mhc_pre"]
        assert kb("hc_post_generic<N, IO>") == ab["mhc_post"]
        assert kb("hc_post_bwd_generic<N, IO, true>") == ab["mhc_post_bwd"]
        assert kb("hc_post_bwd_generic<N, IO, false>") == ab["mhc_post_bwd_nodx"]
        e = 2 if io == "bf16" else 4
        # dx pass, coefficient pass and dφ sum: x, dh, dx, dH, φ and bias in; dx, dφ and dbias out
        dx_part = kb("bwd_dx_kernel<false>") + kb("dphi_bias_sum_kernel") + kb("bwd_coef_kernel")
        assert dx_part == ab["mhc_pre_bwd"]
        assert kb("bwd_dx_kernel<true>") - kb("bwd_dx_kernel<false>") == T * N * N * 4
        assert kb("bwd_proj_kernel<10>") == T * (K * e + D * e) + phi
        assert kb("phi_pack_tile_kernel") == 2 * phi
        assert kb("no_such_kernel") is None
