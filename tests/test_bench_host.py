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


def test_every_timed_call_names_its_kernels():
    b = _bench()
    ab = b.algo_bytes(64, 4, 256, "bf16")
    for table in (b.CALL_KERNELS, b.CALL_KERNELS_F32):
        assert set(table) == set(ab) - {"mhc_post_pre"}
        assert all(table[k] for k in table)
