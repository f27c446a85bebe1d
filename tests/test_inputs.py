"""Host-side checks of the seeded input generator (no arithmetic of the method)."""

import numpy as np
import pytest
import torch

from residual_stream_amd.inputs import make_inputs, round_to_bf16, to_io


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf],
                                 dtype=np.float32)])
    ours = round_to_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(round_to_bf16(np.array([np.nan], dtype=np.float32)))[0]


def test_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: rounds to 1 (even).
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], dtype=np.float32)
    np.testing.assert_array_equal(round_to_bf16(v), np.array([1.0, 1 + 2 ** -6], dtype=np.float32))


def test_generator_is_reproducible_and_shaped():
    a = make_inputs(8, 4, 16, io="bf16", seed=3, grads=True)
    b = make_inputs(8, 4, 16, io="bf16", seed=3, grads=True)
    for f in ("x", "y", "phi", "bias", "dh", "dx_next"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.x.shape == (8, 4, 16) and a.y.shape == (8, 16)
    assert a.phi.shape == (64, 24) and a.bias.shape == (24,)
    assert np.array_equal(a.x, round_to_bf16(a.x))
    c = make_inputs(8, 4, 16, io="bf16", seed=4)
    assert not np.array_equal(a.x, c.x)


def test_generator_distribution():
    inp = make_inputs(64, 4, 256, seed=0)
    assert abs(inp.x.std() - 1) < 0.02
    assert abs(inp.phi.std() * np.sqrt(1024) - 1) < 0.03
    assert inp.alphas == (0.01, 0.01, 0.01) and inp.eps == 1e-6 and inp.iters == 20


def test_unknown_io_rejected():
    with pytest.raises(ValueError):
        to_io(np.zeros(2), "fp8")
