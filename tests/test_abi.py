"""The C-ABI library loads and exports every symbol include/mhc.h declares, and
rejects bad arguments synchronously (host-only checks: nothing is launched)."""

import ctypes
import os
import re

import pytest

from residual_stream_amd import mhc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mhc.LIB_PATH):
        pytest.skip("libmhc.so not built (run __graft_entry__.build())")
    return mhc.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_surface():
    assert _declared_functions() == sorted(mhc.ABI_FUNCTIONS)


def _declared_arity():
    """Number of parameters of each declared function (``(void)`` counts 0)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, params in re.findall(r"\b(mhc_[a-z_0-9]+)\s*\(([^)]*)\)\s*;", text):
        p = params.strip()
        out[name] = 0 if p in ("", "void") else p.count(",") + 1
    return out


def test_binding_signatures_match_the_header(lib):
    # ctypes does not check a call against the C prototype; the argtypes the
    # binding sets must have the header's arity
    arity = _declared_arity()
    assert sorted(arity) == _declared_functions()
    for name, n in arity.items():
        assert len(getattr(lib, name).argtypes) == n, name


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+MHC_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert lib.mhc_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s in range(4):
        assert len(mhc.status_string(s)) > 0
    assert mhc.status_string(99) == "unknown status"


def test_workspace_sizes(lib):
    assert mhc.workspace_bytes("pre", 4096, 4, 5120, mhc.MHC_BF16) >= 0
    b = mhc.workspace_bytes("pre_bwd", 4096, 4, 5120, mhc.MHC_BF16)
    assert b > 4096 * 24 * 4
    assert mhc.workspace_bytes("pre_bwd", 0, 4, 5120, mhc.MHC_BF16) == 0   # empty batch


def _call_pre(lib, d, ptrs):
    return lib.mhc_pre(ctypes.byref(d), *ptrs[:7], None, 0, None)


# Fake device addresses: 16-byte aligned, never dereferenced because every
# call below fails a check before anything is launched.
FAKE = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(12)]


@pytest.mark.parametrize("field,value,expect", [
    ("T", 0, mhc.MHC_OK),  # an empty batch: nothing to compute, nothing launched
    ("T", -5, mhc.MHC_ERR_INVALID_ARG),
    ("N", 3, mhc.MHC_ERR_UNSUPPORTED),
    ("N", 16, mhc.MHC_ERR_UNSUPPORTED),
    ("D", 12, mhc.MHC_ERR_UNSUPPORTED),
    ("D", 0, mhc.MHC_ERR_UNSUPPORTED),
    ("io", 7, mhc.MHC_ERR_INVALID_ARG),
    ("sinkhorn_iters", 0, mhc.MHC_ERR_INVALID_ARG),
    ("eps", -1.0, mhc.MHC_ERR_INVALID_ARG),
    ("eps", float("nan"), mhc.MHC_ERR_INVALID_ARG),
    ("alpha_res", float("inf"), mhc.MHC_ERR_INVALID_ARG),
])
def test_bad_descriptor_rejected_without_launch(lib, field, value, expect):
    # (T = 0 is the one accepted case: the forward returns before launching)
    d = mhc.make_desc(64, 4, 256, mhc.MHC_F32)
    setattr(d, field, value)
    # a null x as well, so even a broken descriptor check cannot launch
    ptrs = [None] + FAKE[1:]
    st = _call_pre(lib, d, ptrs)
    assert st == expect


def test_null_and_misaligned_pointers_rejected(lib):
    d = mhc.make_desc(64, 4, 256, mhc.MHC_F32)
    for i in range(7):
        ptrs = list(FAKE)
        ptrs[i] = None
        assert _call_pre(lib, d, ptrs) == mhc.MHC_ERR_INVALID_ARG
        ptrs = list(FAKE)
        ptrs[i] = ctypes.c_void_p(FAKE[i].value + 4)
        assert _call_pre(lib, d, ptrs) == mhc.MHC_ERR_INVALID_ARG
    assert lib.mhc_post(ctypes.byref(d), None, *FAKE[:4], None) == mhc.MHC_ERR_INVALID_ARG
    assert lib.mhc_post_bwd(ctypes.byref(d), *FAKE[:8], None, None) == mhc.MHC_ERR_INVALID_ARG
    assert lib.mhc_pre_bwd(ctypes.byref(d), *FAKE[:6], None, *FAKE[:3], None, 0,
                           None) == mhc.MHC_ERR_INVALID_ARG


def test_aliasing_rejected(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake device addresses are only passed where no GPU exists")
    d = mhc.make_desc(64, 4, 256, mhc.MHC_F32)
    x = FAKE[0]
    # x_next == x, and x_next overlapping y
    assert lib.mhc_post(ctypes.byref(d), x, FAKE[1], FAKE[2], FAKE[3], x, None) == mhc.MHC_ERR_INVALID_ARG
    assert lib.mhc_post(ctypes.byref(d), x, FAKE[1], FAKE[2], FAKE[3],
                        ctypes.c_void_p(FAKE[1].value + 16), None) == mhc.MHC_ERR_INVALID_ARG
    # h overlapping x in mhc_pre
    assert lib.mhc_pre(ctypes.byref(d), x, FAKE[1], FAKE[2], ctypes.c_void_p(x.value + 64), FAKE[4],
                       FAKE[5], FAKE[6], None, 0, None) == mhc.MHC_ERR_INVALID_ARG


def test_backward_round_limit(lib):
    d = mhc.make_desc(64, 4, 256, mhc.MHC_F32, iters=65)
    assert lib.mhc_pre_bwd(ctypes.byref(d), None, *FAKE[:9], None, 0, None) == mhc.MHC_ERR_UNSUPPORTED
    assert mhc.workspace_bytes("pre_bwd", 64, 4, 256, mhc.MHC_F32, iters=65) > 0
