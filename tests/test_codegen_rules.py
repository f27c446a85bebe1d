"""Rules on the gfx950 code the library's kernels compile to, checked on the
device assembly (hipcc -S, no GPU needed):

* no packed-fp32 VALU instruction (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32):
  every kernel is built with the packed-fp32 feature switched off;
* no buffer store wider than 8 bytes with a register scalar offset: the
  compiler then omits the wait state that keeps the next VALU write from
  changing the store's data registers before they are read, and some lanes
  store a corrupted first word.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from residual_stream_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIP_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


def _asm(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, os.path.splitext(src)[0] + ".s")
    cmd = [build.hipcc(), *build.COMMON, *build.DEVICE_FLAGS, f"-I{build.INCLUDE}", "--cuda-device-only",
           "-S", os.path.join(build.CSRC, src), "-o", out]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert p.returncode == 0, p.stdout[-2000:]
    return out


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    d = str(tmp_path_factory.mktemp("asm"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(HIP_SOURCES))) as ex:
        paths = list(ex.map(lambda s: _asm(s, d), HIP_SOURCES))
    return {os.path.basename(p): open(p).read() for p in paths}


def test_every_kernel_source_compiled(assembly):
    assert len(assembly) == len(HIP_SOURCES)


def test_no_packed_fp32_instructions(assembly):
    for name, text in assembly.items():
        hits = re.findall(r"^\s*(v_pk_(?:add|mul|fma)_f32)\b", text, flags=re.M)
        assert not hits, f"{name}: {sorted(set(hits))}"


def test_wide_buffer_stores_use_a_literal_scalar_offset(assembly):
    pat = re.compile(r"^\s*buffer_store_dword(?:x3|x4)\s+(.*)$", re.M)
    for name, text in assembly.items():
        for m in pat.finditer(text):
            ops = [o.strip() for o in re.split(r",\s*(?![^\[]*\])", m.group(1))]
            soffset = ops[3].split()[0]
            assert soffset == "0", f"{name}: {m.group(0).strip()}"
