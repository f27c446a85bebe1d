"""Builds libmhc.so (the gfx950 kernels behind include/mhc.h) in-tree with hipcc.

Usage: ``python -m residual_stream_amd.build`` (or ``__graft_entry__.build()``).
Cross-compiles for gfx950 on a machine without a GPU.  Always rebuilds.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmhc.so")
ABI_RUN_SRC = os.path.join(os.path.dirname(HERE), "tests", "c", "mhc_abi_run.cpp")
ABI_RUN = os.path.join(os.path.dirname(HERE), "tests", "c", "_build", "mhc_abi_run")

SOURCES = ["mhc_api.cpp", "hc_pre.hip", "hc_pre_mfma.hip", "hc_post.hip", "hc_bwd.hip",
           "hc_pre_bwd_mfma.hip", "hc_pre_decode.hip",
           "hc_post_stable.hip", "hc_pre_tile.hip", "mhc_noalloc.hip"]

ARCH = "gfx950"
# Packed-fp32 VALU instructions are switched off for every device pass.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Wno-unknown-pragmas"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the mHC library needs ROCm's hipcc to build")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature flag and says so; drop that line.
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmds.append([cc, *COMMON, *DEVICE_FLAGS, f"-I{INCLUDE}", *lang, "-c", os.path.join(CSRC, src),
                     "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    # the host-only program that drives the C ABI without Python (a GPU test runs it)
    os.makedirs(os.path.dirname(ABI_RUN), exist_ok=True)
    _run([cc, "-O2", "-std=c++17", f"-I{INCLUDE}", ABI_RUN_SRC, f"-L{HERE}", "-lmhc",
          "-Wl,-rpath,$ORIGIN/../../../residual_stream_amd", "-o", ABI_RUN])
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
