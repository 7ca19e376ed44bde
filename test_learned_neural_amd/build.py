"""Build libtitans_mem.so in-tree with hipcc for gfx950.

Every call recompiles (the "does it build" check).  Objects go to _build/;
the shared library lands next to this file, where the binding loads it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libtitans_mem.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["tm_host.cpp", "tm_generic.hip", "tm_linear.hip", "tm_mlp2_group.hip", "tm_input.hip", "tm_backward.hip",
           "tm_retrieve.hip", "tm_deep.hip"]

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-I" + CSRC]
# no packed fp32 instructions in device code (v_pk_* fp32 forms)
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


# MFMA results in VGPRs: the MFMA kernel post-processes every accumulator on
# the VALU and keeps the memory state in VGPRs
PER_FILE = {"tm_mlp2_group.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra=(), build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [hipcc()] + COMMON + list(extra)
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE + PER_FILE.get(src, [])
    cmd += ["-c", path, "-o", obj]
    subprocess.check_call(cmd)
    return obj


def build(verbose: bool = False, extra=(), out: str = OUT, build_dir: str = BUILD_DIR) -> str:
    """Compile every source and link the library at ``out`` (``extra``:
    additional compiler flags, e.g. -DTM_STAGE_STAMPS=1 for the stage-timing
    build, which stage_stamps.py places beside the library)."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
