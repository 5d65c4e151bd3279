"""Build libforkattn.so (HIP, gfx950) in-tree.

Every source in csrc/ is compiled with hipcc for gfx950 only, with packed-FP32
instruction selection disabled (``-packed-fp32-ops``) and MFMA accumulators
kept in architectural VGPRs (``-amdgpu-mfma-vgpr-form``: the scan kernels read
their accumulators with VALU every chunk, and accumulators held in AGPRs would
cost a copy each way), then linked into ``libforkattn.so`` next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libforkattn.so")
SOURCES = ["capi.cpp", "meta.hip", "attn.hip", "gdn.hip", "block.hip", "mixer.hip", "linear.cpp", "graph.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ["-lhipblaslt"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
