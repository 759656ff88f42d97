"""Build libssd.so (the HIP/gfx950 SSD library) in-tree with hipcc.

    python -m selective_state_space_71_amd.build

Each translation unit under csrc/ is compiled to an object in parallel, then
linked into ``selective_state_space_71_amd/libssd.so``.  Cross-compiles on a
host without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libssd.so")
SOURCES = ["ssd_api.hip", "ssd_fwd_bf16.hip", "ssd_fwd_f32.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the SSD library needs the ROCm toolchain")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops stay off: plain scalar fp32 only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-Wno-unused-result",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr[-6000:]}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every translation unit and link libssd.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr[-6000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"[ssd build] {LIB} ({time.time() - t0:.1f}s)", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
