"""Compile the gfx950 HIP library ``libftmoe.so`` in-tree.

    python -m expert_cached_ffn_amd.build        # or __graft_entry__.build()

Every ``csrc/*.hip`` file is compiled with hipcc for gfx950 and every
``csrc/*.cpp`` file (host code: the CPU expert kernel) with the host compiler
for x86-64-v3 (AVX2 + FMA), one object per file, in parallel, and linked into
``expert_cached_ffn_amd/libftmoe.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libftmoe.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-result",
]


CXX = shutil.which("g++") or "g++"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CXXFLAGS = ["-O3", "-std=c++17", "-fPIC", "-march=x86-64-v3", "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__",
            "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [CXX, *CXXFLAGS, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources for {ARCH}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
