"""Compile the gfx950 HIP library ``libftmoe.so`` in-tree.

    python -m expert_cached_ffn_amd.build              # or __graft_entry__.build()
    python -m expert_cached_ffn_amd.build --sanitize   # host code under ASan + UBSan

Every ``csrc/*.hip`` file is compiled with hipcc for gfx950 and every
``csrc/*.cpp`` file (host code: the CPU expert kernel) with the host compiler
for x86-64-v3 (AVX2 + FMA), one object per file, in parallel, and linked into
``expert_cached_ffn_amd/libftmoe.so``.

``--sanitize`` builds a second copy, ``_build/sanitize/libftmoe.so``, whose
host code (the C ABI's validation, the cache's bookkeeping, the CPU expert
kernel and its thread pool) is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer; device code is compiled as usual.  The .cpp files
are then compiled by the ROCm clang so one sanitizer runtime serves the whole
library.  It is loaded only when FTMOE_LIB names it, in a process that
preloads clang's ASan runtime (``sanitizer_runtime()``).
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


SAN_BUILD = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libftmoe.so")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
# host-side sanitizers only: -Xarch_host in front of each flag keeps device code uninstrumented
SAN_HOST = ["address", "undefined"]
SAN_HIP = [f for san in SAN_HOST for f in ("-Xarch_host", f"-fsanitize={san}")] + \
    ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_CXX = ["-fsanitize=" + ",".join(SAN_HOST), "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the ROCm clang ASan runtime (to LD_PRELOAD into an uninstrumented interpreter)."""
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("clang ASan runtime not found under ROCm's llvm")
    return found[-1]


def _compile(src: str, sanitize: bool = False) -> str:
    out_dir = SAN_BUILD if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    if src.endswith(".cpp"):
        cmd = [CLANGXX, *CXXFLAGS, *SAN_CXX, "-c", src, "-o", obj] if sanitize else \
            [CXX, *CXXFLAGS, "-c", src, "-o", obj]
    else:
        cmd = [HIPCC, *CFLAGS, *(SAN_HIP if sanitize else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile every HIP source and link the library; returns its path."""
    out_dir, lib = (SAN_BUILD, SAN_LIB) if sanitize else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = lib + ".tmp"
    # a shared library leaves the sanitizer runtime's symbols to the process that loads it
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources for {ARCH}" + (" (host ASan + UBSan)" if sanitize else ""))
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
