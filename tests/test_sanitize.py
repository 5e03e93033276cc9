"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

build.py's sanitizer build instruments the host side of every source (argument
validation of the C ABI, the cache's host bookkeeping, the CPU expert kernel
and its thread pool); this test runs the host-side test files against that
build in a child interpreter that preloads clang's ASan runtime.  Any report
aborts the child (halt_on_error), so the test fails on the first finding.
"""
import glob
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

HOST_TESTS = ["tests/test_abi.py", "tests/test_cpu_expert.py"]


def _sanitized_lib():
    from expert_cached_ffn_amd import build
    srcs = build.sources() + glob.glob(os.path.join(build.CSRC, "*.hpp")) + \
        [os.path.join(ROOT, "include", "ft_moe.h"), os.path.abspath(build.__file__)]
    fresh = os.path.exists(build.SAN_LIB) and \
        os.path.getmtime(build.SAN_LIB) >= max(os.path.getmtime(s) for s in srcs)
    if not fresh:
        build.build(verbose=False, sanitize=True)
    return build.SAN_LIB, build.sanitizer_runtime()


@pytest.mark.timeout(900)
def test_host_code_under_asan_and_ubsan():
    try:
        lib, runtime = _sanitized_lib()
    except RuntimeError as e:
        pytest.fail(f"sanitizer build failed: {e}")
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms, "the sanitizer build is not instrumented"
    env = dict(os.environ, FTMOE_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", *HOST_TESTS, "-q", "-m", "not gpu", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, f"host tests under ASan/UBSan failed:\n{tail}"
    assert " passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
