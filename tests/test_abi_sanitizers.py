"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Every library source is compiled with the sanitizers on its host side only
(each -fsanitize= behind -Xarch_host: the device code is built as usual and
never runs here) and linked with tests/asan/abi_harness.cpp, which drives
every entry point's argument validation, the size, layout and plan queries
and the host Z-order. It runs on this GPU-less host: each call it makes
returns before any HIP call. A sanitizer report or a wrong status fails it.
"""

import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from block_sparse_taylor_amd import build as B

HARNESS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "asan", "abi_harness.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-fno-omit-frame-pointer"]


@pytest.mark.timeout(900)
def test_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *SAN,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", B.INCLUDE, "-I", B.CSRC]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src).split(".")[0] + "_san.o"))
        r = subprocess.run([hipcc, *flags, "-x", "hip", "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr
        return obj

    srcs = B.sources() + [HARNESS]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_harness")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
    assert "all expectations met" in run.stdout, out
