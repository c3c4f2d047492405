"""The C-ABI host layer under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

csrc/api.hip (argument checks, workspace arithmetic, status and error text) is
compiled with the sanitizers on its host code only (device code is never
instrumented), linked with the library's other objects and driven by
tests/abi_sanitize_driver.c, which calls every declared entry point with
arguments that must be refused, sizes at the edges of what is accepted, and
empty batches.  No call reaches a kernel launch.  Any sanitizer report aborts
the driver, and the test fails with its output.
"""
import os
import subprocess
import tempfile

import pytest

from compressed_sparse_attention_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fsanitize=integer",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _objects():
    objs = [os.path.join(B.BUILD, os.path.splitext(s)[0] + ".o") for s in B.SOURCES if s != "api.hip"]
    if not all(os.path.exists(o) for o in objs):
        B.build()
    return objs


def test_abi_host_layer_is_sanitizer_clean():
    hipcc = B.hipcc()
    objs = _objects()
    with tempfile.TemporaryDirectory() as d:
        api_o, drv_o, exe = (os.path.join(d, n) for n in ("api_san.o", "driver.o", "driver"))
        for cmd in (
            [hipcc, "--offload-arch=" + B.ARCH, "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
             "-Xclang", "-packed-fp32-ops", *SAN, "-c", os.path.join(B.CSRC, "api.hip"), "-o", api_o],
            ["gcc", "-O1", "-g", "-Wall", "-Werror", "-c", os.path.join(HERE, "abi_sanitize_driver.c"), "-o", drv_o],
            [hipcc, "--offload-arch=" + B.ARCH, *SAN[:6], drv_o, api_o, *objs, "-o", exe],
        ):
            p = subprocess.run(cmd, capture_output=True, text=True)
            assert p.returncode == 0, " ".join(cmd) + "\n" + p.stdout + p.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
        p = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        out = p.stdout + p.stderr
        assert p.returncode == 0 and "ABI_DRIVER_OK" in p.stdout, out[-4000:]
        assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
