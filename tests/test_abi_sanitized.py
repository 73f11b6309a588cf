"""The C ABI layer's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only): moe_api.cpp is compiled with both
sanitizers on its host pass (device code unchanged), linked with the
library's kernel objects and a C program (tests/abi_host_checks.c) that
calls every entry point with the invalid arguments a C caller can pass,
including enum values outside their enumerators, and checks the status
codes.  No call reaches the HIP runtime, so no GPU is needed."""
import glob
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "top_routing_grouped_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNEL_OBJS = ["moe_gemm.hip", "moe_gemm_tiled.hip", "moe_route.hip", "moe_permute.hip", "moe_down_combine.hip",
               "moe_norm.hip", "moe_stream.hip"]


def _kernel_objects():
    objs = [os.path.join(PKG, "_build", f + ".o") for f in KERNEL_OBJS]
    if not all(os.path.exists(o) for o in objs):
        from top_routing_grouped_amd.build import build
        build()
    return objs


@pytest.mark.skipif(not (os.path.exists(HIPCC) and shutil.which("gcc")), reason="needs hipcc and gcc")
def test_host_checks_under_address_and_undefined_sanitizers():
    objs = _kernel_objects()
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    with tempfile.TemporaryDirectory() as d:
        api = os.path.join(d, "api.o")
        subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", *inc, "-x", "hip", "--offload-arch=gfx950",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                        "-Xarch_host", "-fno-sanitize-recover=all",
                        "-c", os.path.join(PKG, "csrc", "moe_api.cpp"), "-o", api],
                       check=True, capture_output=True, text=True)
        drv = os.path.join(d, "drv.o")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Werror", *inc,
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-c", os.path.join(ROOT, "tests", "abi_host_checks.c"), "-o", drv],
                       check=True, capture_output=True, text=True)
        exe = os.path.join(d, "checks")
        subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", drv, api, *objs, "-o", exe],
                       check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "ok: 0 failed" in r.stdout
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
