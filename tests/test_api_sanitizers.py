"""The C-ABI validation layer (mx_grouped_gemm_amd/csrc/bsgemm_api.cpp) under host-side
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

tests/asan/api_validation.cpp calls every entry point with NULL, misaligned, out-of-range and
well-formed arguments and checks the documented status codes; the launchers are stubbed (without a
device nothing reaches them). hipcc builds the host code with the sanitizers (each -fsanitize=
after -Xarch_host, so no device code is instrumented) and links the HIP runtime, which reports no
device here, so a well-formed call must return BSG_ERR_DEVICE.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def test_validation_layer_under_asan_ubsan(tmp_path):
    exe = tmp_path / "api_validation"
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "mx_grouped_gemm_amd", "csrc"),
           os.path.join(ROOT, "mx_grouped_gemm_amd", "csrc", "bsgemm_api.cpp"),
           os.path.join(ROOT, "tests", "asan", "api_validation.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in (build.stderr or "").lower() and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "ok: 0 failure(s)" in run.stdout
