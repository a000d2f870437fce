"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

tests/sanitize/api_fuzz.cpp drives kda_api.cpp's argument handling (workspace sizing,
validation, plan, the launch sequence up to stubbed launches) through 20,000 seeded
argument sets, half of them well formed and half with null, misaligned or overlapping
pointers, extreme sizes and unknown dtypes or flags. The sanitizers are enabled for the
host pass only (no GPU code is instrumented and no GPU is touched); any report fails the
run. This is where signed overflow in the chunk-count arithmetic for extreme T was found
and bounded.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_api_argument_handling_is_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_fuzz")
    host_only = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *host_only,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "chunkwise_delta_rule_kda_amd", "csrc"),
           os.path.join(ROOT, "chunkwise_delta_rule_kda_amd", "csrc", "kda_api.cpp"),
           "-x", "hip", os.path.join(ROOT, "tests", "sanitize", "api_fuzz.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe, "20000"], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert "accepted" in out
