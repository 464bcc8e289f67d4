"""The C ABI's host-side validation built with AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no GPU): a driver walks every
entry point through its rejection paths and its workspace-size queries,
with the kernel launchers replaced by counting stubs, and exits non-zero on
any unexpected status, any launch from a rejected call, or any sanitizer
report (unsloth-zoo issue #850, Suggested fix: failures are loud)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_weight_quantization_moeq_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "asan")


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_validation_under_host_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    exe = str(tmp_path / "driver")
    cmd = [hipcc, "--offload-arch=gfx950", "-x", "hip",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-g", "-O1", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "api.hip"), os.path.join(HERE, "launch_stubs.hip"),
           os.path.join(HERE, "validation_driver.hip"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all checks passed" in r.stdout
