"""The host half of the library (plan, fragments, loss scaler, host step and
its worker pool, error paths) built with AddressSanitizer +
UndefinedBehaviorSanitizer and, separately, with ThreadSanitizer, and run by
a driver that checks results (tests/sanitize/host_driver.cpp).  Host code
only: the device kernels are not part of these builds."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CXX = os.environ.get("HOST_CXX", "/opt/rocm/bin/amdclang++")
CSRC = os.path.join(ROOT, "zero_sharded_mixed_partition_amd", "csrc")
SOURCES = [os.path.join(CSRC, "host.cpp"), os.path.join(CSRC, "cpu_step.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")]


@pytest.mark.parametrize("flags", [["-fsanitize=address,undefined", "-fno-sanitize-recover=all"],
                                   ["-fsanitize=thread"]], ids=["asan-ubsan", "tsan"])
def test_host_library_under_sanitizer(tmp_path, flags):
    if not (os.path.exists(CXX) or shutil.which(CXX)):
        pytest.skip("host compiler not available")
    exe = str(tmp_path / "driver")
    cmd = [CXX, "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-math-errno", "-pthread",
           *flags, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", *SOURCES, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
