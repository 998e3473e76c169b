"""GPU: the C ABI used from a plain C++ program (tests/cabi/step_driver.cpp,
built by __graft_entry__.build()): hipMalloc'd buffers and an explicit HIP
stream, no Python or torch in the process.  The program checks the step
against closed forms (exact norm, the first Adam step from zero moments, the
RNE parameter copy), the skip on an inf, the device-state step bit for bit,
and the host-side rejection of a misaligned pointer."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "cabi", "step_driver")

pytestmark = pytest.mark.gpu


def test_c_client_runs_a_step():
    assert os.path.exists(EXE), "tests/cabi/step_driver is not built: run __graft_entry__.build()"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout[-2000:], r.stderr[-2000:])
