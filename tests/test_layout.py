"""The chunked HGRN2 kernel addresses its LDS tiles through factored forms of three XOR-swizzled
layouts (selective_state_space_diag_amd/csrc/h2_layout.hpp).  This compiles a host program that
checks every factored form against the direct layout function for all lane and loop indices, and
runs it on the CPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")
def test_h2_layout_factored_forms_match(tmp_path):
    exe = tmp_path / "h2_layout_check"
    src = os.path.join(ROOT, "tests", "native", "h2_layout_check.hip")
    inc = os.path.join(ROOT, "selective_state_space_diag_amd", "csrc")
    r = subprocess.run([_hipcc(), "-O1", "-I", inc, src, "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout
