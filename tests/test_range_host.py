"""Host check of the per-row key-range arithmetic shared by the forward
kernels (csrc/mfa_internal.h, row_key_range) under hostile sequence bounds:
tests/range_check.cpp is compiled for the host with hipcc and run.  No GPU
is involved; the kernels call the same inline function."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not found")
def test_row_key_range_stays_in_bounds_for_hostile_sequence_bounds(tmp_path):
    exe = str(tmp_path / "range_check")
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--cuda-host-only", "-x", "hip", "-std=c++17",
           "-I", os.path.join(ROOT, "transformer_mfa_fwd_amd", "csrc"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "range_check.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
