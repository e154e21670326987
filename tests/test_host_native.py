"""Host-side native checks of library helpers (compiled with hipcc, run on
the CPU; no GPU and no HIP runtime calls)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_fastdiv_matches_integer_division(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "fastdiv_check"
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O2", "-std=c++17",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "convolution_nhwc_implicit_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "fastdiv_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
