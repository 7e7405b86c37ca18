"""The work-item plan (host side): compile tests/plan_invariants.cpp against
the kernels' own header with g++ and run it. No GPU involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_paged_e5m2_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def test_plan_invariants(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = str(tmp_path / "plan_invariants")
    cmd = [gxx, "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", CSRC,
           "-o", exe, os.path.join(ROOT, "tests", "plan_invariants.cpp")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("OK"), run.stdout
