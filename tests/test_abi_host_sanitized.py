"""The C-ABI layer on the host under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/abi_host_check.cpp is compiled with g++
together with csrc/xqa_api.cpp, with host fakes for the HIP runtime calls and
the kernel launchers, and run. It checks argument validation (rejected calls
launch nothing), handle sizing and the arguments each entry point hands to
the kernels. No GPU involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "decode_attention_paged_e5m2_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


def test_abi_layer_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("g++ or the ROCm headers are not available")
    exe = str(tmp_path / "abi_host_check")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-o", exe,
           os.path.join(ROOT, "tests", "abi_host_check.cpp"), os.path.join(CSRC, "xqa_api.cpp")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0 and "sanitize" in res.stderr and "cannot find" in res.stderr:
        pytest.skip("sanitizer runtimes are not installed")
    assert res.returncode == 0, res.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("OK"), run.stdout
