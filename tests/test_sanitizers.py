"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU, no GPU):
the oracle driven through every function and format, and the C ABI's host
layer (argument checks, workspace layout, launch-argument packing) built with
stub launchers and driven through every entry point.  Any sanitizer report
aborts the program (-fno-sanitize-recover=all), failing the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc missing")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, "-o", exe,
          os.path.join(ROOT, "oracle", "vqkv_oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
          "-lm"], str(tmp_path))
    out = _run([exe], str(tmp_path))
    assert "oracle driver ok" in out


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the ROCm headers missing")
def test_c_abi_host_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_san")
    _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN, "-o", exe,
          os.path.join(ROOT, "vector_quantized_bit_vqkv_amd", "csrc", "capi.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp")], str(tmp_path))
    out = _run([exe], str(tmp_path))
    assert "abi driver ok" in out
