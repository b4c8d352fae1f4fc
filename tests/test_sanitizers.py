"""The host code under the address and undefined-behaviour sanitizers (CPU
only): the oracle, and abi.cpp's validation, tree-walk planning and launch
configuration with the kernel launchers replaced by host stubs that check
each launch plan against what the kernels assume."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_deltanet_recurrence_gdn_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", *SAN, "-ffp-contract=off", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lpthread", "-lm"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "oracle driver ok" in r.stdout and "runtime error" not in r.stderr


def test_host_abi_under_sanitizers(tmp_path):
    _need("g++")
    if not os.path.isdir("/opt/rocm/include"):
        pytest.skip("HIP headers not available")
    exe = str(tmp_path / "abi_driver")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    _run(["g++", "-std=c++17", *SAN, *inc, "-o", exe, os.path.join(CSRC, "abi.cpp"),
          os.path.join(HERE, "abi_stubs.cpp"), os.path.join(HERE, "abi_driver.cpp")])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert "launch-check failures 0, expectation failures 0" in r.stdout and "runtime error" not in r.stderr
