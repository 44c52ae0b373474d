"""The host side of the library (argument checks, split plan, workspace
sizing, every C-ABI entry point) and the float64 oracle, built for the CPU
with AddressSanitizer and UndefinedBehaviorSanitizer and driven through valid
and invalid arguments. Kernel launches are replaced by host stand-ins that
check the launch arguments; no GPU code is built or run."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "relative_position_bias_amd", "csrc")
SAN = os.path.join(HERE, "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout + res.stderr
    return res


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_host_code_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "host_driver")
        _run(["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN_FLAGS, "-I", os.path.join(ROOT, "include"),
              "-I", CSRC, "-I", os.path.join(ROCM, "include"), os.path.join(CSRC, "rba_host.cpp"),
              os.path.join(SAN, "launch_stub.cpp"), os.path.join(SAN, "host_driver.cpp"), "-o", exe,
              "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
              "-pthread"])
        res = _run([exe], env=ENV, timeout=300)
        assert "all expectations held" in res.stdout
        assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        _run(["gcc", "-std=c11", "-fopenmp", *SAN_FLAGS, os.path.join(ROOT, "oracle", "oracle.c"),
              os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lm"])
        res = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"), timeout=300)
        assert "all calls behaved" in res.stdout
        assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr
