"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU oracle
and of the C ABI's host-side argument validation (CPU only; no GPU code is
built with a sanitizer).  Each driver runs every entry point on small,
ragged and degenerate inputs; any sanitizer report fails the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def run_driver(cmd, exe):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-4000:]
    assert "AddressSanitizer" not in report and "runtime error" not in report, report[-4000:]
    return report


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not available")
def test_oracle_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_driver")
        cmd = ["gcc", "-std=c99", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", *SAN,
               "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "oracle.c"),
               os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"]
        assert "ok" in run_driver(cmd, exe)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers are not available")
def test_abi_validation_under_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "abi_driver")
        csrc = os.path.join(ROOT, "weight_only_mixed_amd", "csrc")
        cmd = ["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", *SAN,
               os.path.join(csrc, "slq_abi.cpp"), os.path.join(ROOT, "tests", "sanitize", "abi_stubs.cpp"),
               os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-o", exe]
        assert "0 failing checks" in run_driver(cmd, exe)
