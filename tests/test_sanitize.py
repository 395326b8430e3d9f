"""Host sanitizer builds (CPU only): the C ABI's argument validation
(fp8_scaled_quantization_scale_amd/csrc/api.cpp, with the kernel launchers
replaced by recording stubs) and the C oracle (oracle/oracle.c), each built
with AddressSanitizer and UndefinedBehaviorSanitizer and driven over edge
inputs by the programs in tests/sanitize/.  Any report aborts the program
(-fno-sanitize-recover=all), so a zero exit means none was raised."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _build_and_run(cmd, exe):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_abi_validation_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "fp8_scaled_quantization_scale_amd", "csrc")
    cmd = (["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                                           "-I" + os.path.join(ROOT, "include"), "-I" + csrc,
                                           os.path.join(csrc, "api.cpp"), os.path.join(HERE, "abi_driver.cpp"),
                                           "-o", exe])
    assert "abi validation ok" in _build_and_run(cmd, exe)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = (["gcc", "-std=c99", "-fno-fast-math", "-ffp-contract=off"] + SAN +
           [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm", "-o", exe])
    assert "oracle ok" in _build_and_run(cmd, exe)
