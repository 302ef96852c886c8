"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The C ABI's validation, sizing and launch marshalling (path_abi.cpp,
path_plan.cpp; the kernel launches stubbed out) and every entry point of the
fp64 oracle are built with g++/gcc -fsanitize=address,undefined and driven
through valid and invalid calls; any sanitizer report fails the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "attention_fwd_amd", "csrc")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def build_and_run(tmp_path, cmd, exe):
    r = subprocess.run(cmd + ["-o", str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=ENV)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"), reason="needs g++ and HIP headers")
def test_abi_validation_under_sanitizers(tmp_path):
    cmd = ["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                                          "-I", CSRC, os.path.join(CSRC, "path_abi.cpp"), os.path.join(CSRC, "path_plan.cpp"),
                                          os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "abi_driver.cpp")]
    assert "abi ok" in build_and_run(tmp_path, cmd, tmp_path / "abi_san")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    cmd = ["gcc", "-std=c99"] + SAN + ["-ffp-contract=off", os.path.join(ROOT, "oracle", "path_oracle.c"),
                                       os.path.join(HERE, "oracle_driver.c"), "-lm", "-lpthread"]
    assert "oracle ok" in build_and_run(tmp_path, cmd, tmp_path / "oracle_san")
