"""Host AddressSanitizer and UndefinedBehaviorSanitizer runs (CPU only).

Two host programs are built with gcc / g++ and -fsanitize=address,undefined
(-fno-sanitize-recover, so any report fails the run) and executed:
  * oracle.c driven on small problems (both masks, several scales, ragged
    sizes, a single token, row and head subsets) and on invalid arguments
    (tests/sanitize/oracle_driver.c);
  * the C ABI's host argument checks (csrc/fa2_api.cpp) and kernel choice
    (csrc/fa2_dispatch.cpp), with the kernel launchers replaced by stubs
    that abort, on shapes up to and past every limit the checks enforce
    (tests/sanitize/api_driver.cpp).
The GPU code is not part of these builds: hipcc's device compilation cannot
be sanitized here.
"""
import os
import shutil
import subprocess

import pytest

from exact_tiled_attention_30_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall"]


def _run(exe, tmp_path):
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, cwd=tmp_path, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", *SAN, "-fopenmp", os.path.join(ROOT, "oracle", "oracle.c"),
                    os.path.join(HERE, "oracle_driver.c"), "-o", exe, "-lm"], check=True)
    assert "oracle sanitizer run: ok" in _run(exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_api_checks_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "api_driver")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(rocm, "include"), "-I", build.INCLUDE, "-I", build.CSRC,
                    os.path.join(build.CSRC, "fa2_api.cpp"),
                    os.path.join(build.CSRC, "fa2_dispatch.cpp"),
                    os.path.join(HERE, "api_driver.cpp"), "-o", exe], check=True)
    assert "api sanitizer run: ok" in _run(exe, tmp_path)
