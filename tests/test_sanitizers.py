"""Host builds under AddressSanitizer and UndefinedBehaviorSanitizer (gcc/g++, no GPU):
the C oracle on small inputs of every entry point, and the library's argument
validation and split planning with stub kernel launchers."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, exe, tmp_path, expect):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    # verify_asan_link_order=0: a library the environment preloads may come before the
    # sanitizer runtime in the process's list
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and expect in r.stdout, r.stdout + r.stderr


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_sanitize")
    _run([gcc, "-std=c11", *SAN, "-fopenmp", os.path.join(ROOT, "tests", "sanitize", "oracle_sanitize.c"), "-o", exe,
          "-lm"], exe, tmp_path, "oracle_sanitize: ok")


def test_api_host_side_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("no g++ or HIP headers")
    exe = str(tmp_path / "api_host_sanitize")
    _run([gxx, "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
          os.path.join(ROOT, "tests", "sanitize", "api_host_sanitize.cpp"), "-o", exe], exe, tmp_path,
         "api_host_sanitize: ok")
