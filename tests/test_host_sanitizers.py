"""The host code built with AddressSanitizer and UndefinedBehaviorSanitizer
and run as executables of their own: the fp64 oracle (C) and the prefill tile
scheduler (schedule.h) through the oracle pins and scheduler checks of
tests/sanitize/san_main.cpp; the C ABI (api.cpp: argument validation, size
arithmetic, host hooks) against recording stand-ins of the kernel launchers
through tests/sanitize/san_api.cpp.  CPU only; the compilers are gcc and g++
(no GPU code is built here)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc and g++")
def test_oracle_and_scheduler_under_sanitizers(tmp_path):
    obj = str(tmp_path / "swa_oracle.o")
    exe = str(tmp_path / "san_main")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-Wno-unknown-pragmas"] + FLAGS +
                   ["-c", os.path.join(ROOT, "oracle", "swa_oracle.c"), "-o", obj], check=True)
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror"] + FLAGS +
                   ["-I", os.path.join(SAN, "shim"), "-I", os.path.join(ROOT, "block_sparse_causal_band_amd", "csrc"),
                    os.path.join(SAN, "san_main.cpp"), obj, "-o", exe, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized host checks: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_c_abi_under_sanitizers(tmp_path):
    exe = str(tmp_path / "san_api")
    csrc = os.path.join(ROOT, "block_sparse_causal_band_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-Wno-unused-parameter"] + FLAGS +
                   ["-I", os.path.join(SAN, "shim"), "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(csrc, "api.cpp"), os.path.join(SAN, "api_stubs.cpp"), os.path.join(SAN, "san_api.cpp"),
                    "-o", exe, "-lm"], check=True)
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized C ABI checks: ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
