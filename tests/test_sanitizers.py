"""AddressSanitizer + UndefinedBehaviorSanitizer runs on the CPU (no GPU).

* The host side of libkda (kda_api.cpp: validation, segment and workspace
  planning, the document-order decision) is built with g++ against stand-ins
  for the HIP runtime and the kernel launchers (tests/sanitize/hip_stubs.cpp)
  and driven through every entry point by tests/sanitize/abi_host_paths.cpp.
* The C oracle is built with the same sanitizers and the oracle pins run on
  it (``KDA_ORACLE_LIB`` points the oracle package at that build; the
  sanitizer runtime is preloaded into the Python process).
Any sanitizer report aborts the child process and fails the test.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")

needs_gcc = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                               reason="gcc/g++ not available")


@needs_gcc
def test_host_paths_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_host_paths"
    subprocess.run(["g++", "-std=c++17", "-O1", *SAN, "-D__HIP_PLATFORM_AMD__",
                    "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "linear_attention_fwd_amd", "csrc", "kda_api.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "hip_stubs.cpp"),
                    os.path.join(ROOT, "tests", "sanitize", "abi_host_paths.cpp"),
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


@needs_gcc
def test_oracle_pins_under_sanitizers(tmp_path):
    lib = tmp_path / "libkda_oracle_san.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *SAN,
                    os.path.join(ROOT, "oracle", "kda_oracle.c"), "-o", str(lib), "-lm"],
                   check=True, capture_output=True, text=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()
    env = dict(ENV, KDA_ORACLE_LIB=str(lib), LD_PRELOAD=asan, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout
    # the pins ran on the sanitizer build, with the sanitizer runtime loaded
    probe = ("import os, oracle; oracle._load(); m = open(f'/proc/{os.getpid()}/maps').read(); "
             "print(('libkda_oracle_san.so' in m) and ('libasan' in m))")
    r = subprocess.run([sys.executable, "-c", probe], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=120)
    assert r.stdout.strip() == "True", r.stdout + r.stderr
