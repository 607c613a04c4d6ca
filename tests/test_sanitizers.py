"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, built with gcc/g++: no device code is involved):

* the oracle built with both sanitizers, and its CPU tests run against that
  build in a child process (the runtime preloaded, leak checks off: the
  Python interpreter is not built for them);
* the C ABI's argument handling (attn_api.cpp) linked with stub launchers
  and fuzzed with random shapes, flags, strides and pointers (ROCm's clang++
  in plain C++ host mode: the internal header uses clang's vector types).
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def _runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def test_oracle_under_sanitizers(tmp_path):
    asan = _runtime()
    lib = tmp_path / "liboracle_san.so"
    cmd = ["gcc", "-O1", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", *SAN, os.path.join(ROOT, "oracle", "oracle.c"), "-o", str(lib), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, LD_PRELOAD=asan, ORACLE_LIB=str(lib),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_bf16.py", "test_oracle_attention.py",
                                                      "test_oracle_schedules.py", "test_oracle_fp8.py",
                                                      "test_oracle_models.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu and not slow", "-p",
                        "no:cacheprovider", *tests], env=env, capture_output=True, text=True, cwd=ROOT,
                       timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "passed" in out


def test_c_abi_argument_handling_under_sanitizers(tmp_path):
    exe = tmp_path / "api_fuzz"
    csrc = os.path.join(ROOT, "flashattention_fa_fwd_amd", "csrc")
    clang = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(clang):
        pytest.skip("ROCm's clang++ is not installed")
    cmd = [clang, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN, "-I", os.path.join(ROOT, "include"),
           "-I", csrc, "-I", "/opt/rocm/include", os.path.join(csrc, "attn_api.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "api_fuzz.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1"))
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "runtime error" not in out, out[-4000:]
    accepted = int(out.split("api fuzz: ")[1].split(" accepted")[0])
    assert accepted > 10000, out  # the accept paths and the launch arguments are exercised
    print(out.strip())
