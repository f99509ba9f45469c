"""Host-side sanitizer runs, no GPU: AddressSanitizer and
UndefinedBehaviorSanitizer builds of
  * the CPU oracle (oracle/mxref.c), run under its pins (tests/test_oracle.py),
  * the C-ABI validation layer (mxfp8_block_scaled_04_amd/csrc/api.cpp) with
    the kernel launchers replaced by host stubs (tests/sanitize/), run under
    the argument-validation tests (tests/test_abi.py).
Both builds are made here with gcc / g++ (host code only; no HIP source is
compiled with a sanitizer) and loaded by a child pytest process with the
ASan runtime preloaded; any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


def _asan_runtime():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def test_oracle_and_abi_validation_under_sanitizers(tmp_path):
    asan = _asan_runtime()
    oracle_so = str(tmp_path / "libmxref_san.so")
    abi_so = str(tmp_path / "libmxmoe_host_san.so")
    _run(["gcc", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-fPIC", "-shared", *SAN,
          os.path.join(ROOT, "oracle", "mxref.c"), "-o", oracle_so, "-lm"])
    _run(["g++", "-std=c++17", "-Wall", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          os.path.join(ROOT, "mxfp8_block_scaled_04_amd", "csrc", "api.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", abi_so])
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, MXREF_LIB=oracle_so, MXMOE_ABI_LIB=abi_so,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle.py", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    log = r.stdout[-4000:] + "\n" + r.stderr[-4000:]
    assert r.returncode == 0, log
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in r.stdout + r.stderr, log
    assert " passed" in r.stdout, log
