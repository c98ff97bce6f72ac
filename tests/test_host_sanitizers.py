"""The library's host C++ (argument validation, the packer, the pool's LRU
planner and bookkeeping) under AddressSanitizer and UndefinedBehaviorSanitizer.

A host-sanitized build of the same sources (device code unchanged) is made,
and the CPU ABI and pool tests run again against it in a subprocess with
clang's sanitizer runtime preloaded; any report ends that run with an error.
CPU only: no kernel is launched."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_pool_tests_under_asan_and_ubsan():
    from int4_expert_ffn_int8_amd import build as b
    if not (os.path.exists(b.HIPCC) or shutil.which(b.HIPCC)):
        pytest.skip("hipcc is not available")
    rt = b.sanitizer_runtime()
    if rt is None:
        pytest.skip("clang's shared ASan runtime is not available")
    lib = b.build_sanitized()
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True,
                           text=True).stdout
    assert "__asan_report" in undef and "__ubsan_handle" in undef, "build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, MOE_LIB_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    which = subprocess.run(
        [sys.executable, "-c",
         "from int4_expert_ffn_int8_amd import binding as B; print(B.load()._name)"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert which.returncode == 0, which.stderr[-3000:]
    assert which.stdout.strip().endswith("libmoe_san.so"), which.stdout
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
         "tests/test_abi_cpu.py", "tests/test_pool_cpu.py"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
