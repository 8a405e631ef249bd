"""The host code of the library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

Argument validation, the decode split plan, overlap checks and dispatch are
host C++; ``build(sanitize=True)`` compiles that code (not the device code)
with -fsanitize=address,undefined and -fno-sanitize-recover. This test runs
the whole C-ABI suite (``test_abi.py``: every rejection path, workspace
sizing, status strings, exported symbols) in a child process with the
sanitizer runtime preloaded and the binding pointed at the sanitized build;
any report aborts the child.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitized_lib():
    from exact_tiled_attention_fwd_amd import build as b
    if not os.path.exists(b.HOSTSAN_LIB_PATH):
        b.build(sanitize=True)
    return b.HOSTSAN_LIB_PATH


def _runtime():
    clang = "/opt/rocm/lib/llvm/bin/clang"
    if not os.path.exists(clang):
        pytest.skip("ROCm clang not found")
    rt = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                        text=True).stdout.strip()
    assert os.path.exists(rt), rt
    return rt


def test_sanitized_build_is_instrumented():
    lib = _sanitized_lib()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_abi_suite_under_host_sanitizers():
    lib, rt = _sanitized_lib(), _runtime()
    env = dict(os.environ, LD_PRELOAD=rt, FA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import ctypes, sys, pytest; assert hasattr(ctypes.CDLL(None), '__asan_init'); "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, out
    assert " passed" in r.stdout, out
