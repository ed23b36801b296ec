"""The CPU-side ABI tests again, against a build of the library whose host
code carries AddressSanitizer and UndefinedBehaviorSanitizer (the device
code is compiled as usual): argument validation, handle checks, error
strings and the workspace sizing run with out-of-bounds, use-after-free and
undefined-behaviour checks armed.  The counterpart, for the host side, of
the memory checker the C++/CUDA page runs over its CUDA code (section 5.1)."""

import glob
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

PKG = os.path.join(ROOT, "autograd_transformer_amd")


def _sanitized_lib():
    from autograd_transformer_amd import build as b
    srcs = glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*"))
    newest = max(os.path.getmtime(f) for f in srcs)
    if not os.path.exists(b.ASAN_LIB) or os.path.getmtime(b.ASAN_LIB) < newest:
        b.build(sanitize=True)
    return b.ASAN_LIB


def _asan_runtime():
    for clang in ("/opt/rocm/llvm/bin/clang", "clang"):
        try:
            out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                                 capture_output=True, text=True, timeout=60).stdout.strip()
        except (OSError, subprocess.TimeoutExpired):
            continue
        if out and os.path.isabs(out) and os.path.exists(out):
            return out
    return None


def test_abi_cpu_tests_pass_under_asan_and_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime on this machine")
    lib = _sanitized_lib()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code not instrumented"
    env = dict(os.environ, TT_LIB_PATH=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr + r.stdout
