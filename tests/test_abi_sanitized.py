"""The host side of the C ABI (argument validation, workspace layout, launch
order) under AddressSanitizer and UndefinedBehaviorSanitizer: the ABI checks
of test_abi_cpu.py and test_binding_checks.py run, in a child process with the
sanitizer runtime preloaded, against a copy of the library whose ABI layer
build() compiles with host sanitizers. No GPU is touched: every call fails
validation before anything is enqueued."""

import os
import subprocess
import sys

import pytest

from block_sparse_attention_stats_amd import build as bld

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    out = subprocess.run([bld.HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                         text=True).stdout.strip()
    if out and os.path.exists(out):
        return out
    base = os.path.join(os.path.dirname(os.path.dirname(bld.HIPCC)), "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(base)) if os.path.isdir(base) else []:
        cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    return None


def test_abi_checks_under_host_sanitizers():
    if not os.path.exists(bld.SAN_LIB):
        pytest.skip("the host-sanitized library is not built (build() makes it)")
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("the AddressSanitizer runtime is not installed")
    syms = subprocess.run(["nm", "-D", bld.SAN_LIB], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the ABI layer is not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys; sys.path.insert(0, %r); import block_sparse_attention_stats_amd as bsa; "
            "bsa.load_library(%r); import pytest; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py', "
            "'tests/test_binding_checks.py']))") % (ROOT, bld.SAN_LIB)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
