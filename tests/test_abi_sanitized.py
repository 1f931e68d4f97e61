"""The C-ABI host checks under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The host code of host.hip (argument validation, pool handles, workspace
layouts and sizing, split choice, timing bookkeeping) is rebuilt with host-side
ASan and UBSan (device code untouched) and tests/test_abi_host.py runs against
it in a child process with the sanitizer runtime preloaded. Any heap overflow,
use after free or undefined behaviour in the host layer aborts that run.
"""
import glob
import os
import subprocess
import sys

import pytest

from paged_kv_decode_reshape_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")) + \
        sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(not all(os.path.exists(_build._obj("release", s)) for s in _build._sources()),
                    reason="release objects not built (run __graft_entry__.build())")
@pytest.mark.skipif(_asan_runtime() is None, reason="no clang ASan runtime found")
def test_abi_host_checks_under_asan_and_ubsan():
    lib = _build.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), PKV_LIBRARY_PATH=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_host.py")],
                         env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, out
    assert "passed" in res.stdout and "AddressSanitizer" not in out and "runtime error" not in out, out
