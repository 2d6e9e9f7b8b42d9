"""The C ABI's host-side validation under AddressSanitizer and
UndefinedBehaviorSanitizer: the library is rebuilt with the host pass
instrumented (device code as usual), and tests/test_abi.py runs against it
in a child process with the ASan runtime preloaded.  No kernel runs: those
tests only reach argument validation."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
@pytest.mark.skipif(_asan_runtime() is None, reason="no ASan runtime")
def test_abi_validation_under_sanitizers():
    from block_sparse_paged_query_amd.build import build
    lib = build(sanitize=True)
    env = dict(os.environ, MSA_LIBRARY=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert " passed" in res.stdout
