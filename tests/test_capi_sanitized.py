"""The C ABI contract tests again, against a copy of the library whose host
code runs under AddressSanitizer and UndefinedBehaviorSanitizer (argument
validation, error text, workspace carving, launch set-up). The copy is built
on demand by `python -m long_context_indexer_block_amd.build --sanitize` and
loaded in a child process with the clang ASan runtime preloaded."""
import glob
import os
import subprocess
import sys

import pytest

from long_context_indexer_block_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale():
    if not os.path.exists(B.SANITIZE_LIB):
        return True
    t = os.path.getmtime(B.SANITIZE_LIB)
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def sanitized_lib():
    try:
        B.hipcc()
        rt = B.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if _stale():
        B.build_sanitized(jobs=8, verbose=False)
    return B.SANITIZE_LIB, rt


def test_sanitized_copy_is_instrumented(sanitized_lib):
    lib, _ = sanitized_lib
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms


def test_capi_contract_under_sanitizers(sanitized_lib):
    lib, rt = sanitized_lib
    env = dict(os.environ, HISA_LIBRARY=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    code = ("import sys, pytest, long_context_indexer_block_amd as H; "
            f"assert H.LIB_PATH == {lib!r}; "
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_capi.py']))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
