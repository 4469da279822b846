"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the whole ABI validation suite (tests/test_abi.py: argument checks that reject
bad calls before any HIP call, layout queries, status strings, the binding's
output checks) runs in a child interpreter against a build of the library
whose host pass is instrumented (bit_fp8_codebook_amd/build.py, build_asan),
with clang's ASan runtime preloaded.  Any sanitizer report fails the test.
CPU only: no kernel is launched."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

CHILD = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import bit_fp8_codebook_amd._lib as L
L.LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main([{suite!r}, '-q', '-p', 'no:cacheprovider']))
"""


def _stale(lib, srcs):
    return not os.path.exists(lib) or any(os.path.getmtime(s) > os.path.getmtime(lib) for s in srcs)


def test_abi_suite_under_host_sanitizers():
    from bit_fp8_codebook_amd import build
    try:
        rt = build.asan_runtime()
        build.hipcc()
    except RuntimeError as e:
        pytest.skip(str(e))
    srcs = build.sources() + [os.path.join(ROOT, "include", "q3.h")]
    if _stale(build.ASAN_LIB, srcs):
        build.build_asan(verbose=False)
    code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=build.ASAN_LIB,
                        suite=os.path.join(ROOT, "tests", "test_abi.py"))
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout
