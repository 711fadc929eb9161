"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with the host side instrumented (device code as usual),
then runs the ABI tests -- argument validation and error paths of every entry
point, workspace queries, the host functions that compute the fractal and
head-aware tile orders -- in a child process that preloads the sanitizer
runtime and loads that build. Any sanitizer report aborts the child.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_under_asan_and_ubsan():
    from block_sparse_attention_avg_amd import _build
    try:
        lib = _build.build_sanitized()
        runtime = _build.asan_runtime()
    except RuntimeError as e:          # no hipcc / runtime in this image
        pytest.skip(str(e))
    env = dict(os.environ, LD_PRELOAD=runtime, BSA_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    check = ("import block_sparse_attention_avg_amd as b; import sys; "
             "sys.exit(0 if b.load()._name.endswith('libbsa_san.so') else 3)")
    r = subprocess.run([sys.executable, "-c", check], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
