"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the library with the host side instrumented (argument checks,
workspace layout, chunk scheduler; the device code is built as usual) and
runs the ABI tests (tests/test_abi.py) against that build in a fresh process
that preloads the sanitizer runtime.  Any invalid memory access or undefined
behaviour in the host code the tests reach aborts that process.  CPU only: on
a host without a GPU the entry points stop at their device check, after every
argument check has run.
"""
import os
import subprocess
import sys

import pytest

from chunked_kl_loss_row_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(900)
def test_abi_tests_pass_under_host_sanitizers(tmp_path):
    runtime = build.sanitizer_runtime()
    if not os.path.exists(build.HIPCC) or not runtime:
        pytest.skip("hipcc or the clang sanitizer runtime is not available")
    lib = build.build(sanitize=True, dest=str(tmp_path / "libkdchunk_sanitized.so"))
    env = dict(os.environ, KDCHUNK_LIB=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the sanitized library must be the one the tests load
    probe = subprocess.run([sys.executable, "-c",
                            "from chunked_kl_loss_row_amd import binding as B; B.lib(); print(B.LIB_PATH)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.strip() == lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout
