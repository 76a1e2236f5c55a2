"""The CPU ABI tests again, against a build of libdcp whose host code (dcp_api.cpp: argument
validation, the shard plan, kernel choice and workspace layout) carries AddressSanitizer and
UndefinedBehaviorSanitizer. Any report ends the run with an error, so a pass means that every
host-checked path of tests/test_abi.py ran clean."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_asan_and_ubsan():
    from sequence_sharded_kv_amd import _build
    try:
        _build.hipcc()
        runtime = _build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = _build.build_sanitized()
    # the host code is instrumented by both sanitizers
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ, LD_PRELOAD=runtime, DCP_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
