"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

A host-instrumented build (demand_paged_kv_amd.build.build_host_sanitized: device code as
usual, host code instrumented) runs the argument-validation tests of test_abi.py in a
fresh interpreter with the ASan runtime preloaded; any sanitizer report fails the test.
No GPU call is made: the validation answers before any launch."""
import os
import subprocess
import sys

import pytest

from demand_paged_kv_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_validation_under_sanitizers():
    try:
        lib = BLD.build_host_sanitized(verbose=False)
        runtime = BLD.asan_runtime()
    except RuntimeError as e:
        pytest.fail(str(e))
    code = ("import sys\n"
            "from demand_paged_kv_amd import binding as B\n"
            f"B.load({lib!r})\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', 'tests/test_abi.py',"
            " '-k', 'not single_hip_runtime']))\n")
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "6 passed" in r.stdout, r.stdout[-2000:]
