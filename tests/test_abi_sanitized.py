"""The host-side ABI tests again, against the library whose C ABI layer is built with host
AddressSanitizer and UndefinedBehaviorSanitizer (no GPU: every call there fails validation
or is pure host logic before any device work)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_abi_tests_under_host_sanitizers():
    from unified_transformer_recommender_onetrans_amd.sanitized_build import ASAN_RUNTIME, build_sanitized
    if not os.path.exists(ASAN_RUNTIME):
        pytest.skip("clang ASan runtime not found")
    lib = build_sanitized()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report_load" in out and "__ubsan_handle" in out, "library is not instrumented"
    env = dict(os.environ, ONETRANS_LIB=lib, LD_PRELOAD=ASAN_RUNTIME,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_attention_routes.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
