"""The C-ABI tests (tests/test_abi.py) against a build whose host code,
api.hip's argument checking included, runs under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only: every call there is rejected before the
HIP runtime is touched, so no kernel runs). Any memory error or undefined
behaviour aborts the child process with the sanitizer's report."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(600)
def test_abi_under_sanitizers():
    sys.path.insert(0, ROOT)
    from exact_attention_110_amd import build as B
    try:
        lib = B.build_sanitized()
        rt = B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"sanitized build unavailable: {e}")
    code = ("import sys, pytest\n"
            f"sys.path.insert(0, {ROOT!r})\n"
            "from exact_attention_110_amd import binding\n"
            f"binding.LIB_PATH = {lib!r}\n"
            f"sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', {os.path.join(ROOT, 'tests', 'test_abi.py')!r}]))\n")
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt
    # the interpreter and torch are not instrumented: leak checking and the
    # container-overflow check would report their allocations, not ours
    env["ASAN_OPTIONS"] = "detect_leaks=0:detect_container_overflow=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, cwd=ROOT)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
