"""The C-ABI argument checks (tests/test_boundary.py) against a build of the
host library instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only; the kernels are the normal build's), on the CPU: any invalid
memory access, leak-free use of freed memory or undefined behaviour in the
validation, error-reporting and set-up paths aborts the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_checks_under_sanitizers():
    from bit_attention_oscar_amd import build as b
    try:
        lib = b.build_sanitized()
        rt = b.sanitizer_runtime()
    except RuntimeError as e:          # no HIP toolchain here
        pytest.skip(str(e))
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OSCAR_KV_LIBRARY": lib,
    })
    p = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (p.stdout + p.stderr)[-3000:]
    assert p.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert " passed" in p.stdout, tail
