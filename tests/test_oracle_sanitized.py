"""The CPU reference under AddressSanitizer and UndefinedBehaviorSanitizer.

Runs every pin of test_oracle_pins.py, and the single-threaded side of the
threaded-build comparison, against an instrumented build of oracle/lsa_oracle.c
in a subprocess that preloads the ASan runtime; any out-of-bounds access, use
of freed memory or undefined behaviour aborts that run.  (The mutation tests
are not run this way: a planted mistake may well read out of bounds, which is
one more way of being rejected, not a fault of the reference.)"""
import os
import subprocess
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.timeout(600)
def test_pins_pass_under_address_and_ub_sanitizers():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    env = dict(os.environ)
    env.update({
        "LSA_ORACLE_SANITIZE": "1",
        "LD_PRELOAD": asan,
        # Python itself leaks by design at exit; the reference frees what it allocates
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_oracle_pins.py",
                        "tests/test_oracle_threads.py"],
                       cwd=REPO, env=env, capture_output=True, text=True, timeout=580)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, tail
