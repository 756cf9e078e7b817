"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.c is built a second time with -fsanitize=address,undefined (every report
fatal) and the oracle's pin tests are run again in a child process that preloads
the sanitizer runtimes and loads that build: an out-of-bounds access, a use of
freed memory or undefined arithmetic in any oracle function those pins reach
fails this test.  CPU only."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers():
    import oracle

    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    oracle.build(force=True, sanitized=True)
    env = dict(os.environ)
    env.update(ORACLE_SANITIZED="1", LD_PRELOAD=asan + ":" + ubsan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    pins = sorted(os.path.join(ROOT, "tests", f) for f in os.listdir(os.path.join(ROOT, "tests"))
                  if f.startswith("test_oracle_") and f != os.path.basename(__file__))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *pins], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
