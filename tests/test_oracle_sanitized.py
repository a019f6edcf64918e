"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.c is built a second time with -fsanitize=address,undefined (oracle/__init__.py, ORACLE_SANITIZE)
and the oracle's own test files run against that build in a child process that preloads the
sanitizer runtimes; any out-of-bounds access, use after free or undefined behaviour aborts the
child, and the test fails with the sanitizer's report.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_pretokenize.py", "tests/test_oracle_bpe.py", "tests/test_oracle_deepseek.py",
        "tests/test_oracle_spans.py", "tests/test_oracle_added.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_under_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    env = dict(os.environ)
    env.update(ORACLE_SANITIZE="1", LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    sys.path.insert(0, ROOT)
    # build the sanitized library first (in this process: gcc only, nothing loaded)
    b = subprocess.run([sys.executable, "-c", "import oracle; oracle.build(force=True)"], cwd=ROOT,
                       env=dict(env, LD_PRELOAD=""), capture_output=True, text=True)
    assert b.returncode == 0, b.stdout + b.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
