"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: builds
rkv_oracle.c with -fsanitize=address,undefined (gcc, host code only) and runs
the oracle's pin tests against that build in a child process that preloads
the sanitizer runtime.  Any out-of-bounds access, use after free or
undefined operation in the oracle ends the child with a report."""
import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PINS = ["test_oracle_hsa.py", "test_oracle_mt.py", "test_oracle_snapkv.py", "test_oracle_split.py",
        "test_oracle_summaries.py"]


def _runtime(name: str) -> str:
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else ""


@pytest.mark.timeout(900)
def test_oracle_pins_under_sanitizers():
    asan = _runtime("libasan.so")
    if not asan:
        pytest.skip("gcc's libasan is not installed")
    oracle.build(sanitize=True)
    env = dict(os.environ)
    env.update({
        "RKV_ORACLE_SANITIZE": "1",
        "LD_PRELOAD": asan,
        # the interpreter itself is not instrumented: leak checks off, the
        # oracle's own errors fatal
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    pins = [os.path.join(HERE, f) for f in PINS if os.path.exists(os.path.join(HERE, f))]
    assert pins
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", *pins], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=850)
    tail = (r.stdout[-3000:] + "\n" + r.stderr[-3000:])
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
