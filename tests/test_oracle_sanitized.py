"""The oracle's pin tests again, against a build of kvq_ref.c with
AddressSanitizer and UBSan (gcc, -fno-sanitize-recover=all): an
out-of-bounds access, a use after free or undefined behaviour anywhere the
pins reach aborts the run.  The tests run in a subprocess with the ASan
runtime preloaded (the interpreter itself is not instrumented) and leak
checks off (the interpreter's own allocations)."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = sorted(f for f in os.listdir(os.path.join(ROOT, "tests")) if f.startswith("test_oracle_")
              and f != "test_oracle_sanitized.py")


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime not installed")
def test_oracle_pins_under_asan_ubsan():
    lib = oracle.build_sanitized()
    env = dict(os.environ)
    env.update(KVQ_ORACLE_LIB=lib, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join("tests", f) for f in PINS]], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=1200)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
