"""The CPU tests that call into libkvq.so (the C ABI's argument checks and
error returns, the width allocator's host greedy, the window-roll count rule
and CacheCard framing), run again against a build whose host code has
AddressSanitizer and UBSan (hipcc, host pass only, -fno-sanitize-recover=all):
an out-of-bounds access, a use after free or undefined behaviour on any host
path these tests reach aborts the run.  The tests run in a subprocess that
selects that build with KVQ_LIB and preloads clang's ASan runtime (the
interpreter is not instrumented); leak checks are off (the interpreter's own
allocations)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["test_abi.py", "test_alloc.py", "test_append_counts.py", "test_card.py"]


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_runtime() is None, reason="clang's ASan runtime not installed")
def test_host_layer_under_asan_ubsan():
    from quantized_kv_cache_group_amd import build
    lib = build.build_host_sanitized()
    # the build is instrumented: its host code calls the ASan and UBSan handlers
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                          check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms
    env = dict(os.environ)
    env.update(KVQ_LIB=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join("tests", f) for f in HOST_TESTS]], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
