"""Build ``libkvq.so`` (the HIP library behind include/kvq.h) in-tree for gfx950.

Each source is compiled with hipcc to an object, then linked into one shared
library next to this file.  Flags:
  * --offload-arch=gfx950 only (no other targets, no CUDA paths);
  * packed fp32 instructions disabled for the device code;
  * IEEE fp32 denormals kept, fp32 divide correctly rounded;
  * the quantizer's translation unit also has -ffp-contract=off, so its
    codes, scales and biases follow the documented binary32 sequence.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-munsafe-fp-atomics",
]
PER_FILE = {
    "quantize.hip": ["-ffp-contract=off", "-fno-honor-nans", "-mno-amdgpu-ieee"],
}
SOURCES = ["kvq_api.cpp", "quantize.hip", "attend_generic.hip", "decode_gqa.hip", "decode_g4.hip", "chunk.hip",
           "mla.hip", "card.hip", "sparse.hip", "alloc.hip"]


# Host-side AddressSanitizer + UBSan (the device code is compiled as in the
# normal build): every sanitizer flag applies to the host pass only.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_BUILD = os.path.join(HERE, "_build_asan")
ASAN_LIB = os.path.join(HERE, "libkvq_asan.so")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    lang = [] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


def build_host_sanitized() -> str:
    """The same library with its host code (argument checks, planning, the
    width allocator's greedy, launch code) built with AddressSanitizer and
    UBSan, as libkvq_asan.so beside the normal build.  It is never loaded by
    default: a process selects it with KVQ_LIB and must preload clang's ASan
    runtime (the interpreter is not instrumented)."""
    os.makedirs(ASAN_BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, ASAN_BUILD, HOST_SANITIZE), SOURCES))
    tmp = ASAN_LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SANITIZE, "-shared-libsan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    print(build())
