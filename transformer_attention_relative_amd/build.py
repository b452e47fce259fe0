"""Build the gfx950 shared library ``librelattn.so`` in-tree with hipcc.

    python -m transformer_attention_relative_amd.build [-v]

Every call recompiles (a stale library is never reused silently).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "librelattn.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["relattn_kernels.hip", "relattn_api.cpp"]
# the benchmark's MFMA peak probe, a separate library
PROBE_SOURCE = "mfma_peak.hip"
PROBE_PATH = os.path.join(PKG_DIR, "libmfma_peak.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 instructions stay off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no NaNs in the kernels' arithmetic (scores are finite or -inf): fmaxf
    # then maps to v_max / v_max3 without quieting each operand first
    "-fno-honor-nans",
    # an inline-assembly diagnostic (e.g. a clobbered register the compiler
    # reserves) fails the build
    "-Werror=inline-asm",
    "-Wno-unused-command-line-argument",
]


BUILD_DIR = os.path.join(ROOT, "_build")


def hipcc_path() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librelattn.so)")


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd)}")
    return proc


def compile_object(source: str, extra=()) -> str:
    """Compile one source of csrc/ to an object under _build/; return its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    obj = os.path.join(BUILD_DIR, os.path.splitext(source)[0] + ".o")
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    _run([hipcc_path(), *flags, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          "-c", os.path.join(CSRC, source), "-o", obj + ".tmp"])
    os.replace(obj + ".tmp", obj)
    return obj


def link(objects, out_path, extra=()):
    tmp = out_path + ".tmp"
    _run([hipcc_path(), "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objects, "-o", tmp])
    os.replace(tmp, out_path)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source for gfx950 (the library and the benchmark's
    MFMA probe); return the library's .so path."""
    t0 = time.time()
    objs = [compile_object(src) for src in SOURCES]
    link(objs, LIB_PATH)
    link([compile_object(PROBE_SOURCE)], PROBE_PATH)
    if verbose:
        print(f"built {LIB_PATH} in {time.time() - t0:.1f}s")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
