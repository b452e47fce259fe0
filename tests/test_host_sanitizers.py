"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only; the device code is not instrumented).

relattn_api.cpp (argument validation, T5 thresholds, workspace sizing, the
launch plan) is compiled with the sanitizers for the host side only and
linked with the normal kernel object into a separate library under _build/.
tests/test_abi_cpu.py then runs against that library in a child process with
the sanitizer runtime preloaded; any report aborts the child.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from transformer_attention_relative_amd import build as B  # noqa: E402

SAN_LIB = os.path.join(B.BUILD_DIR, "librelattn_hostsan.so")
# host-side only: each sanitizer flag goes to the host compilation
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined",
            "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def sanitized_library():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("the clang AddressSanitizer runtime is not installed")
    kobj = os.path.join(B.BUILD_DIR, "relattn_kernels.o")
    if not os.path.exists(kobj):
        kobj = B.compile_object("relattn_kernels.hip")
    aobj = B.compile_object("relattn_api.cpp", extra=HOST_SAN)
    # the sanitized object replaces the normal one under another name
    san_obj = os.path.join(B.BUILD_DIR, "relattn_api_hostsan.o")
    os.replace(aobj, san_obj)
    B.link([kobj, san_obj], SAN_LIB, extra=["-Xarch_host", "-fsanitize=address,undefined",
                                            "-shared-libasan"])
    # restore the normal host object for later links
    B.compile_object("relattn_api.cpp")
    return SAN_LIB, rt


def test_abi_checks_run_clean_under_asan_and_ubsan(sanitized_library):
    lib, rt = sanitized_library
    env = dict(os.environ)
    env.update(RELATTN_LIB=lib, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (proc.stdout + proc.stderr)[-4000:]
    assert proc.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in proc.stderr and "runtime error" not in proc.stderr, tail
    assert " passed" in proc.stdout, tail


def test_the_sanitized_library_is_the_one_loaded(sanitized_library):
    # the child really loads the sanitized build (it exports the sanitizer's
    # module constructor)
    lib, rt = sanitized_library
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_init" in syms or "__asan_register_globals" in syms
