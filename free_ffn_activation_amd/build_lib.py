"""Compile the HIP sources of the package into libprox.so (gfx950).

Usage: python -m free_ffn_activation_amd.build_lib  (or call build_library()).
Always recompiles; the output sits next to this file.

Host-sanitizer build (CPU only): python -m free_ffn_activation_amd.build_lib
--host-sanitizers [--run-tests] builds libprox_hostsan.so, whose host code
(argument validation, planning, the C ABI) carries AddressSanitizer and
UndefinedBehaviorSanitizer while the device code is built as usual, and with
--run-tests runs the host-only ABI tests against it (the sanitizer runtime is
preloaded into the Python process; no GPU is touched).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libprox.so")
LIB_HOSTSAN = os.path.join(PKG, "libprox_hostsan.so")
SOURCES = ["prox_api.hip", "stage1.hip", "stage1_batch.hip", "stage1_qt.hip", "stage2_upgate.hip", "stage2_down.hip",
           "stage2_fused.hip", "stage2_batch.hip", "stage1_w16.hip", "pack.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fvisibility=hidden", "-munsafe-fp-atomics",
    # packed fp32 VALU ops are kept out of every kernel on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]

# Host-only instrumentation: every sanitizer flag is routed to the host
# compilation with -Xarch_host, so no device code is instrumented.
HOSTSAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
    "-shared-libsan", "-g",
]
HOSTSAN_TESTS = ["tests/test_abi_cpu.py", "tests/test_budget_cpu.py"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libprox.so)")


def _compile(out: str, extra, verbose: bool) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stdout}\n{proc.stderr}")
    os.replace(tmp, out)
    return out


def build_library(verbose: bool = False) -> str:
    return _compile(LIB, [], verbose)


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that the host-sanitizer build links."""
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")) + \
        sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"))
    if not cands:
        raise RuntimeError("no libclang_rt.asan runtime under /opt/rocm/llvm")
    return cands[-1]


def build_hostsan_library(verbose: bool = False) -> str:
    return _compile(LIB_HOSTSAN, HOSTSAN_FLAGS, verbose)


def run_hostsan_tests() -> int:
    """The host-only ABI tests against libprox_hostsan.so, sanitizer runtime
    preloaded; any report aborts the run."""
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan_runtime(), PROX_LIBRARY=LIB_HOSTSAN,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *HOSTSAN_TESTS]
    print("LD_PRELOAD=" + env["LD_PRELOAD"], "PROX_LIBRARY=" + LIB_HOSTSAN, " ".join(cmd), flush=True)
    return subprocess.run(cmd, cwd=ROOT, env=env).returncode


if __name__ == "__main__":
    if "--host-sanitizers" in sys.argv:
        print(build_hostsan_library(verbose="-v" in sys.argv))
        if "--run-tests" in sys.argv:
            sys.exit(run_hostsan_tests())
    else:
        print(build_library(verbose="-v" in sys.argv))
