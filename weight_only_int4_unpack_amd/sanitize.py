"""Sanitizer build of the host side, and the C-ABI tests run against it.

Builds ``libw4a16_asan.so`` from ``csrc/w4a16_host.cpp`` (argument checks,
route/tile selector, workspace bookkeeping, host pack/unpack) with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer (every finding fatal), linked
against host-only stand-ins for the kernels (``csrc/sanitize_stubs.cpp``),
then runs ``tests/test_abi.py`` with that library in place of the real one
(``W4A16_LIB``) and the sanitizer runtimes preloaded into Python. CPU only:
no GPU code is built or run.

Usage: ``python -m weight_only_int4_unpack_amd.sanitize`` (exit status of
the test run).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libw4a16_asan.so")
ROCM = "/opt/rocm"


def build() -> str:
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(CSRC, "w4a16_host.cpp"), os.path.join(CSRC, "sanitize_stubs.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer build failed:\n{' '.join(cmd)}\n{r.stderr}")
    return OUT


def runtime(name: str) -> str:
    return subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True, check=True).stdout.strip()


def main() -> int:
    lib = build()
    env = dict(os.environ)
    env["W4A16_LIB"] = lib
    env["LD_PRELOAD"] = ":".join([runtime("libasan.so"), runtime("libubsan.so")])
    # Python itself is not instrumented: its allocations at exit are not ours
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["CUDA_VISIBLE_DEVICES"] = ""
    env["HIP_VISIBLE_DEVICES"] = ""
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env)
    return r.returncode


if __name__ == "__main__":
    sys.exit(main())
