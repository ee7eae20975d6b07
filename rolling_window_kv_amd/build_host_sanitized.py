"""Build an instrumented copy of librkv.so for the host-sanitizer test.

The host half of every source (argument validation, the restart policy, the
mel filterbank, state set-up, launch wrappers) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer; the device code is compiled
as usual.  The result is not the product library: it goes to
_build/host_sanitized/librkv_host_sanitized.so and is loaded only by
tests/test_host_sanitizers.py (through RKV_LIBRARY, with the sanitizer
runtime preloaded into an uninstrumented Python).  No GPU is needed.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

from rolling_window_kv_amd.build import ARCH, CSRC, HIPCC, PKG, ROOT

OUT = os.path.join(PKG, "_build", "host_sanitized")
LIB = os.path.join(OUT, "librkv_host_sanitized.so")

# every sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address,undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
FLAGS = [f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, *HOST_SAN]


def runtime() -> str:
    """Path of the ASan runtime matching the compiler (to preload)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = "/opt/rocm/llvm/bin/clang"
    out = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True, check=True).stdout.strip()
    return out


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def comp(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *HOST_SAN[:2],
                        "-o", LIB, *objs], capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    return LIB


if __name__ == "__main__":
    print(build())
