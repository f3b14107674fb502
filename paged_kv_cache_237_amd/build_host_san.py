"""Builds libpa_host_san.so: the library's host layer (api.cpp,
block_manager.cpp) compiled by g++ with AddressSanitizer and
UndefinedBehaviorSanitizer (any finding aborts), linked with
csrc/host_stub.cpp in place of the kernels and the HIP runtime.  No device
code is compiled.  tests/test_host_sanitizers.py runs the CPU suites of the
ABI and the block manager against it (PA_LIB_PATH selects the library the
binding loads; the sanitizer runtime is preloaded)."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa_host_san.so")
SOURCES = ["api.cpp", "block_manager.cpp", "host_stub.cpp"]
FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
         "-Wall", "-Wno-unused-function"]


def rocm_include() -> str:
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")


def sanitizer_runtime() -> str:
    """Path of g++'s AddressSanitizer runtime (to preload into python), or ''."""
    p = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else ""


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["g++", *FLAGS, "-I", rocm_include(), "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
