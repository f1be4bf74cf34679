"""CPU build of the host validation layer (api.cpp, paley.cpp) under
AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers
replaced by launch_stubs.cpp: ``_build/libhadarot_hostsan.so``.  g++ only; no
device code is built.  Used by tests/test_host_sanitizers.py, which runs
tests/test_abi_host.py against this library."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "hadamard_rotation_preprocessing_amd", "csrc")
OUT = os.path.join(HERE, "_build", "libhadarot_hostsan.so")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def build() -> str:
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-shared", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include")] + SAN + [
           os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "paley.cpp"), os.path.join(HERE, "launch_stubs.cpp"),
           "-o", OUT]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("sanitizer build failed")
    return OUT


def asan_runtime() -> str:
    """Path of g++'s shared AddressSanitizer runtime (preloaded into Python)."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()


if __name__ == "__main__":
    print(build())
