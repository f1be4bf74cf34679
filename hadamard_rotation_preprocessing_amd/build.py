"""Build step: compiles the HIP library libhadarot.so for gfx950 with hipcc.

Usage: ``python -m hadamard_rotation_preprocessing_amd.build`` (or
``__graft_entry__.build()``).  Output: ``hadamard_rotation_preprocessing_amd/lib/libhadarot.so``,
and ``lib/libhrstream.so``, the plain streaming kernel bench.py times as a
reference (csrc/stream_ref.hip; not part of the rotate + quantize path).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libhadarot.so")
STREAM_LIB = os.path.join(LIBDIR, "libhrstream.so")   # bench.py's streaming reference

ARCH = os.environ.get("HADAROT_ARCH", "gfx950")

# Device code: no packed-fp32 instructions (the compiler would otherwise form
# v_pk_* from ordinary float code; the host pass ignores the feature), and MFMA
# results in ordinary VGPRs (no accumulation-register copies).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("command failed: %s" % " ".join(cmd))
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)


def build(verbose: bool = True) -> str:
    """Compile every source and link libhadarot.so; returns its path."""
    hipcc = _hipcc()
    obj_dir = os.path.join(LIBDIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    sources = [("kernels.hip", True), ("fast.hip", True), ("colrot.hip", True), ("api.cpp", False), ("paley.cpp", False)]
    cmds, objs = [], []
    for src, device in sources:
        out = os.path.join(obj_dir, src + ".o")
        cmd = [hipcc, "-c"] + (["-x", "hip"] if device else []) + [os.path.join(CSRC, src), "-o", out]
        cmd += COMMON + ["--offload-arch=" + ARCH]
        if device:
            cmd += DEVICE_FLAGS
        cmds.append(cmd)
        objs.append(out)
    # the sources are independent: compile them side by side
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    # bench.py's streaming reference (a separate library: not part of the path)
    tmp = STREAM_LIB + ".tmp"
    _run([hipcc, "-shared", "-x", "hip", os.path.join(CSRC, "stream_ref.hip"), "-o", tmp] + COMMON +
         ["--offload-arch=" + ARCH] + DEVICE_FLAGS, verbose)
    os.replace(tmp, STREAM_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
