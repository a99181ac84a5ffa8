"""Build libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkda.so")
SOURCES = ["api.hip", "debug.hip", "gate.hip", "decode.hip", "decode_gated.hip", "prefill.hip", "prep.hip",
           "state.hip", "shortconv.hip", "backward.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source into one shared library; returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [
        hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU ops stay off: hipcc otherwise forms them from plain float code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-munsafe-fp-atomics", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-o", tmp,
    ] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libkda.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
