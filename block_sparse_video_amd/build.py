"""Build step for the gfx950 VSA library (``libvsa.so``), in-tree.

Compiles the HIP kernels and the C-ABI host code in one hipcc invocation.
Packed FP32 instructions are disabled for device code
(``-target-feature -packed-fp32-ops``); hipcc's host pass warns that it does
not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libvsa.so")
SOURCES = ["pool_pack.hip", "select_coarse.hip", "fine_attn.hip", "gemm_qkvg.hip", "subblock.hip",
           "noalloc.hip", "vsa_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def hipcc_command(out: str = LIB_PATH, extra=()) -> list[str]:
    return [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra, "-o", out, *[os.path.join(CSRC, s) for s in SOURCES]]


def build(verbose: bool = False) -> str:
    """Always recompiles.  Writes to a temporary name and renames, so a
    process that has the old library loaded is not disturbed."""
    tmp = LIB_PATH + ".tmp"
    cmd = hipcc_command(tmp)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
