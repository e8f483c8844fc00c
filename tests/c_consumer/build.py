"""Compile the plain-C consumer of the library (``vsa_c_example.c``) in
place.  It links ``libvsa.so``, the generator and, being a test program, the
CPU oracle, with run paths relative to its own directory, so the built tree
can move.  Always recompiles."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "vsa_c_example")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = EXE) -> list[str]:
    rpath = ":".join(["$ORIGIN/../../block_sparse_video_amd", "$ORIGIN/../../oracle",
                      "$ORIGIN/../../synth", os.path.join(ROCM, "lib")])
    return ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
            "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
            os.path.join(HERE, "vsa_c_example.c"), "-o", out,
            "-L", os.path.join(ROOT, "block_sparse_video_amd"), "-lvsa",
            "-L", os.path.join(ROOT, "oracle"), "-loracle_vsa",
            "-L", os.path.join(ROOT, "synth"), "-lsynth",
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath," + rpath]


def build() -> str:
    """Needs libvsa.so, liboracle_vsa.so and libsynth.so built first."""
    tmp = EXE + ".tmp"
    r = subprocess.run(command(tmp), capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed ({r.returncode}):\n{' '.join(command(tmp))}\n{r.stderr}")
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
