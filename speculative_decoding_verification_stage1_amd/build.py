"""Build libss.so (the HIP library) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libss.so")
SOURCES = [os.path.join(CSRC, "ss_api.hip")]
ARCH = os.environ.get("SS_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # IEEE binary32 as written: no contraction of a*b+c, correctly rounded
    # division, no fast-math
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep private arrays (the GEMM's staged loads) in registers: moving
    # them into LDS would take the LDS the GEMM's tiles need
    "-mllvm", "-disable-promote-alloca-to-lds",
]


def build(verbose: bool = False) -> str:
    cmd = ["hipcc", *HIPCC_FLAGS, "-o", LIB + ".tmp", *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
    if verbose and (r.stdout or r.stderr):
        print(r.stdout + r.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
