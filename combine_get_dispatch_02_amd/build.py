"""Build libep.so (the HIP library behind include/ep.h) for gfx950 with hipcc.

Run ``python -m combine_get_dispatch_02_amd.build`` (or ``__graft_entry__.build()``).
The shared library is written next to this file so that it travels with the
source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libep.so")
SOURCES = ["ep_api.hip", "layout.hip", "dispatch.hip", "dispatch_ht.hip", "dispatch_ll.hip",
           "combine.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # fp32 stays IEEE: no fast-math, denormals kept, correctly rounded divide.
    "-fno-fast-math",
    "-ffp-contract=off",
    # never emit packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-parameter",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
