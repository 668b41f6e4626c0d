"""Build libmoe.so in-tree: every csrc/*.hip compiled for gfx950 with hipcc.

Flags: correctly rounded fp32 division and square root and no fp contraction
(the router's fixed-order arithmetic relies on both), and packed-fp32 code
generation disabled (the compiler would otherwise pair scalar fp32 ops into
v_pk_* instructions).  The grouped MFMA GEMMs take the VGPR form of the matrix
instructions: each block dot's result is converted and scaled at once, and
results left in accumulation registers cost a copy per element (four more
VALU instructions per MFMA in the down projection).
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


# extra flags per source file
FILE_FLAGS = {
    "ffn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "ffn_rows.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "peak.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc", *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
