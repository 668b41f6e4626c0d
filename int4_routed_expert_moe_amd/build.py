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
import re
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


# Kernels whose speed was measured to depend on their register allocation,
# with the VGPR count of the measured build: a build above it gets a warning
# (the multi-token int4 gate/up went from 103 to 136 us per launch at 8
# tokens when an unrelated edit moved it from 250 to 256 VGPRs).
VGPR_WATCH = {
    "_ZN3moe12_GLOBAL__N_115k_gate_up_smallILi4ELi1ELi3ELb0EEEvNS_9LayerArgsE": 199,
    "_ZN3moe12_GLOBAL__N_115k_gate_up_smallILi4ELi2ELi3ELb0EEEvNS_9LayerArgsE": 250,
}
RESOURCE_REPORT = os.path.join(BUILD_DIR, "resource_usage.txt")


def _resources(remarks: str):
    """(kernel, VGPRs, AGPRs, scratch bytes per lane, waves per SIMD) from the
    compiler's kernel-resource-usage remarks."""
    out, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            out.append(cur)
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[m.group(1).split()[0]] = int(m.group(2))
    return out


def _compile(src: str):
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = ["hipcc", *HIP_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []),
           "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj, _resources(r.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    kernels = {k["name"]: k for _, res in done for k in res}
    with open(RESOURCE_REPORT, "w") as f:
        f.write("kernel VGPRs AGPRs scratch_bytes_per_lane waves_per_SIMD\n")
        for name in sorted(kernels):
            k = kernels[name]
            f.write(f"{name} {k.get('VGPRs', -1)} {k.get('AGPRs', -1)} {k.get('ScratchSize', -1)} "
                    f"{k.get('Occupancy', -1)}\n")
    for name, budget in VGPR_WATCH.items():
        got = kernels.get(name, {}).get("VGPRs")
        if got is not None and got > budget:
            sys.stderr.write(f"warning: {name} uses {got} VGPRs (measured build: {budget}); "
                             "time it before keeping this change\n")
    tmp = LIB + ".tmp"
    subprocess.run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp],
                   check=True, capture_output=not verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
