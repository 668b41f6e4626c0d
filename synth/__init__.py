"""Seeded synthetic inputs for the routed-MoE layer (shared by tests and bench).

This package holds no arithmetic of the layer itself: it draws numbers and
packs synthetic expert weights the way an offline converter would.  The
generator definitions (counter-based SplitMix64 draws, a 12-uniform
Irwin-Hall normal, uniform variates, per-row absmax quantisation and packing)
are in ``synth.c``; ``synth_gpu.hip`` reproduces the expert records bit for bit
in device memory for the multi-gigabyte weight sets.

Workloads (shapes and distributions of the method's real layer; all seeded):
  tiny     hidden 256, intermediate 128, 8 experts in 2 groups (keep 1 group,
           top-2), 1 shared expert, 4 tokens, bias ~U(-0.1, 0.1)
  decode   hidden 6144, intermediate 2048, 256 experts in 8 groups (keep 4,
           top-8), 1 shared expert, 1 token, bias ~U(-0.1, 0.1)
  verify   same layer, 4 or 16 tokens; the second half of the tokens are copies
           of the first half plus N(0, 0.1^2) noise
  prefill  same layer, 2048 tokens, Zipf-skewed bias (0.5 * rank^-1.1 over a
           seeded permutation of the ranks)
  stack    16 such layers, independent seeds, Zipf-skewed bias, RMSNorm +
           residual between layers, 1 or 8 tokens, int4 or int2 experts
Distributions: tokens ~N(0,1); router weights ~N(0, 0.02^2) fp32; expert
gate/up/down weights ~N(0, 0.02^2) quantised per row to packed int4 (or int2,
int8) with fp32 absmax scales, or per 32-block to MXFP4.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
GPU_LIB_PATH = os.path.join(_HERE, "libsynth_gpu.so")

T_X, T_ROUTER, T_BIAS, T_NOISE, T_ZIPF = 1, 2, 3, 7, 8
SHARED_ID = 0xFFFFFFFF
WEIGHT_SIGMA = 0.02

_lib = None
_glib = None


MXFP4 = -4  # weight-format code: MXFP4 experts (FP4 E2M1 codes, E8M0 scale per 32)
FP8 = -8  # weight-format code: FP8 E4M3 experts (one fp32 scale per 128x128 block)


@dataclass(frozen=True)
class LayerShape:
    hidden: int
    inter: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    n_shared: int = 1
    routed_scaling: float = 2.5
    wbits: int = 4  # 8, 4, 2 (integer codes, fp32 row scales), MXFP4 or FP8

    @property
    def label(self) -> str:
        return {MXFP4: "mxfp4", FP8: "fp8"}.get(self.wbits, f"int{self.wbits}")

    def with_bits(self, wbits: int) -> "LayerShape":
        return LayerShape(self.hidden, self.inter, self.n_experts, self.n_group,
                          self.topk_group, self.top_k, self.n_shared, self.routed_scaling, wbits)


TINY = LayerShape(256, 128, 8, 2, 1, 2)
REAL = LayerShape(6144, 2048, 256, 8, 4, 8)

SEEDS = dict(tiny=100, decode=101, verify=102, prefill=103, stack=104)


def build(gpu: bool = True) -> None:
    src = os.path.join(_HERE, "synth.c")
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                    "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas", src, "-o",
                    LIB_PATH + ".tmp", "-lm"], check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    if gpu:
        gsrc = os.path.join(_HERE, "synth_gpu.hip")
        subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                        "-fhip-fp32-correctly-rounded-divide-sqrt", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", "-fPIC", "-shared", gsrc, "-o",
                        GPU_LIB_PATH + ".tmp"], check=True)
        os.replace(GPU_LIB_PATH + ".tmp", GPU_LIB_PATH)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        u64, u32, i64, c_i, c_f, c_v = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_float, ctypes.c_void_p)
        L.synth_key.argtypes = [u64, u32, u32, u32, u32]
        L.synth_key.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_draw.restype = u64
        L.synth_normal_fill.argtypes = [u64, u64, i64, c_f, c_v]
        L.synth_normal_fill.restype = None
        L.synth_uniform_fill.argtypes = [u64, u64, i64, c_f, c_f, c_v]
        L.synth_uniform_fill.restype = None
        L.synth_blob_bytes.argtypes = [c_i, c_i, c_i]
        L.synth_blob_bytes.restype = ctypes.c_size_t
        L.synth_expert_blob.argtypes = [u64, u32, u32, c_i, c_i, c_i, c_f, c_v]
        L.synth_expert_blob.restype = c_i
        L.synth_weight_row.argtypes = [u64, u32, u32, u32, c_i, c_i, c_f, c_v]
        L.synth_weight_row.restype = None
        _lib = L
    return _lib


def gpu_lib():
    global _glib
    if _glib is None:
        if not os.path.exists(GPU_LIB_PATH):
            raise RuntimeError(f"{GPU_LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(GPU_LIB_PATH)
        L.synth_gpu_expert_blobs.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                             ctypes.c_void_p]
        L.synth_gpu_expert_blobs.restype = ctypes.c_int
        _glib = L
    return _glib


def key(seed, layer, tensor, expert=0, matrix=0) -> int:
    return int(lib().synth_key(seed, layer, tensor, expert, matrix))


def normal(k: int, n: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_fill(k, start, n, sigma, out.ctypes.data)
    return out


def uniform(k: int, n: int, lo: float, hi: float, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_uniform_fill(k, start, n, lo, hi, out.ctypes.data)
    return out


def blob_bytes(shape: LayerShape) -> int:
    return int(lib().synth_blob_bytes(shape.hidden, shape.inter, shape.wbits))


def expert_blob(shape: LayerShape, seed: int, layer: int, expert: int) -> np.ndarray:
    """Packed record of one expert (expert = SHARED_ID for the shared expert)."""
    out = np.empty(blob_bytes(shape), np.uint8)
    rc = lib().synth_expert_blob(seed, layer, expert, shape.hidden, shape.inter, shape.wbits,
                                 WEIGHT_SIGMA, out.ctypes.data)
    if rc:
        raise ValueError("synth_expert_blob rejected the shape")
    return out


def weight_row(seed, layer, expert, matrix, n, row) -> np.ndarray:
    """Float weights (before quantisation) of one row; matrix 0 gate, 1 up, 2 down."""
    out = np.empty(n, np.float32)
    lib().synth_weight_row(seed, layer, expert, matrix, n, row, WEIGHT_SIGMA, out.ctypes.data)
    return out


def expert_blobs_gpu(shape: LayerShape, seed: int, layer: int, expert_ids, out_ptr: int,
                     stride: int, stream: int = 0) -> None:
    """Write the records of ``expert_ids`` to device memory at out_ptr + i*stride."""
    ids = np.ascontiguousarray(np.asarray(expert_ids, np.uint32))
    rc = gpu_lib().synth_gpu_expert_blobs(seed, layer, ids.ctypes.data, ids.size, shape.hidden,
                                          shape.inter, shape.wbits, WEIGHT_SIGMA, out_ptr, stride,
                                          stream)
    if rc:
        raise RuntimeError(f"synth_gpu_expert_blobs failed (rc={rc})")


def router_weights(shape: LayerShape, seed: int, layer: int = 0) -> np.ndarray:
    k = key(seed, layer, T_ROUTER)
    return normal(k, shape.n_experts * shape.hidden, WEIGHT_SIGMA).reshape(
        shape.n_experts, shape.hidden)


def router_bias_uniform(shape: LayerShape, seed: int, layer: int = 0, lo=-0.1, hi=0.1):
    return uniform(key(seed, layer, T_BIAS), shape.n_experts, lo, hi)


def zipf_ranks(n: int, seed: int, layer: int = 0) -> np.ndarray:
    """Seeded permutation of the ranks 1..n (Fisher-Yates on SplitMix64 draws)."""
    k = key(seed, layer, T_ZIPF)
    ranks = np.arange(1, n + 1)
    L = lib()
    for i in range(n - 1, 0, -1):
        j = int(L.synth_draw(k, i) % (i + 1))
        ranks[i], ranks[j] = ranks[j], ranks[i]
    return ranks


def router_bias_zipf(shape: LayerShape, seed: int, layer: int = 0, beta=0.5, exponent=1.1):
    ranks = zipf_ranks(shape.n_experts, seed, layer).astype(np.float64)
    return (beta * ranks ** (-exponent)).astype(np.float32)


def tokens(shape: LayerShape, seed: int, T: int, layer: int = 0, start: int = 0) -> np.ndarray:
    """T tokens ~N(0,1); token i of the stream is the same whatever T is."""
    k = key(seed, layer, T_X)
    return normal(k, T * shape.hidden, 1.0, start * shape.hidden).reshape(T, shape.hidden)


def tokens_perturbed(shape: LayerShape, seed: int, T: int, layer: int = 0, noise=0.1,
                     start: int = 0) -> np.ndarray:
    """First half ~N(0,1); second half = first half + N(0, noise^2)."""
    assert T % 2 == 0
    base = tokens(shape, seed, T // 2, layer, start)
    k = key(seed, layer, T_NOISE)
    eps = normal(k, (T // 2) * shape.hidden, noise, start * shape.hidden).reshape(T // 2, -1)
    return np.concatenate([base, base + eps]).astype(np.float32)
