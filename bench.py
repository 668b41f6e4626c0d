#!/usr/bin/env python3
"""Throughput of the routed-MoE layer step on one MI355X.

A step is one full pass of the layer (router scores and group-limited top-k,
Q8_0 of the hidden state, batch-union grouping, expert gate/up + SwiGLU,
Q8_0 of h, down projection, weighted combine with the shared expert) over one
batch of synthetic tokens, through ``moe_layer`` in libmoe.

Default workload ("decode"): one token per step through one layer at the real
shape (hidden 6144, expert intermediate 2048, 256 routed experts in 8 groups,
top-4 groups, top-8 experts, 1 shared expert, int4 experts with fp32 row
scales, Q8_0 activations).  Every step takes a fresh token, and consecutive
steps cycle over a ring of independently seeded layer instances resident in
HBM, so a step's ~177 MB of weights are not still in the 256 MB last-level
cache from the previous step.

Timing: W untimed warm-up steps, then exactly K steps between two device
synchronisations.  With --graph (default) the K steps are replayed from HIP
graphs captured over blocks of consecutive steps (launch-bound at ~30 us per
step otherwise).  A second, eager pass over the same steps launches every
kernel with HIP events stamped from its own dispatch (hipExtLaunchKernelGGL)
to give per-kernel durations; the dominant kernel's duration gives the
roofline figure.  The CPU baseline is the oracle (plain C, OpenMP) timed on a
bounded sample of the same workload on this host.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / int8 MFMA % (prefill)"
HBM_PEAK_GBPS = 8000.0
INT8_PEAK_TOPS = 5000.0  # dense int8 MFMA, MI355X
# 32-bit vector lane operations per second: 256 CUs x 4 SIMDs x 16 lanes per
# clock at 2.4 GHz (a wave64 VALU instruction issues over 4 clocks)
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
HOST_LINK_PEAK_GBPS = 64.0  # PCIe 5.0 x16, one direction (host to GPU)

WORKLOADS = {
    "decode": dict(T=1, tokens="normal", bias="uniform", seed="decode", ring=8),
    "verify4": dict(T=4, tokens="perturbed", bias="uniform", seed="verify", ring=8),
    "verify16": dict(T=16, tokens="perturbed", bias="uniform", seed="verify", ring=4),
    "prefill": dict(T=2048, tokens="normal", bias="zipf", seed="prefill", ring=2),
    # every token routed to the same 8 experts (their bias raised by 2.0): nine dense
    # GEMMs of 2048 tokens (8 routed + shared), the layer's matrix-core-bound sub-problem
    "prefill_dense": dict(T=2048, tokens="normal", bias="dense", seed="prefill", ring=2),
    # 16 consecutive layers per step (pre-norm residual between them), all resident
    "stack1": dict(T=1, tokens="normal", bias="zipf", seed="stack", ring=16, layers=16),
    "stack8": dict(T=8, tokens="normal", bias="zipf", seed="stack", ring=16, layers=16),
}


ACT_TEXT = {"q8_0": "Q8_0 activations",
            "row": "activations with one scale per row (per token, per token and expert)"}


def describe(name, shape, T, ring, layers=1, top_p=0.0, cache_slots=0, act="q8_0"):
    tp = (f", adaptive expert top-p {top_p:g} (shortest rank-order prefix holding that share of "
          f"the selected scores, weights renormalised)" if 0 < top_p < 1 else "")
    wfmt = ("MXFP4 (FP4 E2M1 codes + an E8M0 scale per 32)" if shape.wbits == -4
            else "FP8 E4M3 (+ an fp32 scale per 128x128 block)" if shape.wbits == -8
            else f"int{shape.wbits} (codes + fp32 row scales)")
    if cache_slots:
        tp += (f"; routed experts in pinned host memory, {cache_slots} of {shape.n_experts} per "
               f"layer cached in HBM (LRU + hot store pinned from recorded usage), misses "
               f"streamed over the host link")
    if layers > 1:
        return (f"{name}: {T} token(s) per step through a stack of {layers} routed-MoE layers "
                f"(independent seeds, Zipf-skewed bias, unit-gain RMSNorm + residual between "
                f"layers; hidden {shape.hidden}, expert intermediate {shape.inter}, "
                f"{shape.n_experts} experts in {shape.n_group} groups, top-{shape.topk_group} "
                f"groups, top-{shape.top_k}, {shape.n_shared} shared expert, {wfmt} "
                f"experts, {ACT_TEXT[act]}{tp})" +
                ("" if cache_slots else ", all layers resident in HBM"))
    return (f"{name}: {T} token(s) per step through one routed-MoE layer (hidden {shape.hidden}, "
            f"expert intermediate {shape.inter}, {shape.n_experts} experts in {shape.n_group} "
            f"groups, top-{shape.topk_group} groups, top-{shape.top_k}, {shape.n_shared} shared "
            f"expert, {wfmt} experts, {ACT_TEXT[act]}{tp}); weights "
            f"cycled over {ring} seeded layer instances" + ("" if cache_slots else " in HBM"))


class Hip:
    """The HIP runtime already loaded by PyTorch (event timing only)."""

    def __init__(self):
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("HIP runtime not loaded")
        L = ctypes.CDLL(path)
        L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                          ctypes.c_void_p]
        L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.L = L

    def event(self):
        e = ctypes.c_void_p()
        rc = self.L.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.L.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, e):
        self.L.hipEventDestroy(ctypes.c_void_p(e))

    def clear_error(self):
        """Reset HIP's last-error state (left set by timing unrecorded events)."""
        self.L.hipGetLastError()


def layer_bytes(shape, T, U, bb):
    """Algorithmic HBM bytes of one step: router matrix and bias, the records of
    the U distinct routed experts and the shared expert, x in, y out."""
    E, H = shape.n_experts, shape.hidden
    return E * H * 4 + E * 4 + (U + shape.n_shared) * bb + 2 * T * H * 4


def gate_up_record_bytes(shape):
    """Bytes of an expert record's gate and up parts (codes and their scales)."""
    H, I = shape.hidden, shape.inter
    if shape.wbits == -4:  # MXFP4: 4-bit codes and one scale byte per 32
        return 2 * I * H // 2 + 2 * I * H // 32
    if shape.wbits == -8:  # FP8: byte codes and one fp32 scale per 128x128 block
        return 2 * I * H + 2 * (I // 128) * (H // 128) * 4
    return 2 * I * H * shape.wbits // 8 + 2 * I * 4


def gate_up_bytes(shape, T, U, small):
    """Algorithmic bytes of one gate/up launch.

    Small-batch path (1..16 tokens): gate and up codes and row scales of the U
    routed experts, Q8_0 of x in, Q8_0 of h out for the T*K routed pairs, and
    the shared expert's fp32 h in / Q8_0 out (its gate/up runs beside the
    selection).  Larger batches: the same for U + shared experts with fp32 h
    out."""
    H, I, K, S = shape.hidden, shape.inter, shape.top_k, shape.n_shared
    per_expert = gate_up_record_bytes(shape)
    q8 = 1 + 4 / 32  # bytes per element of a Q8_0 vector (codes + fp32 block scales)
    x_in = T * H * q8
    if small:
        return U * per_expert + x_in + T * K * I * q8 + S * T * I * (4 + q8)
    return (U + S) * per_expert + x_in + (T * K + T * S) * I * 4


def gate_up_bounds(shape, T, U, pairs, act_row):
    """The prefill gate/up launch at each peak, in seconds: its int8 operations
    (2 per multiply-accumulate) at the MFMA peak, its algorithmic bytes at the
    HBM peak, and for Q8_0 activations its fix-ups (a convert and a
    multiply-add per pair, gate or up row and 32-block) at the VALU rate.
    pairs: routed (token, expert) pairs; the shared expert adds T.  Returns
    (bounds, ops, bytes, fixups)."""
    n_pairs = pairs + T * shape.n_shared
    ops = 2.0 * n_pairs * 2 * shape.inter * shape.hidden
    nbytes = gate_up_bytes(shape, T, U, False)
    fix = 0.0 if act_row else n_pairs * 2 * shape.inter * shape.hidden / 32
    bounds = {"mfma": ops / (INT8_PEAK_TOPS * 1e12), "hbm": nbytes / (HBM_PEAK_GBPS * 1e9),
              "alu": 2.0 * fix / VALU_LANE_OPS}
    return bounds, ops, nbytes, fix


# the sources of the small-batch kernels whose counters profiles/ records
TRAFFIC_SOURCES = ("decode.h", "decode.hip", "common.h", "kernels.h")


def sources_sha256():
    import hashlib
    csrc = os.path.join(ROOT, "int4_routed_expert_moe_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read()
                                   for f in TRAFFIC_SOURCES)).hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the gate/up kernel from the committed rocprofv3
    counter summary (FETCH_SIZE + WRITE_SIZE, calibrated), or None when the
    kernel sources changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"<!-- traffic kernel=gate_up workload=(\S+) src_sha256=([0-9a-f]+) "
                  r"bytes_per_launch=(\d+) -->", open(path).read())
    if not m or m.group(1) != workload:
        return None
    if sources_sha256() != m.group(2):
        return None
    return float(m.group(3))


def cpu_baseline_stack(shape, seed, layers, tokens_fn, T, n_steps, top_p=0.0):
    """Oracle on the first steps of the stack workload (all layers)."""
    import oracle
    import synth
    kw = dict(H=shape.hidden, I=shape.inter, n_experts=shape.n_experts, n_group=shape.n_group,
              topk_group=shape.topk_group, top_k=shape.top_k, scale=shape.routed_scaling,
              wbits=shape.wbits, top_p_value=top_p)
    caches = [dict() for _ in layers]
    shared = [synth.expert_blob(shape, seed, l, synth.SHARED_ID) for l in range(len(layers))]
    spent, done = 0.0, 0
    for i in range(n_steps):
        h = tokens_fn(i)
        t0 = time.perf_counter()
        xn = oracle.rmsnorm(h)
        spent += time.perf_counter() - t0
        for l, (wr, bias) in enumerate(layers):
            idx, _, _ = oracle.route(xn, wr, bias, shape.n_group, shape.topk_group, shape.top_k,
                                     shape.routed_scaling, top_p)
            for e in np.unique(idx[idx >= 0]):  # drawn outside the timed region
                if int(e) not in caches[l]:
                    caches[l][int(e)] = synth.expert_blob(shape, seed, l, int(e))
            t0 = time.perf_counter()
            out = oracle.layer(xn, wr, bias, caches[l].__getitem__, shared[l], residual=h,
                               want_norm=True, **kw)
            spent += time.perf_counter() - t0
            h, xn = out["y"], out["y_norm"]
        done += T
    return dict(value=done / spent, unit="tokens/s", cores=oracle.threads(), kind="oracle",
                sample=f"first {n_steps} step(s) ({done} tokens through all {len(layers)} layers) "
                       f"of the same workload, {spent:.1f} s of oracle time (plain C, OpenMP "
                       f"over output rows; expert records drawn outside the timed region)")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(shape, seed, wr, bias, tokens_fn, T, budget_s, top_p=0.0, act_block=32):
    """Oracle (plain C + OpenMP) on the first steps of the same workload: with
    all its threads, then (a third of the budget) on one thread."""
    import oracle
    import synth
    cache = {}

    def blob_of(e):
        if e not in cache:
            cache[e] = synth.expert_blob(shape, seed, 0, e)
        return cache[e]

    shared = synth.expert_blob(shape, seed, 0, synth.SHARED_ID)
    kw = dict(H=shape.hidden, I=shape.inter, n_experts=shape.n_experts, n_group=shape.n_group,
              topk_group=shape.topk_group, top_k=shape.top_k, scale=shape.routed_scaling,
              wbits=shape.wbits, top_p_value=top_p, act_block=act_block)

    def timed(budget):
        done_tok, spent, steps = 0, 0.0, 0
        while spent < budget and steps < 1024:
            x = tokens_fn(steps)
            idx, _, _ = oracle.route(x, wr, bias, shape.n_group, shape.topk_group, shape.top_k,
                                     shape.routed_scaling, top_p)
            for e in np.unique(idx[idx >= 0]):
                blob_of(int(e))  # drawn outside the timed region
            t0 = time.perf_counter()
            oracle.layer(x, wr, bias, blob_of, shared, **kw)
            spent += time.perf_counter() - t0
            done_tok += x.shape[0]
            steps += 1
        return done_tok, spent, steps

    threads = oracle.threads()
    done_tok, spent, steps = timed(budget_s)
    oracle.set_threads(1)
    d1, s1, n1 = timed(budget_s / 3)
    oracle.set_threads(threads)
    return dict(value=done_tok / spent, unit="tokens/s", cores=threads, kind="oracle",
                value_single_thread=d1 / s1, cpu_model=cpu_model(), host_cpus=os.cpu_count(),
                sample=f"first {steps} step(s) ({done_tok} tokens) of the same workload on layer "
                       f"instance 0, {spent:.1f} s of oracle time on {threads} threads; then the "
                       f"first {n1} step(s) on one thread ({s1:.1f} s) (plain C, OpenMP over "
                       f"output rows; expert records drawn outside the timed region)")


def measured_mfma_peak(torch, moe, dev, n_wg=1024, iters=4000):
    """int8 TOPS of moe_mfma_peak (matrix cores only, 4 waves per SIMD)."""
    out = torch.empty(n_wg * 256, dtype=torch.int32, device=dev)
    moe.mfma_peak(n_wg, 64, out)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ops = moe.mfma_peak(n_wg, iters, out)
    e1.record()
    torch.cuda.synchronize()
    return ops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def measured_read_peak(torch, moe, hip, dev, bufs, nbytes, grids=(2048, 8192, 16384), reps=16):
    """GB/s of moe_read_peak reading nbytes from each of bufs in turn (the
    layer instances' expert records: not in the last-level cache, like the
    step's weights), timed by the kernel's own dispatch as the stages are:
    for each grid size the mean over reps launches after one pass over bufs,
    and the best of the grid sizes (no single one is best at every size)."""
    nbytes = nbytes // 16 * 16
    out = torch.empty(max(grids) * 4, dtype=torch.int32, device=dev)
    best = 0.0
    for n_wg in grids:
        for b in bufs:
            moe.read_peak(b, nbytes, n_wg, out)
        evs = [(hip.event(), hip.event()) for _ in range(reps)]
        for k, (a, z) in enumerate(evs):
            moe.read_peak(bufs[k % len(bufs)], nbytes, n_wg, out, a, z)
        torch.cuda.synchronize()
        ms = [hip.elapsed_ms(a, z) for a, z in evs]
        for a, z in evs:
            hip.destroy(a)
            hip.destroy(z)
        best = max(best, nbytes / (float(np.mean(ms)) * 1e-3) / 1e9)
    return best


def small_phase_bytes(shape, U, bb):
    """Weight bytes each dependent launch of the small-batch step streams: the
    router matrix, the shared expert's gate/up (beside the selection), the U
    routed experts' gate/up, and the down rows of the U routed and the shared
    experts."""
    E, H, S = shape.n_experts, shape.hidden, shape.n_shared
    gu = gate_up_record_bytes(shape)
    down = bb - gu  # the record's down codes and scales
    return [E * H * 4, S * gu, U * gu, (U + S) * down]


def measured_step_floor(torch, moe, stream, dev, bufs, phase_bytes, n_steps=64, reps=8,
                        grids=(2048, 8192)):
    """Microseconds per step of plain streaming reads (moe_read_peak), one
    dependent launch per phase of the step reading that phase's bytes, step i
    from layer instance i mod len(bufs) (phases at disjoint offsets), replayed
    from a HIP graph like the timed steps: the time any design pays whose
    phases are separate launches streaming those bytes at the plain-read rate
    (best of the grid sizes)."""
    out = torch.empty(max(grids) * 4, dtype=torch.int32, device=dev)
    offs = np.concatenate([[0], np.cumsum([(b + 255) // 256 * 256 for b in phase_bytes])])
    best = None
    for n_wg in grids:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n_steps):
                buf = bufs[i % len(bufs)]
                for p, nb in enumerate(phase_bytes):
                    if nb >= 16:
                        moe.read_peak(buf[int(offs[p]):], int(nb) // 16 * 16, n_wg, out)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) / (reps * n_steps) * 1e6
        best = us if best is None else min(best, us)
        del g
    return best


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--wbits", default="4", choices=("8", "4", "2", "mxfp4", "fp8"),
                    help="expert weights: int8/int4/int2 codes with row scales, MXFP4, or FP8 "
                         "E4M3 with 128x128 block scales")
    ap.add_argument("--ring", type=int, default=0,
                    help="layer instances to cycle (0 = the workload's ring; 1 with --cache-slots)")
    ap.add_argument("--act", default="q8_0", choices=("q8_0", "row"),
                    help="activation format: Q8_0 blocks of 32, or one scale per row")
    ap.add_argument("--topp", type=float, default=0.0,
                    help="adaptive expert top-p in (0, 1); 0 = off (plain top-k)")
    ap.add_argument("--cache-slots", type=int, default=0,
                    help="routed experts in pinned host memory, this many per layer cached in "
                         "HBM (0 = every expert resident in HBM)")
    ap.add_argument("--cache-pinned", type=int, default=-1,
                    help="slots pinned from the warm-up's recorded usage (-1 = half)")
    ap.add_argument("--cache-promote", type=int, default=2, help="promotions per layer call")
    ap.add_argument("--cache-wait", action="store_true",
                    help="with --cache-slots: each moe_cache_step waits for its read-back and "
                         "copies (the synchronous cache)")
    ap.add_argument("--lookahead", action="store_true",
                    help="stacks with --cache-slots: route layer l+1 from layer l's input and "
                         "prefetch its predicted experts before layer l runs")
    ap.add_argument("--layers", type=int, default=0,
                    help="layers of a stack workload (0 = the workload's)")
    ap.add_argument("--no-graph", action="store_true", help="launch every step eagerly")
    ap.add_argument("--graph-block", type=int, default=64, help="steps per captured graph")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run a plain elementwise kernel over this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "the layer step runs on one GPU; --gpus must be 1 "
                                   "(sharding it across GPUs is designed, not built)"}))
        sys.exit(2)

    import torch

    import int4_routed_expert_moe_amd as moe
    import synth

    wl = WORKLOADS[args.workload]
    shape = synth.REAL.with_bits({"mxfp4": synth.MXFP4, "fp8": synth.FP8}.get(args.wbits)
                                 or int(args.wbits))
    T = wl["T"]
    NL = wl.get("layers", 1)
    if NL > 1 and args.layers:
        NL = args.layers
    if args.lookahead and (NL < 2 or not args.cache_slots):
        print(json.dumps({"error": "--lookahead needs a stack workload and --cache-slots"}))
        sys.exit(2)
    # with the expert cache one layer instance by default: its steady state needs many calls
    # per layer, and eight interleaved caches each see an eighth of them
    R = NL if NL > 1 else (args.ring or (1 if args.cache_slots else wl["ring"]))
    seed = synth.SEEDS[wl["seed"]]
    K, W = args.steps, args.warmup
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    moe.lib()
    hip = Hip()
    act = moe.ACT_ROW if args.act == "row" else moe.ACT_Q8_0
    cfg = moe.Config.of(shape, args.topp, act)
    bb = moe.blob_bytes(cfg)
    stream = torch.cuda.Stream(device=dev)  # default priority; graphs cannot capture stream 0
    torch.cuda.set_stream(stream)

    # --- resident inputs: R layer instances, tokens for every step ----------
    ring = []
    for l in range(R):
        wr = synth.router_weights(shape, seed, l)
        bias = (synth.router_bias_zipf(shape, seed, l) if wl["bias"] == "zipf"
                else synth.router_bias_uniform(shape, seed, l))
        if wl["bias"] == "dense":
            bias[:shape.top_k] += np.float32(2.0)
        ex = torch.empty(shape.n_experts * bb, dtype=torch.uint8, device=dev)
        sh = torch.empty(bb, dtype=torch.uint8, device=dev)
        synth.expert_blobs_gpu(shape, seed, l, list(range(shape.n_experts)), ex.data_ptr(), bb,
                               stream.cuda_stream)
        synth.expert_blobs_gpu(shape, seed, l, [synth.SHARED_ID], sh.data_ptr(), bb,
                               stream.cuda_stream)
        ring.append(dict(wr=torch.from_numpy(wr).to(dev), bias=torch.from_numpy(bias).to(dev),
                         wr_h=wr, bias_h=bias, ex=ex, sh=sh))
        if args.cache_slots:  # the cold copy in pinned host memory; HBM keeps only the cache
            torch.cuda.synchronize()
            host = torch.empty(ex.numel(), dtype=torch.uint8, pin_memory=True)
            host.copy_(ex)
            ring[-1].update(host=host, ex=None)
            del ex
            torch.cuda.empty_cache()

    def tokens_for(step):
        if wl["tokens"] == "perturbed":
            return synth.tokens_perturbed(shape, seed, T, start=step * (T // 2))
        return synth.tokens(shape, seed, T, start=step * T)

    n_tok_steps = W + K
    if wl["tokens"] == "perturbed":
        xs = np.stack([tokens_for(i) for i in range(n_tok_steps)])
    else:
        xs = synth.tokens(shape, seed, n_tok_steps * T).reshape(n_tok_steps, T, shape.hidden)
    x_all = torch.from_numpy(xs).to(dev)
    idx_all = torch.zeros((n_tok_steps, NL, T, shape.top_k), dtype=torch.int32, device=dev)
    y = torch.empty((T, shape.hidden), dtype=torch.float32, device=dev)
    hbuf = [torch.empty((T, shape.hidden), dtype=torch.float32, device=dev) for _ in range(2)]
    xnbuf = [torch.empty((T, shape.hidden), dtype=torch.float32, device=dev) for _ in range(2)]
    ws = torch.zeros(moe.layer_workspace(cfg, T), dtype=torch.uint8, device=dev)
    ws_route = torch.zeros(moe.route_workspace(cfg, T), dtype=torch.uint8, device=dev)
    # predictions of layer l+1's routing (lookahead), kept per step for their accuracy
    pred_all = torch.full((n_tok_steps, NL, T, shape.top_k), -1, dtype=torch.int32, device=dev)
    pred_w = torch.empty((T, shape.top_k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    L = moe.lib()
    c_cfg = moe.Config.c(cfg)

    def call_layer(r, x_ptr, res_ptr, y_ptr, yn_ptr, idx_ptr, events):
        if "cache" in r:  # records through the cache's table, then the cache's bookkeeping
            rc = L.moe_layer_ptrs(ctypes.byref(c_cfg), T, x_ptr, r["wr"].data_ptr(),
                                  r["bias"].data_ptr(), r["cache"].table.data_ptr(),
                                  r["sh"].data_ptr(), res_ptr, y_ptr, yn_ptr, 1e-5, idx_ptr, None,
                                  ws.data_ptr(), ws.numel(), events, None, stream.cuda_stream)
            if rc == 0:
                rc = L.moe_cache_step(r["cache"]._h, idx_ptr, T * shape.top_k,
                                      int(args.cache_wait), stream.cuda_stream)
        else:
            rc = L.moe_layer(ctypes.byref(c_cfg), T, x_ptr, r["wr"].data_ptr(),
                             r["bias"].data_ptr(), r["ex"].data_ptr(), r["sh"].data_ptr(),
                             res_ptr, y_ptr, yn_ptr, 1e-5, idx_ptr, None, ws.data_ptr(),
                             ws.numel(), events, None, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"moe_layer failed: {L.moe_last_error().decode()}")

    def run_step(i, events=None):
        """events: None, or one moe_events per layer."""
        ev = (lambda l: None) if events is None else (lambda l: ctypes.byref(events[l]))
        if NL == 1:
            call_layer(ring[i % R], x_all[i].data_ptr(), None, y.data_ptr(), None,
                       idx_all[i, 0].data_ptr(), ev(0))
            return
        # pre-norm stack: xn = RMSNorm(h); h <- h + MoE_l(xn), the layer also
        # writes RMSNorm of the new h for the next layer
        rc = L.moe_rmsnorm(T, shape.hidden, x_all[i].data_ptr(), xnbuf[0].data_ptr(), 1e-5,
                           stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"moe_rmsnorm failed: {L.moe_last_error().decode()}")
        h_ptr = x_all[i].data_ptr()
        for l in range(NL):
            a, b = l % 2, (l + 1) % 2
            if args.lookahead:
                if l + 1 < NL:  # layer l+1 routed from layer l's input, its experts prefetched
                    nxt = ring[l + 1]
                    pred_idx = pred_all[i, l + 1]
                    rc = L.moe_route(ctypes.byref(c_cfg), T, xnbuf[a].data_ptr(),
                                     nxt["wr"].data_ptr(), nxt["bias"].data_ptr(),
                                     pred_idx.data_ptr(), pred_w.data_ptr(), ws_route.data_ptr(),
                                     ws_route.numel(), stream.cuda_stream)
                    if rc == 0:
                        rc = L.moe_cache_prefetch(nxt["cache"]._h, pred_idx.data_ptr(),
                                                  T * shape.top_k, stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"lookahead failed: {L.moe_last_error().decode()}")
                rc = L.moe_cache_publish(ring[l]["cache"]._h, stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"moe_cache_publish failed: {L.moe_last_error().decode()}")
            call_layer(ring[l], xnbuf[a].data_ptr(), h_ptr, hbuf[b].data_ptr(),
                       xnbuf[b].data_ptr(), idx_all[i, l].data_ptr(), ev(l))
            h_ptr = hbuf[b].data_ptr()

    if args.copy_mb:  # a plain streaming kernel of known size, for hardware-counter calibration
        n = args.copy_mb << 20  # reads n bytes, writes n bytes
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # --- warm-up ------------------------------------------------------------
    if args.cache_slots:
        # the learning cache: an LRU-only pass records usage, then each layer's
        # cache is rebuilt with its hottest experts pinned
        S = min(args.cache_slots, shape.n_experts)
        P = S // 2 if args.cache_pinned < 0 else min(args.cache_pinned, S)
        for r in ring:
            r["cache"] = moe.ExpertCache(cfg, r["host"], S, 0, args.cache_promote,
                                         T * shape.top_k, device=dev)
        for i in range(W):
            run_step(i)
        torch.cuda.synchronize()
        for r in ring:
            usage = r["cache"].usage()
            r["cache"].close()
            r["cache"] = moe.ExpertCache(cfg, r["host"], S, P, args.cache_promote,
                                         T * shape.top_k, usage=usage, device=dev)
    for i in range(W):
        run_step(i)
    torch.cuda.synchronize()
    cache0 = [r["cache"].stats() for r in ring] if args.cache_slots else None

    # --- timed region ---------------------------------------------------------
    use_graph = not args.no_graph and not args.cache_slots  # the cache steps on the host
    graphs = []
    if use_graph:
        B = max(1, min(args.graph_block, K))
        for b0 in range(W, W + K, B):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(b0, min(b0 + B, W + K)):
                    run_step(i)
            graphs.append(g)
        for g in graphs:  # one untimed replay of every graph
            g.replay()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if use_graph:
        for g in graphs:
            g.replay()
    else:
        for i in range(W, W + K):
            run_step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec = t1 - t0
    cache1 = [r["cache"].stats() for r in ring] if args.cache_slots else None

    # --- spread: the timed steps again, in >= 50 blocks timed on the stream ---
    quant = None
    if use_graph:
        qb = max(1, min(B, K // 50))
        qgraphs = []
        for b0 in range(W, W + K - qb + 1, qb):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(b0, b0 + qb):
                    run_step(i)
            qgraphs.append(g)
        for g in qgraphs:
            g.replay()
        torch.cuda.synchronize()
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(qgraphs) + 1)]
        marks[0].record(stream)
        for g, m in zip(qgraphs, marks[1:]):
            g.replay()
            m.record(stream)
        torch.cuda.synchronize()
        per = np.array([marks[i].elapsed_time(marks[i + 1]) / qb for i in range(len(qgraphs))])
        quant = {"p10": float(np.percentile(per, 10)), "p50": float(np.median(per)),
                 "p90": float(np.percentile(per, 90)), "samples": len(per),
                 "steps_per_sample": qb}
        del qgraphs

    # --- per-kernel durations (eager pass, events stamped by the dispatch) ----
    n_ev = max(1, min(K, 256 // NL))
    stage_names = list(moe.STAGES)
    evs = []
    for i in range(n_ev):
        per_layer = []
        for l in range(NL):
            me = moe.MoeEvents()
            for s in range(len(stage_names)):
                me.start[s] = hip.event()
                me.stop[s] = hip.event()
            per_layer.append(me)
        evs.append(per_layer)
    torch.cuda.synchronize()
    for j in range(n_ev):
        run_step(W + j, evs[j])
    torch.cuda.synchronize()
    stage_ms = {}
    for s, name in enumerate(stage_names):
        try:  # stages the chosen path did not launch have unrecorded events
            v = [hip.elapsed_ms(me.start[s], me.stop[s]) for per_layer in evs for me in per_layer]
        except RuntimeError:
            continue
        stage_ms[name] = float(np.mean(v))  # per layer
    for per_layer in evs:
        for me in per_layer:
            for s in range(len(stage_names)):
                hip.destroy(me.start[s])
                hip.destroy(me.stop[s])
    hip.clear_error()

    # --- work accounting ------------------------------------------------------
    idx_h = idx_all.cpu().numpy()

    def lookahead_accuracy():
        """Share of layer l+1's routed experts (l >= 0) that the prediction
        from layer l's input named, over the timed steps."""
        if not args.lookahead:
            return None
        pr = pred_all.cpu().numpy()
        got = tot = 0
        for i in range(W, W + K):
            for l in range(1, NL):
                for t in range(T):
                    real = set(idx_h[i, l, t][idx_h[i, l, t] >= 0].tolist())
                    got += len(real & set(pr[i, l, t].tolist()))
                    tot += len(real)
        return got / max(tot, 1)

    def distinct(v):  # routed experts of one step (-1: ranks dropped by top-p)
        return np.unique(v[v >= 0]).size

    U_l = [float(np.mean([distinct(idx_h[i, l]) for i in range(W, W + K)])) for l in range(NL)]
    pairs = float(np.mean([(idx_h[i] >= 0).sum() for i in range(W, W + K)])) / NL
    U = float(np.mean(U_l))
    step_bytes = sum(layer_bytes(shape, T, u, bb) for u in U_l)
    fp8 = shape.wbits == synth.FP8  # otherwise vector kernels (no matrix-core path)
    # the layer's small-batch path (four kernels) records no separate Q8_0 stage
    small = T <= 16 and "quant" not in stage_ms
    dom_sec = stage_ms["gate_up"] * 1e-3
    cache_info = None
    step_floor = None
    if args.cache_slots:
        d = {k: sum(c1[k] - c0[k] for c0, c1 in zip(cache0, cache1))
             for k in ("steps", "routed", "hits", "misses", "promotions", "bytes_copied",
                       "prefetched")}
        calls = max(d["steps"], 1)  # layer calls accounted in the timed region
        miss_bytes = d["misses"] * bb  # a missed record is streamed once over the host link
        link = (miss_bytes + d["bytes_copied"]) / calls * (K * NL) / sec / 1e9
        cache_info = {"slots_per_layer": min(args.cache_slots, shape.n_experts),
                      "pinned_per_layer": (min(args.cache_slots, shape.n_experts) // 2
                                           if args.cache_pinned < 0 else args.cache_pinned),
                      "hbm_resident_fraction": min(args.cache_slots, shape.n_experts)
                      / shape.n_experts,
                      "hit_rate": d["hits"] / max(d["routed"], 1),
                      "misses_per_layer_call": d["misses"] / calls,
                      "promotions_per_layer_call": d["promotions"] / calls,
                      "prefetches_per_layer_call": d["prefetched"] / calls,
                      "lookahead": bool(args.lookahead),
                      "prediction_accuracy": lookahead_accuracy(),
                      "synchronous_steps": bool(args.cache_wait),
                      "host_link_gbps": link}
    if args.cache_slots:  # bound by the host link: missed records + promotion copies
        roof = {"bound": "host-link", "kernel": "whole step (misses stream over the host link)",
                "achieved": cache_info["host_link_gbps"], "peak": HOST_LINK_PEAK_GBPS,
                "unit": "GB/s", "frac": cache_info["host_link_gbps"] / HOST_LINK_PEAK_GBPS,
                "traffic": None}
    elif small or fp8:  # HBM-bound GEMV: algorithmic bytes of the gate/up launch
        dom = ("gate_up (routed FP8 expert gate/up + SwiGLU + Q8_0 of h, exact block dots)"
               if fp8 and small else
               "gate_up (FP8 expert gate/up + SwiGLU, exact block dots)" if fp8 else
               "gate_up (routed expert gate/up + SwiGLU + Q8_0 of h)")
        dom_bytes = float(np.mean([gate_up_bytes(shape, T, u, small) for u in U_l]))
        roof = {"bound": "hbm", "kernel": dom, "achieved": dom_bytes / dom_sec / 1e9,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
        roof["frac"] = roof["achieved"] / HBM_PEAK_GBPS
        # counters were taken on the int4 workload without top-p
        roof["traffic"] = (measured_traffic(args.workload)
                           if args.wbits == "4" and not args.topp else None)
        roof.update(bytes_per_launch=dom_bytes, launch_us=dom_sec * 1e6)
        # the same byte count read plainly (moe_read_peak): the HBM rate this
        # chip reaches for a read of that size
        pk = measured_read_peak(torch, moe, hip, dev, [r["ex"] for r in ring], int(dom_bytes))
        roof["achievable_peak"] = pk
        roof["frac_of_achievable"] = roof["achieved"] / pk
        if small and NL == 1 and not fp8 and use_graph:
            # the step's dependent launches as plain reads of their bytes
            phases = small_phase_bytes(shape, U, bb)
            floor_us = measured_step_floor(torch, moe, stream, dev, [r["ex"] for r in ring],
                                           phases)
            step_floor = {"phase_bytes": phases, "floor_us": floor_us,
                          "step_us": sec / K * 1e6, "frac": floor_us / (sec / K * 1e6)}
    else:  # grouped GEMMs: the gate/up launch against its matrix-core, HBM and fix-up bounds
        fmt = "per-row activation scales" if args.act == "row" else "Q8_0 activations"
        dom = f"gate_up (grouped {shape.label} x int8 MFMA GEMM, {fmt}, + SwiGLU)"
        # algorithmic bytes: every used expert's gate and up once, activations in, h out
        gu_bounds, ops, gu_bytes, gu_fix = gate_up_bounds(shape, T, U, pairs, args.act == "row")
        mfma_tops = ops / dom_sec / 1e12
        bound = max(gu_bounds, key=gu_bounds.get)
        if bound == "mfma":
            roof = {"bound": "mfma", "kernel": dom, "achieved": mfma_tops,
                    "peak": INT8_PEAK_TOPS, "unit": "TFLOP/s",
                    "note": "int8 operations (2 per multiply-accumulate) against the dense "
                            "int8 MFMA peak"}
        elif bound == "hbm":
            roof = {"bound": "hbm", "kernel": dom, "achieved": gu_bytes / dom_sec / 1e9,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "note": "algorithmic bytes (each used expert's gate and up once) against "
                            "the HBM peak: with many experts per step the weights outweigh "
                            "the matrix-core work"}
        else:
            roof = {"bound": "alu", "kernel": dom, "achieved": 2.0 * gu_fix / dom_sec / 1e12,
                    "peak": VALU_LANE_OPS / 1e12, "unit": "T VALU lane-ops/s",
                    "note": "the Q8_0 fix-ups alone (a convert and a multiply-add per pair, "
                            "row and 32-block) against 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = None
        roof.update(ops_per_launch=ops, bytes_per_launch=gu_bytes, launch_us=dom_sec * 1e6,
                    bounds_us={k: v * 1e6 for k, v in gu_bounds.items()})
        # the metric's int8 MFMA fraction, also against the int8 MFMA rate a
        # matrix-core-only loop reaches here
        roof["mfma_frac"] = mfma_tops / INT8_PEAK_TOPS
        pk = measured_mfma_peak(torch, moe, dev)
        roof["achievable_peak"] = pk
        roof["mfma_frac_of_achievable"] = mfma_tops / pk
        if "down" in stage_ms:  # the down projection: half the operations of gate/up
            roof["down_mfma_frac"] = ops / 2 / (stage_ms["down"] * 1e-3) / 1e12 / INT8_PEAK_TOPS
        # Q8_0: every (pair, output row, 32-block) of gate, up and down takes a
        # convert and a multiply-add after its block dot (the activation scale
        # changes every 32 codes); with one scale per row there is no fix-up
        n_pairs = pairs + T * shape.n_shared
        fix = (0.0 if args.act == "row" else
               n_pairs * 3 * shape.inter * shape.hidden / 32)
        valu_s = 2.0 * fix / VALU_LANE_OPS
        roof["valu_fixup"] = {"fixups": fix, "lane_ops": 2.0 * fix,
                              "peak_lane_ops_per_s": VALU_LANE_OPS, "bound_us": valu_s * 1e6}
        # whole step against the largest of its HBM, matrix-core and fix-up bounds
        bounds = {"hbm": step_bytes / (HBM_PEAK_GBPS * 1e9),
                  "mfma": 1.5 * ops / (INT8_PEAK_TOPS * 1e12), "alu": valu_s}
        roof["step_bound"] = max(bounds, key=bounds.get)
        roof["step_bounds_us"] = {k: v * 1e6 for k, v in bounds.items()}
        roof["step_frac_of_bound"] = max(bounds.values()) / (sec / K)

    out = {
        "metric": METRIC,
        "value": K * T / sec,  # tokens through the whole step (all layers of a stack)
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": sec / K * 1e3,
        "step_ms_quantiles": quant,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp4e2m1xi8->i32" if shape.wbits == -4 else "fp8e4m3xi8->i32"
                  if shape.wbits == -8 else f"i{shape.wbits}xi8->i32")
                 + ("" if args.act == "q8_0" else " (per-row activation scales)"),
        "data": "synthetic",
        "config": {"workload": describe(args.workload, shape, T, R, NL, args.topp,
                                        min(args.cache_slots, shape.n_experts), args.act),
                   "tokens_per_step": T, "layers_per_step": NL, "layer_instances": R,
                   "hip_graph": use_graph, "top_p": args.topp or None,
                   "distinct_routed_experts_per_step": U,
                   "routed_pairs_per_layer": pairs},
        "hbm_gbps": step_bytes / (sec / K) / 1e9,
        "hbm_frac": step_bytes / (sec / K) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": step_bytes,
        "stage_us": {k: round(v * 1e3, 2) for k, v in stage_ms.items()},
        "roofline": roof,
    }
    if step_floor:
        out["step_floor"] = step_floor
    if cache_info:
        out["cache"] = cache_info
    if not args.no_cpu:
        if NL > 1:
            out["cpu_baseline"] = cpu_baseline_stack(shape, seed,
                                                     [(r["wr_h"], r["bias_h"]) for r in ring],
                                                     tokens_for, T, 2, args.topp)
        else:
            r0 = ring[0]
            out["cpu_baseline"] = cpu_baseline(shape, seed, r0["wr_h"], r0["bias_h"], tokens_for,
                                               T, args.cpu_budget, args.topp, act)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
