"""Stacks of routed-MoE layers with a pre-norm residual between them (the
16-layer decode stack workload; reading R11): every layer through the C ABI
on the GPU, checked against the CPU oracle.

- teacher-forced: each layer's own GPU input (RMSNorm'd x and residual h) is
  fed to the oracle layer; indices and weights bit-exact, outputs within
  2e-3 * RMS;
- free-running: the oracle runs the whole chain from the same tokens.  The
  two chains' layer inputs then differ by rounding, and a layer has two
  discontinuities, the top-k selection and the Q8_0 rounding of its input.
  A token may take a different discrete path only where the inputs the two
  chains actually reached put the oracle within reach of one of them: a
  selection margin (K-th vs (K+1)-th biased score, or TG-th vs (TG+1)-th
  group score, fp64) no larger than the scores can move between the two
  inputs (2 * max_e |sb_gpu - sb_oracle| for the pick, 4 * for the group
  score, a sum of two), or a differing Q8_0 code whose oracle-side value
  x/d is no farther from a rounding boundary than the GPU-side one.  Such
  tokens are dropped from later comparisons; on every other token the two
  chains' inputs must stay within (layer + 1) * 2e-3 * RMS and the final
  outputs must match.
"""
import numpy as np
import pytest
import torch

import int4_routed_expert_moe_amd as moe
import oracle
import synth
from _inputs import DeviceLayer, assert_close_rms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


def h(t):
    return t.detach().cpu().numpy()


def gpu_stack(layers, x, dev):
    s = layers[0].shape
    cfg = moe.Config.of(s)
    T = x.shape[0]
    h_d = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    xn_d = moe.rmsnorm(h_d)
    ins, idxs, ws = [], [], []
    for lay in layers:
        ins.append((h(h_d), h(xn_d)))
        idx_d = torch.empty((T, s.top_k), dtype=torch.int32, device=dev)
        w_d = torch.empty((T, s.top_k), dtype=torch.float32, device=dev)
        h_d, xn_d = moe.layer(cfg, xn_d, lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                              residual=h_d, want_norm=True, idx_out=idx_d, w_out=w_d)
        idxs.append(h(idx_d))
        ws.append(h(w_d))
    return ins, idxs, ws, (h(h_d), h(xn_d))


def teacher_forced(layers, ins, idxs, ws, last):
    outs = ins[1:] + [last]
    for l, lay in enumerate(layers):
        h_in, xn_in = ins[l]
        ref = lay.oracle_layer(xn_in, residual=h_in, want_norm=True)
        assert np.array_equal(ref["idx"], idxs[l]), f"layer {l}"
        assert np.array_equal(ref["w"], ws[l]), f"layer {l}"
        assert_close_rms(outs[l][0], ref["y"], 2e-3, f"layer {l} h")
        assert_close_rms(outs[l][1], ref["y_norm"], 2e-3, f"layer {l} xn")


def q8_units(x, d):
    """x / d per element of each 32-block (0 where the block is zero), fp64."""
    dd = np.repeat(np.asarray(d, np.float64), 32, axis=-1)
    return np.where(dd > 0, np.asarray(x, np.float64) / np.where(dd > 0, dd, 1.0), 0.0)


def free_running(layers, x, idxs, last, gpu_ins):
    s = layers[0].shape
    hh = np.asarray(x, np.float32)
    xn = oracle.rmsnorm(hh)
    flipped = set()
    for l, lay in enumerate(layers):
        xg = gpu_ins[l][1]  # the GPU chain's input to layer l
        for t in range(x.shape[0]):
            if t not in flipped:
                rms = np.sqrt(np.mean(np.asarray(xn[t], np.float64) ** 2))
                assert np.max(np.abs(xg[t] - xn[t])) <= (l + 1) * 2e-3 * rms, (l, t)
        q_o, d_o = oracle.q8_0(xn)
        q_g, d_g = oracle.q8_0(xg)
        u_o, u_g = q8_units(xn, d_o), q8_units(xg, d_g)
        dist = np.abs(np.abs(u_o) - np.floor(np.abs(u_o)) - 0.5)  # to the nearest x.5
        _, sb_o = oracle.router_scores(xn, lay.wr, lay.bias)
        _, sb_g = oracle.router_scores(xg, lay.wr, lay.bias)
        ref = lay.oracle_layer(xn, residual=hh, want_norm=True)
        for t in range(x.shape[0]):
            if t in flipped:
                continue
            diff = q_o[t] != q_g[t]
            if diff.any():  # a boundary lies between the two sides' x/d
                reach = np.abs(u_g[t] - u_o[t]) + 1e-6
                assert np.all(dist[t][diff] <= reach[diff]), \
                    (l, t, "Q8_0 code away from a boundary", dist[t][diff], reach[diff])
                flipped.add(t)
                continue
            if not np.array_equal(ref["idx"][t], idxs[l][t]):
                delta = float(np.max(np.abs(sb_g[t].astype(np.float64) - sb_o[t])))
                slack = 2.0 ** -22  # fp32 rounding of the scores
                m = ref["margin"][t]
                assert m[0] <= 2 * delta + slack or m[1] <= 4 * delta + slack, \
                    (l, t, "selection flip with margins", m, "score moves", delta)
                flipped.add(t)
        hh, xn = ref["y"], ref["y_norm"]
    keep = [t for t in range(x.shape[0]) if t not in flipped]
    assert len(keep) * 2 > x.shape[0], f"{len(flipped)} of {x.shape[0]} tokens diverged"
    assert_close_rms(last[0][keep], hh[keep], 2e-3, "final h")
    assert_close_rms(last[1][keep], xn[keep], 2e-3, "final xn")
    return len(flipped)


def test_stack_tiny_16_layers(dev):
    layers = [DeviceLayer(synth.TINY, synth.SEEDS["stack"], layer=l, bias="zipf")
              for l in range(16)]
    x = synth.tokens(synth.TINY, synth.SEEDS["stack"], 4)
    ins, idxs, ws, last = gpu_stack(layers, x, dev)
    teacher_forced(layers, ins, idxs, ws, last)
    assert free_running(layers, x, idxs, last, ins) == 0


def test_stack_tiny_verify_batch(dev):
    layers = [DeviceLayer(synth.TINY, synth.SEEDS["stack"], layer=l, bias="zipf")
              for l in range(4)]
    x = synth.tokens(synth.TINY, synth.SEEDS["stack"], 8, start=100)
    ins, idxs, ws, last = gpu_stack(layers, x, dev)
    teacher_forced(layers, ins, idxs, ws, last)
    free_running(layers, x, idxs, last, ins)


_stacks = {}


def real_stack(bits):
    """16 real-shape layers (independent seeds, Zipf-skewed bias), kept for the
    module: 77.9 GB of int4 records (39.1 GB int2) in HBM."""
    if bits not in _stacks:
        _stacks.clear()
        shape = synth.REAL.with_bits(bits)
        _stacks[bits] = [DeviceLayer(shape, synth.SEEDS["stack"], layer=l, bias="zipf")
                         for l in range(16)]
    return _stacks[bits]


def teardown_module(module):
    _stacks.clear()


@pytest.mark.parametrize("bits,T", [(4, 1), (4, 8), (2, 1), (2, 8)])
def test_stack_real_16_layers(dev, bits, T):
    """The 16-layer stack at the real shape, decode at batch 1 and 8, int4 and
    int2, teacher-forced and free-running."""
    layers = real_stack(bits)
    x = synth.tokens(layers[0].shape, synth.SEEDS["stack"], T, start=5 * T)
    ins, idxs, ws, last = gpu_stack(layers, x, dev)
    teacher_forced(layers, ins, idxs, ws, last)
    free_running(layers, x, idxs, last, ins)
