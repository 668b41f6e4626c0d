"""Stacks of routed-MoE layers with a pre-norm residual between them (the
16-layer decode stack workload; reading R11): every layer through the C ABI
on the GPU, checked against the CPU oracle.

- teacher-forced: each layer's own GPU input (RMSNorm'd x and residual h) is
  fed to the oracle layer; indices bit-exact, outputs within 2e-3 * RMS;
- free-running: the oracle runs the whole chain from the same tokens.  Layer
  inputs then differ by the per-layer error (teacher-forced bound: 2e-3 *
  RMS, which the chain can add up layer after layer), and the layer has two
  discontinuities: the top-k selection and the Q8_0 rounding of its input.
  A token may take a different discrete path only where the oracle sits at
  one of them: a selection margin (K-th vs (K+1)-th biased score, or TG-th
  vs (TG+1)-th group score, fp64) below 1e-5, or a differing Q8_0 code whose
  unrounded value x/d is within (layers so far + 1) * 2e-3 * RMS(x) / d code
  units of a rounding boundary.  Such tokens are dropped from later
  comparisons; every other token must match.
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


def q8_boundary_distance(x, d):
    """Distance, in code units, of |x|/d from the nearest half-integer."""
    v = np.abs(np.asarray(x, np.float64)) / np.repeat(np.where(d > 0, d, 1.0), 32, axis=-1)
    return np.abs(v - np.floor(v) - 0.5)


def free_running(layers, x, idxs, last, gpu_ins):
    hh = np.asarray(x, np.float32)
    xn = oracle.rmsnorm(hh)
    flipped = set()
    for l, lay in enumerate(layers):
        q_o, d_o = oracle.q8_0(xn)
        q_g, _ = oracle.q8_0(gpu_ins[l][1])  # the GPU chain's layer input
        dist = q8_boundary_distance(xn, d_o)
        # how far the chains' inputs may be apart here, in code units of each block
        slack = (l + 1) * 2e-3 * np.sqrt(np.mean(np.asarray(xn, np.float64) ** 2, axis=1))
        reach = slack[:, None] / np.repeat(np.where(d_o > 0, d_o, np.inf), 32, axis=-1)
        ref = lay.oracle_layer(xn, residual=hh, want_norm=True)
        for t in range(x.shape[0]):
            if t in flipped:
                continue
            diff = q_o[t] != q_g[t]
            if diff.any():
                assert np.all(dist[t][diff] <= reach[t][diff]), \
                    (l, t, "Q8_0 code away from a boundary", dist[t][diff], reach[t][diff])
                flipped.add(t)
                continue
            if not np.array_equal(ref["idx"][t], idxs[l][t]):
                assert min(abs(ref["margin"][t, 0]), abs(ref["margin"][t, 1])) < 1e-5, (l, t)
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


def test_stack_real_int4_batch8(dev):
    layers = [DeviceLayer(synth.REAL, synth.SEEDS["stack"], layer=l, bias="zipf")
              for l in range(3)]
    x = synth.tokens(synth.REAL, synth.SEEDS["stack"], 8)
    ins, idxs, ws, last = gpu_stack(layers, x, dev)
    teacher_forced(layers, ins, idxs, ws, last)
    free_running(layers, x, idxs, last, ins)


def test_stack_real_int2_decode(dev):
    shape = synth.REAL.with_bits(2)
    layers = [DeviceLayer(shape, synth.SEEDS["stack"], layer=l, bias="zipf") for l in range(2)]
    x = synth.tokens(shape, synth.SEEDS["stack"], 2, start=5)
    ins, idxs, ws, last = gpu_stack(layers, x, dev)
    teacher_forced(layers, ins, idxs, ws, last)
    free_running(layers, x, idxs, last, ins)
