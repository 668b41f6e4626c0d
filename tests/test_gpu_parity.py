"""GPU parity: every libmoe call against the CPU oracle on seeded inputs.

Bar: integer results (Q8_0 codes and scales, selected experts, grouping,
int32 block dots) bit-exact; the router weights bit-exact (same fp32 steps);
float layer outputs within max|err| <= 2e-3 * RMS(oracle output).
Where fp32 decides an integer from a value the two sides compute differently
(the Q8_0 of the SwiGLU output h), the oracle re-takes that decision on the
GPU's own h in the same precision and must agree bit for bit.
"""
import json
import os

import numpy as np
import pytest

import int4_routed_expert_moe_amd as moe
import oracle
import synth
from _inputs import DeviceLayer, assert_close_rms

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def tiny(dev):
    return DeviceLayer(synth.TINY, synth.SEEDS["tiny"])


@pytest.fixture(scope="module")
def real(dev):
    return DeviceLayer(synth.REAL, synth.SEEDS["decode"])


def to_d(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def h(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ------------------------------------------------------------------ generator

def test_gpu_generator_matches_host(dev):
    for shape in (synth.TINY, synth.REAL, synth.REAL.with_bits(2), synth.REAL.with_bits(8),
                  synth.REAL.with_bits(synth.MXFP4), synth.TINY.with_bits(synth.MXFP4)):
        bb = synth.blob_bytes(shape)
        ids = [0, 3, synth.SHARED_ID]
        out = torch.empty(len(ids) * bb, dtype=torch.uint8, device=dev)
        synth.expert_blobs_gpu(shape, 11, 2, ids, out.data_ptr(), bb,
                               torch.cuda.current_stream().cuda_stream)
        got = h(out).reshape(len(ids), bb)
        for i, e in enumerate(ids):
            assert np.array_equal(got[i], synth.expert_blob(shape, 11, 2, e)), (shape, e)


# ------------------------------------------------------------------ Q8_0

@pytest.mark.parametrize("rows,n", [(1, 6144), (4, 256), (37, 2048), (3, 32), (2048, 6144)])
def test_quant_act_bit_exact(dev, rows, n):
    x = synth.normal(synth.key(5, rows, n), rows * n).reshape(rows, n)
    x *= np.exp2(synth.normal(synth.key(6, rows, n), rows).astype(np.float32) * 4)[:, None]
    x[0, :32] = 0.0
    q, d = moe.quant_act(to_d(x, dev))
    qo, do = oracle.q8_0(x)
    assert np.array_equal(h(q), qo)
    assert np.array_equal(h(d), do)


def test_quant_act_hand_blocks_and_extremes(dev):
    blocks = json.load(open(os.path.join(GOLDEN, "q8_0_blocks.json")))["blocks"]
    rows = []
    for b in blocks:
        x = np.zeros(32, np.float32)
        for k, v in b["x"].items():
            x[int(k)] = v
        rows.append(x)
    rng = np.random.default_rng(0)
    rows.append((rng.integers(-127, 128, 32)).astype(np.float32))
    rows.append(np.full(32, 3.0e38, np.float32) * rng.choice([-1, 1], 32).astype(np.float32))
    rows.append((rng.standard_normal(32) * 1e-30).astype(np.float32))
    rows.append(np.linspace(-1, 1, 32, dtype=np.float32))
    x = np.stack(rows)
    q, d = moe.quant_act(to_d(x, dev))
    qo, do = oracle.q8_0(x)
    assert np.array_equal(h(q), qo)
    assert np.array_equal(h(d), do)
    for i, b in enumerate(blocks):
        assert h(d)[i, 0] == np.float32(b["d"])


# ------------------------------------------------------------------ router

def _route_check(layer, x, dev, top_p=0.0):
    s = layer.shape
    cfg = moe.Config.of(s, top_p)
    idx, w = moe.route(cfg, to_d(x, dev), layer.wr_d, layer.bias_d)
    ri, rw, margin = oracle.route(x, layer.wr, layer.bias, s.n_group, s.topk_group, s.top_k,
                                  s.routed_scaling, top_p)
    assert np.array_equal(h(idx), ri)
    assert np.array_equal(h(w).view(np.uint32), rw.view(np.uint32))
    return margin


def test_route_tiny(dev, tiny):
    _route_check(tiny, synth.tokens(synth.TINY, synth.SEEDS["tiny"], 4), dev)


@pytest.mark.parametrize("T,start", [(1, 0), (1, 1), (1, 7), (8, 100)])
def test_route_decode(dev, real, T, start):
    _route_check(real, synth.tokens(synth.REAL, synth.SEEDS["decode"], T, start=start), dev)


@pytest.mark.parametrize("T", [4, 16])
def test_route_verify(dev, real, T):
    _route_check(real, synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], T), dev)


def test_route_prefill_zipf(dev):
    lay = DeviceLayer(synth.REAL, synth.SEEDS["prefill"], bias="zipf")
    x = synth.tokens(synth.REAL, synth.SEEDS["prefill"], 2048)
    _route_check(lay, x, dev)


# Adaptive expert top-p (the cut runs in the wave-per-token selector here).

@pytest.mark.parametrize("p", [0.3, 0.7, 0.9])
def test_route_top_p(dev, real, p):
    x = synth.tokens(synth.REAL, synth.SEEDS["decode"], 40, start=3)
    _route_check(real, x, dev, top_p=p)
    idx, _ = moe.route(moe.Config.of(synth.REAL, p), to_d(x, dev), real.wr_d, real.bias_d)
    if p < 0.8:
        assert (h(idx) < 0).any()  # the cut drops ranks on this workload


# ------------------------------------------------------------------ grouping

def _idx_case(T, K, E, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "one":
        return np.tile(np.arange(K, dtype=np.int32), (T, 1))
    if kind == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        rows = [rng.choice(E, K, replace=False, p=p) for _ in range(T)]
    else:
        rows = [rng.choice(E, K, replace=False) for _ in range(T)]
    idx = np.stack(rows).astype(np.int32)
    if kind == "dup":
        idx[T // 2:] = idx[:T - T // 2]
    return idx


@pytest.mark.parametrize("T,K,E,kind", [
    (1, 8, 256, "rand"), (4, 2, 8, "rand"), (16, 8, 256, "dup"), (2048, 8, 256, "zipf"),
    (100, 8, 256, "one"), (3, 4, 1024, "rand"), (777, 5, 300, "rand"), (1, 1, 2, "rand"),
    (4096, 16, 64, "rand"),
])
def test_group_bit_exact(dev, T, K, E, kind):
    _group_check(dev, _idx_case(T, K, E, kind, T * 31 + K), E)


@pytest.mark.parametrize("T,K,E", [(1, 8, 256), (16, 8, 256), (2048, 8, 256), (37, 3, 10)])
def test_group_with_dropped_ranks(dev, T, K, E):
    idx = _idx_case(T, K, E, "rand", T + K)
    keep = np.random.default_rng(T).integers(1, K + 1, T)
    for t in range(T):
        idx[t, keep[t]:] = -1
    _group_check(dev, idx, E)


def _group_check(dev, idx, E):
    T, K = idx.shape
    cfg = moe.Config(hidden=256, inter=128, n_experts=E, n_group=1, topk_group=1, top_k=K)
    g = moe.group(cfg, to_d(idx, dev))
    ref = oracle.group(idx, E)
    for k in ("counts", "offsets", "active"):
        assert np.array_equal(h(g[k]), ref[k]), k
    assert np.array_equal(h(g["perm"])[:T * K], ref["perm"])
    assert np.array_equal(h(g["inv"])[:T * K], ref["inv"])
    assert int(h(g["n_active"])[0]) == ref["n_active"]


# ------------------------------------------------------------------ expert FFN

def _ffn_check(layer, x, dev, check_chain=True):
    s = layer.shape
    cfg = moe.Config.of(s)
    H, I, K, wb = s.hidden, s.inter, s.top_k, s.wbits
    T = x.shape[0]
    idx, _, _ = oracle.route(x, layer.wr, layer.bias, s.n_group, s.topk_group, K,
                             s.routed_scaling)
    q, d = oracle.q8_0(x)
    dbg = moe.debug_buffers(cfg, T, dev)
    eo, so = moe.expert_ffn(cfg, to_d(q, dev), to_d(d, dev), to_d(idx, dev), layer.experts_d,
                            layer.shared_d, debug=dbg)
    eo, so = h(eo), h(so)
    dbg = {k: h(v) for k, v in dbg.items()}
    pairs = [(t * K + k, int(idx[t, k]), t) for t in range(T) for k in range(K)]
    pairs += [(T * K + t, synth.SHARED_ID, t) for t in range(T)]
    # fp32 sums of n per-block terms in any order: error within ~n * 2^-24 of
    # the magnitude (the block-sum order is open); 8x margin
    tol_h = max(1e-5, 8 * (H // 32) * 2.0 ** -24)
    tol_y = max(1e-5, 8 * (I // 32) * 2.0 ** -24)
    worst = 0.0
    for p, e, t in pairs:
        blob = layer.blob(e)
        ref = oracle.gate_up(blob, H, I, wb, q[t], d[t], want_dots=True)
        assert np.array_equal(dbg["gate_dots"][p], ref["gate_dots"]), (p, e)
        assert np.array_equal(dbg["up_dots"][p], ref["up_dots"]), (p, e)
        assert_close_rms(dbg["h"][p], ref["h"], tol_h, f"h pair {p}")
        qh, dh = oracle.q8_0(dbg["h"][p])
        assert np.array_equal(dbg["q_h"][p], qh), p
        assert np.array_equal(dbg["d_h"][p], dh), p
        y_ref, dd_ref = oracle.down(blob, H, I, wb, dbg["q_h"][p], dbg["d_h"][p], want_dots=True)
        assert np.array_equal(dbg["down_dots"][p], dd_ref), p
        y = eo[t, p % K] if p < T * K else so[t]
        assert_close_rms(y, y_ref, tol_y, f"y pair {p} (same q_h)")
        if check_chain:
            chain = oracle.expert(blob, H, I, wb, q[t], d[t])["y"]
            worst = max(worst, assert_close_rms(y, chain, 2e-3, f"y pair {p}"))
    return worst


def test_ffn_tiny(dev, tiny):
    _ffn_check(tiny, synth.tokens(synth.TINY, synth.SEEDS["tiny"], 4), dev)


def test_ffn_tiny_int2(dev):
    lay = DeviceLayer(synth.TINY.with_bits(2), synth.SEEDS["tiny"])
    _ffn_check(lay, synth.tokens(synth.TINY, synth.SEEDS["tiny"], 4), dev)


def test_ffn_decode(dev, real):
    _ffn_check(real, synth.tokens(synth.REAL, synth.SEEDS["decode"], 1, start=3), dev)


def test_ffn_verify4(dev, real):
    _ffn_check(real, synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], 4), dev,
               check_chain=False)


# The matrix-core path (batches above 16 tokens, int4): same dumps, same bar.

@pytest.mark.parametrize("T", [40, 200])
def test_ffn_tiny_mfma(dev, tiny, T):
    _ffn_check(tiny, synth.tokens(synth.TINY, synth.SEEDS["tiny"], T, start=11), dev)


def test_ffn_real_mfma(dev, real):
    _ffn_check(real, synth.tokens(synth.REAL, synth.SEEDS["prefill"], 24), dev, check_chain=False)


# int8-weight experts (the same record format with 8-bit codes) take the
# matrix-core path at every batch size.

@pytest.fixture(scope="module")
def real8(dev):
    return DeviceLayer(synth.REAL.with_bits(8), synth.SEEDS["decode"])


# MXFP4 experts (FP4 E2M1 codes, E8M0 scale per 32): the dumped block dots
# are sum 2 fp4(c) q, exact integers.

@pytest.fixture(scope="module")
def real_mx(dev):
    return DeviceLayer(synth.REAL.with_bits(synth.MXFP4), synth.SEEDS["decode"])


@pytest.mark.parametrize("T", [1, 4, 40])
def test_ffn_tiny_mxfp4(dev, T):
    lay = DeviceLayer(synth.TINY.with_bits(synth.MXFP4), synth.SEEDS["tiny"])
    _ffn_check(lay, synth.tokens(synth.TINY, synth.SEEDS["tiny"], T, start=6), dev)


def test_ffn_decode_mxfp4(dev, real_mx):
    _ffn_check(real_mx, synth.tokens(synth.REAL, synth.SEEDS["decode"], 1, start=3), dev)


def test_ffn_prefill_mxfp4(dev, real_mx):
    _ffn_check(real_mx, synth.tokens(synth.REAL, synth.SEEDS["prefill"], 24), dev,
               check_chain=False)


# FP8 E4M3 experts with 128x128 block scales: the vector kernels at every
# batch size; the dumped block dots are sum 512 fp8(c) q, exact integers.

@pytest.fixture(scope="module")
def real_f8(dev):
    return DeviceLayer(synth.REAL.with_bits(synth.FP8), synth.SEEDS["decode"])


@pytest.mark.parametrize("T", [1, 4, 40])
def test_ffn_tiny_fp8(dev, T):
    lay = DeviceLayer(synth.TINY.with_bits(synth.FP8), synth.SEEDS["tiny"])
    _ffn_check(lay, synth.tokens(synth.TINY, synth.SEEDS["tiny"], T, start=4), dev)


def test_ffn_decode_fp8(dev, real_f8):
    _ffn_check(real_f8, synth.tokens(synth.REAL, synth.SEEDS["decode"], 1, start=3), dev)


def test_ffn_verify_fp8(dev, real_f8):
    _ffn_check(real_f8, synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], 4), dev,
               check_chain=False)


def test_ffn_prefill_fp8(dev, real_f8):
    _ffn_check(real_f8, synth.tokens(synth.REAL, synth.SEEDS["prefill"], 24), dev,
               check_chain=False)


@pytest.mark.parametrize("T", [1, 4, 40])
def test_ffn_tiny_int8(dev, T):
    lay = DeviceLayer(synth.TINY.with_bits(8), synth.SEEDS["tiny"])
    _ffn_check(lay, synth.tokens(synth.TINY, synth.SEEDS["tiny"], T, start=2), dev)


def test_ffn_decode_int8(dev, real8):
    _ffn_check(real8, synth.tokens(synth.REAL, synth.SEEDS["decode"], 1, start=3), dev)


def test_ffn_verify_int8(dev, real8):
    _ffn_check(real8, synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], 4), dev,
               check_chain=False)


def test_ffn_real_mfma_int8(dev, real8):
    _ffn_check(real8, synth.tokens(synth.REAL, synth.SEEDS["prefill"], 24), dev,
               check_chain=False)


# ------------------------------------------------------------------ combine

@pytest.mark.parametrize("T,K,H,res,norm", [(1, 8, 6144, False, False), (4, 2, 256, True, True),
                                            (16, 8, 6144, True, False), (5, 1, 64, False, True)])
def test_combine(dev, T, K, H, res, norm):
    rng = np.random.default_rng(T + K + H)
    eo = rng.standard_normal((T, K, H)).astype(np.float32)
    w = rng.uniform(0, 1, (T, K)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    r = rng.standard_normal((T, H)).astype(np.float32) if res else None
    out = moe.combine(to_d(eo, dev), to_d(w, dev), to_d(sh, dev),
                      to_d(r, dev) if res else None, want_norm=norm)
    ref = oracle.combine(eo, w, sh, r, want_norm=norm)
    if norm:
        assert_close_rms(h(out[0]), ref[0], 1e-5, "y")
        assert_close_rms(h(out[1]), ref[1], 1e-5, "y_norm")
    else:
        assert_close_rms(h(out), ref, 1e-5, "y")


def test_rmsnorm(dev):
    x = synth.tokens(synth.REAL, 3, 5)
    assert_close_rms(h(moe.rmsnorm(to_d(x, dev))), oracle.rmsnorm(x), 1e-5)


# ------------------------------------------------------------------ whole layer

def _layer_check(layer, x, dev, residual=None, want_norm=False, top_p=0.0):
    s = layer.shape
    cfg = moe.Config.of(s, top_p)
    T = x.shape[0]
    idx_d = torch.empty((T, s.top_k), dtype=torch.int32, device=dev)
    w_d = torch.empty((T, s.top_k), dtype=torch.float32, device=dev)
    out = moe.layer(cfg, to_d(x, dev), layer.wr_d, layer.bias_d, layer.experts_d, layer.shared_d,
                    residual=None if residual is None else to_d(residual, dev),
                    want_norm=want_norm, idx_out=idx_d, w_out=w_d)
    ref = layer.oracle_layer(x, residual, want_norm, top_p)
    assert np.array_equal(h(idx_d), ref["idx"])
    assert np.array_equal(h(w_d), ref["w"])
    if want_norm:
        assert_close_rms(h(out[0]), ref["y"], 2e-3, "y")
        assert_close_rms(h(out[1]), ref["y_norm"], 2e-3, "y_norm")
        return h(out[0])
    assert_close_rms(h(out), ref["y"], 2e-3, "y")
    return h(out)


def test_layer_tiny(dev, tiny):
    _layer_check(tiny, synth.tokens(synth.TINY, synth.SEEDS["tiny"], 4), dev)


def test_layer_tiny_ragged_batches(dev, tiny):
    for T in (1, 3, 5, 9, 33):
        _layer_check(tiny, synth.tokens(synth.TINY, 77, T), dev)


@pytest.mark.parametrize("start", [0, 1, 2])
def test_layer_decode(dev, real, start):
    _layer_check(real, synth.tokens(synth.REAL, synth.SEEDS["decode"], 1, start=start), dev)


@pytest.mark.parametrize("T", [4, 16])
def test_layer_verify(dev, real, T):
    _layer_check(real, synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], T), dev)


def test_layer_residual_norm(dev, real):
    x = synth.tokens(synth.REAL, 9, 2)
    res = synth.tokens(synth.REAL, 10, 2)
    _layer_check(real, x, dev, residual=res, want_norm=True)


def test_layer_int2_decode(dev):
    lay = DeviceLayer(synth.REAL.with_bits(2), synth.SEEDS["stack"])
    _layer_check(lay, synth.tokens(synth.REAL, synth.SEEDS["stack"], 1), dev)


@pytest.mark.parametrize("T", [1, 4, 16, 40])
def test_layer_top_p(dev, real, T):
    """Decode, verify and the chained path (T > 16) with top-p 0.7."""
    x = synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], T) if T > 1 else \
        synth.tokens(synth.REAL, synth.SEEDS["decode"], 1, start=4)
    _layer_check(real, x, dev, top_p=0.7)


def test_layer_top_p_tiny_ragged(dev, tiny):
    for T, p in ((1, 0.5), (5, 0.6), (33, 0.55)):
        _layer_check(tiny, synth.tokens(synth.TINY, 79, T), dev, top_p=p)


def test_combine_skips_dropped_rows(dev):
    rng = np.random.default_rng(3)
    T, K, H = 3, 8, 256
    eo = rng.standard_normal((T, K, H)).astype(np.float32)
    w = rng.uniform(0.1, 1, (T, K)).astype(np.float32)
    w[:, 5:] = 0.0
    eo[:, 5:] = np.nan  # never read
    out = h(moe.combine(to_d(eo, dev), to_d(w, dev), None, None))
    eo[:, 5:] = 0.0
    assert_close_rms(out, oracle.combine(eo, w), 1e-5, "y")


def test_layer_tiny_mxfp4(dev):
    lay = DeviceLayer(synth.TINY.with_bits(synth.MXFP4), synth.SEEDS["tiny"])
    for T in (1, 4, 9, 33):
        _layer_check(lay, synth.tokens(synth.TINY, 80, T), dev)


@pytest.mark.parametrize("T,start", [(1, 0), (1, 1), (4, 0), (16, 0), (40, 0)])
def test_layer_mxfp4(dev, real_mx, T, start):
    x = synth.tokens(synth.REAL, synth.SEEDS["decode"], T, start=start) if T == 1 else \
        synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], T)
    _layer_check(real_mx, x, dev)


def test_layer_tiny_int8(dev):
    lay = DeviceLayer(synth.TINY.with_bits(8), synth.SEEDS["tiny"])
    for T in (1, 4, 9, 33):
        _layer_check(lay, synth.tokens(synth.TINY, 78, T), dev)


@pytest.mark.parametrize("start", [0, 1])
def test_layer_int8_decode(dev, real8, start):
    _layer_check(real8, synth.tokens(synth.REAL, synth.SEEDS["decode"], 1, start=start), dev)


@pytest.mark.parametrize("T", [4, 16])
def test_layer_int8_verify(dev, real8, T):
    _layer_check(real8, synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], T), dev)


# FP8 layers: the small-batch kernels up to 4 tokens, the chained vector
# kernels above.

def test_layer_tiny_fp8(dev):
    lay = DeviceLayer(synth.TINY.with_bits(synth.FP8), synth.SEEDS["tiny"])
    for T in (1, 2, 3, 4, 5, 9, 33):
        _layer_check(lay, synth.tokens(synth.TINY, 76, T), dev)


@pytest.mark.parametrize("T,start", [(1, 0), (1, 1), (1, 2), (3, 0), (4, 0), (16, 0)])
def test_layer_fp8(dev, real_f8, T, start):
    # perturbed pairs of tokens (even T) share most experts
    x = synth.tokens(synth.REAL, synth.SEEDS["decode"], T, start=start) if T % 2 else \
        synth.tokens_perturbed(synth.REAL, synth.SEEDS["verify"], T)
    _layer_check(real_f8, x, dev)


@pytest.mark.parametrize("T", [1, 4])
def test_layer_fp8_residual_norm_top_p(dev, real_f8, T):
    """The small-batch FP8 kernels with the residual, the RMSNorm kernel and
    top-p 0.7 together."""
    x = synth.tokens(synth.REAL, 12, T)
    res = synth.tokens(synth.REAL, 13, T)
    _layer_check(real_f8, x, dev, residual=res, want_norm=True, top_p=0.7)


def test_layer_int8_residual_norm(dev, real8):
    x = synth.tokens(synth.REAL, 9, 2)
    res = synth.tokens(synth.REAL, 10, 2)
    _layer_check(real8, x, dev, residual=res, want_norm=True)


def test_layer_deterministic(dev, real):
    x = to_d(synth.tokens_perturbed(synth.REAL, 5, 16), dev)
    cfg = moe.Config.of(synth.REAL)
    a = h(moe.layer(cfg, x, real.wr_d, real.bias_d, real.experts_d, real.shared_d))
    b = h(moe.layer(cfg, x, real.wr_d, real.bias_d, real.experts_d, real.shared_d))
    assert np.array_equal(a, b)


def test_zero_tokens_is_noop(dev, tiny):
    cfg = moe.Config.of(synth.TINY)
    x = torch.empty((0, 256), dtype=torch.float32, device=dev)
    y = moe.layer(cfg, x, tiny.wr_d, tiny.bias_d, tiny.experts_d, tiny.shared_d)
    assert y.shape == (0, 256)


def test_layer_graph_replays_match_eager(dev, real):
    """moe_layer captured in a HIP graph: every replay equals the eager result,
    with unrelated eager work and synchronisations between replays."""
    cfg = moe.Config.of(synth.REAL)
    st = torch.cuda.Stream(device=dev)
    xs = [to_d(synth.tokens_perturbed(synth.REAL, 21 + i, 4), dev) for i in range(3)]
    ws = torch.zeros(moe.layer_workspace(cfg, 4), dtype=torch.uint8, device=dev)
    with torch.cuda.stream(st):
        eager = [h(moe.layer(cfg, x, real.wr_d, real.bias_d, real.experts_d, real.shared_d,
                             workspace=ws)) for x in xs]
        ys = [torch.empty((4, 6144), dtype=torch.float32, device=dev) for _ in xs]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for x, y in zip(xs, ys):
                moe.layer(cfg, x, real.wr_d, real.bias_d, real.experts_d, real.shared_d, y=y,
                          workspace=ws)
        for rep in range(4):
            for y in ys:
                y.fill_(float("nan"))
            other = moe.layer(cfg, to_d(synth.tokens(synth.REAL, 99 + rep, 2), dev), real.wr_d,
                              real.bias_d, real.experts_d, real.shared_d)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for y, e in zip(ys, eager):
                assert np.array_equal(h(y), e), f"replay {rep}"
            assert np.all(np.isfinite(h(other)))


_prefill = {}


def teardown_module(module):
    _prefill.clear()


def prefill_run(dev):
    """Prefill at full size (2048 tokens, Zipf-skewed bias) through moe_layer,
    run once for the module, with h and Q8_0(h) of every pair dumped:
    (layer, x, idx, w, y, dumps)."""
    if not _prefill:
        lay = DeviceLayer(synth.REAL, synth.SEEDS["prefill"], bias="zipf")
        s = lay.shape
        T = 2048
        cfg = moe.Config.of(s)
        x = synth.tokens(s, synth.SEEDS["prefill"], T)
        idx_d = torch.empty((T, s.top_k), dtype=torch.int32, device=dev)
        w_d = torch.empty((T, s.top_k), dtype=torch.float32, device=dev)
        full = moe.layer_debug_buffers(cfg, 1, dev)  # shapes only
        P = T * (s.top_k + s.n_shared)
        dumps = {k: torch.zeros((P,) + tuple(full[k].shape[1:]), dtype=full[k].dtype, device=dev)
                 for k in ("h", "q_h", "d_h")}
        y = h(moe.layer(cfg, to_d(x, dev), lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                        idx_out=idx_d, w_out=w_d, debug=dumps))
        y_plain = h(moe.layer(cfg, to_d(x, dev), lay.wr_d, lay.bias_d, lay.experts_d,
                              lay.shared_d))
        assert np.array_equal(y, y_plain)
        _prefill.update(lay=lay, x=x, idx=h(idx_d), w=h(w_d), y=y,
                        dumps={k: h(v) for k, v in dumps.items()})
    return _prefill


def test_layer_prefill_full_size_routing(dev):
    """Every index and weight of the 2048 tokens bit-exact."""
    r = prefill_run(dev)
    s = r["lay"].shape
    idx, w, _ = oracle.route(r["x"], r["lay"].wr, r["lay"].bias, s.n_group, s.topk_group,
                             s.top_k, s.routed_scaling)
    assert np.array_equal(r["idx"], idx)
    assert np.array_equal(r["w"], w)
    counts = np.bincount(idx.ravel(), minlength=s.n_experts)
    assert counts.max() > 64  # several token tiles for the hot experts


def _prefill_sample(r, chunk):
    """Token chunk `chunk` of the 256 checked: 0 = the hottest expert's first
    64-token tile, 1 = its last tile (with the tokens after it to fill 64),
    2-3 = tokens spread over the batch."""
    s = r["lay"].shape
    idx = r["idx"]
    hot = int(np.argmax(np.bincount(idx.ravel(), minlength=s.n_experts)))
    toks = np.flatnonzero((idx == hot).any(axis=1))  # the hot expert's list, in order
    if chunk == 0:
        return toks[:64]
    if chunk == 1:
        last = toks[(len(toks) - 1) // 64 * 64:]
        rest = np.setdiff1d(np.arange(2048), np.concatenate([toks[:64], last]))
        return np.concatenate([last, rest[-(64 - len(last)):]]) if len(last) < 64 else last
    rng = np.random.default_rng(chunk)
    return np.sort(rng.choice(2048, 64, replace=False))


@pytest.mark.parametrize("chunk", [0, 1, 2, 3])
def test_layer_prefill_full_size_outputs(dev, chunk):
    """The layer output of 256 of the 2048 tokens (every token of the hottest
    expert's first and last tiles among them) against the oracle run on
    those tokens alone (tokens are independent once routed), its down
    projections taken on the GPU's own Q8_0(h) once that decision is checked
    (DeviceLayer.oracle_layer_on_gpu_qh).  Tokens whose every Q8_0(h) code
    equals the oracle's own also match the plain oracle layer."""
    r = prefill_run(dev)
    sel = _prefill_sample(r, chunk)
    assert len(sel) == 64
    lay = r["lay"]
    ref = lay.oracle_layer_on_gpu_qh(r["x"][sel], r["dumps"], tokens=sel)
    assert np.array_equal(ref["idx"], r["idx"][sel])
    for i, t in enumerate(sel):
        assert_close_rms(r["y"][t], ref["y"][i], 2e-3, f"y token {t}")
    if ref["qh_flips"] == 0:
        plain = lay.oracle_layer(r["x"][sel])
        assert_close_rms(r["y"][sel], plain["y"], 2e-3, "y (plain oracle)")


# Every token the same: every routed slot carries all T tokens, so the gate/up
# kernel streams each row once for many chunks of tokens whose activations it
# stages in LDS, over several staging rounds when the slot holds more tokens
# than one round takes (int4 at this width: 6), the last round ragged.

def _same_tokens(shape, T):
    return np.repeat(synth.tokens(shape, 11, 1), T, axis=0)


@pytest.mark.parametrize("T", [3, 7, 13, 16])
def test_layer_identical_tokens(dev, real, T):
    _layer_check(real, _same_tokens(synth.REAL, T), dev)


@pytest.mark.parametrize("T", [5, 16])
def test_layer_identical_tokens_mxfp4(dev, real_mx, T):
    _layer_check(real_mx, _same_tokens(synth.REAL, T), dev)


def test_layer_identical_tokens_int2(dev):
    lay = DeviceLayer(synth.REAL.with_bits(2), synth.SEEDS["stack"])
    for T in (5, 13):
        _layer_check(lay, _same_tokens(synth.REAL, T), dev)


@pytest.mark.parametrize("T", [2, 4, 16])
def test_layer_identical_tokens_fp8(dev, real_f8, T):
    """Every token on the same experts: at 2 and 4 tokens the small-batch
    kernels' slots hold all of them (staged in LDS, rows streamed once)."""
    _layer_check(real_f8, _same_tokens(synth.REAL, T), dev)


def test_layer_identical_tokens_tiny(dev, tiny):
    for bits in (4, 2, synth.MXFP4, 8, synth.FP8):
        lay = tiny if bits == 4 else DeviceLayer(synth.TINY.with_bits(bits), synth.SEEDS["tiny"])
        for T in (3, 9, 16):
            _layer_check(lay, _same_tokens(synth.TINY, T), dev)
