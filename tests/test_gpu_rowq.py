"""The per-row activation format (moe_cfg.act_block = MOE_ACT_ROW, reading
R17: one fp32 scale per row of x and of h, one exact int32 dot per output
row) on the GPU against the oracle:

- moe_quant_act with the block spanning the row: codes and scales bit-exact;
- moe_expert_ffn (the row-dot MFMA kernels at every batch size) with every
  dump: gate/up row dots bit-exact against the oracle on x; h within the fp32
  bound; the codes of h exactly the per-row quantisation of the GPU's h; the
  down row dots bit-exact against the oracle on those codes;
- moe_layer: indices bit-exact, outputs within 2e-3 * RMS of the oracle layer
  whose down projections take the GPU's own codes of h (checked as above),
  up to prefill at full size;
- every code pattern (int4 -8, int8 -128) and extreme activations.
"""
import numpy as np
import pytest
import torch

import int4_routed_expert_moe_amd as moe
import oracle
import synth
from _inputs import DeviceLayer, assert_close_rms, pairs_of

pytestmark = pytest.mark.gpu
ROW = oracle.ACT_ROW


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


_layers = {}


def layer_of(shape_name, bits, seed_name="decode", bias="uniform"):
    key = (shape_name, bits, seed_name, bias)
    if key not in _layers:
        base = synth.REAL if shape_name == "real" else synth.TINY
        _layers[key] = DeviceLayer(base.with_bits(bits), synth.SEEDS[seed_name], bias=bias)
    return _layers[key]


def teardown_module(module):
    _layers.clear()


def to_d(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def h(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def heavy(shape, T, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, shape.hidden)) *
         np.exp2(rng.standard_normal((T, shape.hidden)) * 2)).astype(np.float32)
    if T > 1:
        x[1] = 0.0  # a zero row: d = 0, every code 0
    if T > 2:
        x[2, 7] = 1e5  # one element dominating its row
    return x


@pytest.mark.parametrize("rows,n", [(1, 6144), (37, 2048), (2048, 6144), (5, 32), (3, 256)])
def test_quant_act_rows_bit_exact(dev, rows, n):
    x = heavy(synth.LayerShape(n, 128, 8, 2, 1, 2), rows, rows + n)
    q, d = moe.quant_act(to_d(x, dev), block=n)
    qo, do = oracle.quant_act(x, ROW)
    assert np.array_equal(h(q), qo)
    assert np.array_equal(h(d).view(np.uint32), do.view(np.uint32))


def check_ffn_rows(lay, x, dev):
    """moe_expert_ffn in the per-row format, every dump against the oracle."""
    s = lay.shape
    cfg = moe.Config.of(s, act_block=moe.ACT_ROW)
    H, I, wb = s.hidden, s.inter, s.wbits
    T = x.shape[0]
    idx, _, _ = oracle.route(x, lay.wr, lay.bias, s.n_group, s.topk_group, s.top_k,
                             s.routed_scaling)
    q, d = oracle.quant_act(x, ROW)
    dbg_d = moe.debug_buffers(cfg, T, dev)
    eo, so = moe.expert_ffn(cfg, to_d(q, dev), to_d(d, dev), to_d(idx, dev), lay.experts_d,
                            lay.shared_d, debug=dbg_d)
    eo, so = h(eo), h(so)
    dbg = {k: h(v) for k, v in dbg_d.items()}
    tol_h = max(1e-5, 8 * (H // 32) * 2.0 ** -24)
    blobs = {}
    for p, e, t in pairs_of(idx, s.n_shared):
        if e not in blobs:
            blobs[e] = lay.blob(e)
        ref = oracle.gate_up(blobs[e], H, I, wb, q[t], d[t], want_dots=True, act_block=ROW)
        assert np.array_equal(dbg["gate_dots"][p], ref["gate_dots"]), ("gate", p, e)
        assert np.array_equal(dbg["up_dots"][p], ref["up_dots"]), ("up", p, e)
        assert_close_rms(dbg["h"][p], ref["h"], tol_h, f"h pair {p}")
        qh, dh = oracle.quant_act(dbg["h"][p], ROW)
        assert np.array_equal(dbg["q_h"][p], qh) and np.array_equal(dbg["d_h"][p], dh), p
        y_ref, dd = oracle.down(blobs[e], H, I, wb, qh, dh, want_dots=True, act_block=ROW)
        assert np.array_equal(dbg["down_dots"][p], dd), ("down", p, e)
        y = eo[t, p % s.top_k] if p < T * s.top_k else so[t]
        assert_close_rms(y, y_ref, max(1e-5, 8 * 2.0 ** -24), f"y pair {p} (same codes)")


@pytest.mark.parametrize("bits", [4, 8])
def test_ffn_rows_tiny(dev, bits):
    lay = layer_of("tiny", bits, "tiny")
    for T in (1, 4, 40, 200):
        check_ffn_rows(lay, heavy(lay.shape, T, 50 + T), dev)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("T", [1, 24, 70])
def test_ffn_rows_real(dev, bits, T):
    lay = layer_of("real", bits)
    x = synth.tokens(lay.shape, synth.SEEDS["prefill"], T) if T > 1 else heavy(lay.shape, 1, 9)
    check_ffn_rows(lay, x, dev)


def check_layer_rows(lay, x, dev, residual=None, want_norm=False):
    s = lay.shape
    cfg = moe.Config.of(s, act_block=moe.ACT_ROW)
    T = x.shape[0]
    idx_d = torch.empty((T, s.top_k), dtype=torch.int32, device=dev)
    w_d = torch.empty((T, s.top_k), dtype=torch.float32, device=dev)
    full = moe.layer_debug_buffers(cfg, T, dev)
    dumps = {k: full[k] for k in ("h", "q_h", "d_h", "q", "d")}
    res = None if residual is None else to_d(residual, dev)
    out = moe.layer(cfg, to_d(x, dev), lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                    residual=res, want_norm=want_norm, idx_out=idx_d, w_out=w_d, debug=dumps)
    plain = moe.layer(cfg, to_d(x, dev), lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                      residual=res, want_norm=want_norm)
    y = h(out[0] if want_norm else out)
    assert np.array_equal(y, h(plain[0] if want_norm else plain))
    dumps = {k: h(v) for k, v in dumps.items()}
    qo, do = oracle.quant_act(x, ROW)
    assert np.array_equal(dumps["q"], qo) and np.array_equal(dumps["d"], do)
    ref = lay.oracle_layer_on_gpu_qh(x, dumps, residual=residual, want_norm=want_norm,
                                     act_block=ROW)
    assert np.array_equal(h(idx_d), ref["idx"]) and np.array_equal(h(w_d), ref["w"])
    assert_close_rms(y, ref["y"], 2e-3, "y")
    if want_norm:
        assert_close_rms(h(out[1]), ref["y_norm"], 2e-3, "y_norm")
    return y, ref


@pytest.mark.parametrize("bits", [4, 8])
def test_layer_rows_tiny(dev, bits):
    lay = layer_of("tiny", bits, "tiny")
    for T in (1, 9, 40):
        _, ref = check_layer_rows(lay, synth.tokens(lay.shape, 60 + T, T), dev)
        if ref["qh_flips"] == 0:  # then the plain oracle layer matches too
            plain = lay.oracle_layer(synth.tokens(lay.shape, 60 + T, T), act_block=ROW)
            assert np.array_equal(plain["idx"], ref["idx"])


@pytest.mark.parametrize("T", [1, 16, 64])
def test_layer_rows_real(dev, T):
    lay = layer_of("real", 4)
    x = synth.tokens_perturbed(lay.shape, 70 + T, T) if T > 1 else synth.tokens(lay.shape, 70, 1)
    check_layer_rows(lay, x, dev, residual=synth.tokens(lay.shape, 71, T), want_norm=True)


def test_layer_rows_prefill_full_size(dev):
    """2048 tokens, Zipf-skewed routing: every index bit-exact; 64 tokens
    (among them the hottest expert's first tile) against the oracle on the
    GPU's own codes of h."""
    lay = layer_of("real", 4, "prefill", "zipf")
    s = lay.shape
    cfg = moe.Config.of(s, act_block=moe.ACT_ROW)
    T = 2048
    x = synth.tokens(s, synth.SEEDS["prefill"], T)
    idx_d = torch.empty((T, s.top_k), dtype=torch.int32, device=dev)
    P = T * (s.top_k + s.n_shared)
    dumps = dict(h=torch.zeros((P, s.inter), dtype=torch.float32, device=dev),
                 q_h=torch.zeros((P, s.inter), dtype=torch.int8, device=dev),
                 d_h=torch.zeros((P, 1), dtype=torch.float32, device=dev))
    y = h(moe.layer(cfg, to_d(x, dev), lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                    idx_out=idx_d, debug=dumps))
    idx = h(idx_d)
    ri, _, _ = oracle.route(x, lay.wr, lay.bias, s.n_group, s.topk_group, s.top_k,
                            s.routed_scaling)
    assert np.array_equal(idx, ri)
    hot = int(np.argmax(np.bincount(idx.ravel(), minlength=s.n_experts)))
    toks = np.flatnonzero((idx == hot).any(axis=1))
    sel = np.unique(np.concatenate([toks[:48], np.arange(0, T, T // 16)]))
    dumps = {k: h(v) for k, v in dumps.items()}
    ref = lay.oracle_layer_on_gpu_qh(x[sel], dumps, tokens=sel, act_block=ROW)
    for i, t in enumerate(sel):
        assert_close_rms(y[t], ref["y"][i], 2e-3, f"y token {t}")


def pattern_record_int(shape, seed):
    """Rows of the lowest code, lowest/highest alternating, every code in
    turn, and random codes (int4 -8..7, int8 -128..127)."""
    rng = np.random.default_rng(seed)
    wb = shape.wbits
    lo, hi = -(1 << (wb - 1)), (1 << (wb - 1)) - 1
    allc = np.arange(lo, hi + 1)

    def mat(rows, n):
        c = rng.choice(allc, (rows, n)).astype(np.int16)
        k = np.arange(n)
        c[0::4] = lo
        c[1::4] = np.where(k % 2 == 0, lo, hi)[None, :]
        c[2::4] = allc[(k[None, :] + np.arange(c[2::4].shape[0])[:, None]) % allc.size]
        return c.astype(np.int8)

    H, I = shape.hidden, shape.inter
    mats = [mat(I, H), mat(I, H), mat(H, I)]
    sc = [(rng.uniform(0.5, 1.5, m.shape[0]) * 0.02 / (hi + 1)).astype(np.float32) for m in mats]
    return np.concatenate([oracle.pack(m.ravel(), wb) for m in mats] + [v.view(np.uint8) for v in sc])


@pytest.mark.parametrize("bits", [4, 8])
def test_rows_code_patterns(dev, bits):
    lay = DeviceLayer(synth.TINY.with_bits(bits), synth.SEEDS["tiny"])
    for e in list(range(lay.shape.n_experts)) + [synth.SHARED_ID]:
        lay.set_record(e, pattern_record_int(lay.shape, 3 + (e % 7)))
    for T in (1, 40):
        x = heavy(lay.shape, T, 90 + T)
        x[0, ::2] = np.where(np.arange(lay.shape.hidden // 2) % 2 == 0, -1.0, 1.0)
        check_ffn_rows(lay, x, dev)
        check_layer_rows(lay, x, dev)
