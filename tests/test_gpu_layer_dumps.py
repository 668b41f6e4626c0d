"""The integer work of the path moe_layer runs, bit for bit.

For 1..16 tokens moe_layer runs the fused small-batch kernels (router,
selection beside the shared expert's gate/up, batch union + routed gate/up +
Q8_0 of h, down + combine; from 4 tokens (int4 and int2; MXFP4 from 8, int8
from 12) the down projection as MFMA tiles from the slot table); above that
it chains the separate kernels.  With a
moe_layer_debug those kernels also write what they compute: Q8_0 of x, the
batch union, the exact int32 block dots of gate/up and down, h and its Q8_0.
Each is compared with the CPU oracle on the same seeded inputs:

- Q8_0 of x, the union, and every gate/up block dot: bit-exact against the
  oracle on x;
- h: within the fp32 summation bound of the oracle's fp64 value; its Q8_0
  bit-exact against the oracle re-quantising the GPU's own h (the same fp32
  decision on the same value);
- every down block dot: bit-exact against the oracle on the GPU's Q8_0(h);
- the layer output within 2e-3 * RMS, and bit-identical to a call without
  dumps (the production build of the same kernels).

Also here: exact router ties on the GPU (lowest index wins), hand-built
records with every code of every weight format (int4 -8, int8 -128, all int2
codes, all 16 FP4 codes including -0, extreme E8M0 scales) on every kernel
path, a workspace full of garbage, and records read through a table of
pointers (some in host memory) against the oracle.
"""
import numpy as np
import pytest
import torch

import int4_routed_expert_moe_amd as moe
import oracle
import synth
from _inputs import DeviceLayer, assert_close_rms, pairs_of

pytestmark = pytest.mark.gpu

FORMATS = {"int4": 4, "int2": 2, "int8": 8, "mxfp4": synth.MXFP4, "fp8": synth.FP8}
UNION = ("counts", "offsets", "perm", "inv", "active")


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


_layers = {}


def real_layer(fmt):
    """One real-shape layer per weight format, kept for the module."""
    if fmt not in _layers:
        _layers[fmt] = DeviceLayer(synth.REAL.with_bits(FORMATS[fmt]), synth.SEEDS["decode"])
    return _layers[fmt]


def teardown_module(module):
    _layers.clear()


def to_d(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def h(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def batch(shape, T, seed):
    """Decode (one token) or the verify recipe (half the tokens are perturbed
    copies of the other half)."""
    if T == 1:
        return synth.tokens(shape, seed, 1, start=3)
    return synth.tokens_perturbed(shape, seed, T)


def check_dots(lay, q, d, idx, dbg, what=""):
    """Every pair's block dots, h and Q8_0(h) from the dumps against the oracle."""
    s = lay.shape
    H, I, wb = s.hidden, s.inter, s.wbits
    tol_h = max(1e-5, 8 * (H // 32) * 2.0 ** -24)
    T, K = idx.shape
    blobs = {}
    for p, e, t in pairs_of(idx, s.n_shared):
        if e not in blobs:
            blobs[e] = lay.blob(e)
        blob = blobs[e]
        ref = oracle.gate_up(blob, H, I, wb, q[t], d[t], want_dots=True)
        assert np.array_equal(dbg["gate_dots"][p], ref["gate_dots"]), (what, "gate", p, e)
        assert np.array_equal(dbg["up_dots"][p], ref["up_dots"]), (what, "up", p, e)
        assert_close_rms(dbg["h"][p], ref["h"], tol_h, f"{what} h pair {p}")
        qh, dh = oracle.q8_0(dbg["h"][p])
        assert np.array_equal(dbg["q_h"][p], qh), (what, "q_h", p)
        assert np.array_equal(dbg["d_h"][p], dh), (what, "d_h", p)
        _, dd = oracle.down(blob, H, I, wb, dbg["q_h"][p], dbg["d_h"][p], want_dots=True)
        assert np.array_equal(dbg["down_dots"][p], dd), (what, "down", p, e)
    # no dump for a slot dropped by top-p
    for t in range(T):
        for k in range(K):
            if idx[t, k] < 0:
                assert not dbg["gate_dots"][t * K + k].any() and not dbg["down_dots"][t * K + k].any()


def check_layer_dumps(lay, x, dev, top_p=0.0, table=None, residual=None, workspace=None):
    """moe_layer (or moe_layer_ptrs with `table`) with every dump, against the
    oracle; returns the layer output."""
    s = lay.shape
    cfg = moe.Config.of(s, top_p)
    T = x.shape[0]
    K, E = s.top_k, s.n_experts
    xd = to_d(x, dev)
    res = None if residual is None else to_d(residual, dev)
    idx_d = torch.empty((T, K), dtype=torch.int32, device=dev)
    w_d = torch.empty((T, K), dtype=torch.float32, device=dev)
    dbg_d = moe.layer_debug_buffers(cfg, T, dev)
    if table is None:
        call = lambda **kw: moe.layer(cfg, xd, lay.wr_d, lay.bias_d, lay.experts_d,  # noqa: E731
                                      lay.shared_d, residual=res, workspace=workspace, **kw)
    else:
        call = lambda **kw: moe.layer_ptrs(cfg, xd, lay.wr_d, lay.bias_d, table,  # noqa: E731
                                           lay.shared_d, residual=res, workspace=workspace, **kw)
    y = h(call(idx_out=idx_d, w_out=w_d, debug=dbg_d))
    y_plain = h(call())
    assert np.array_equal(y, y_plain), "dumping build differs from the production kernels"
    dbg = {k: h(v) for k, v in dbg_d.items()}
    ri, rw, _ = oracle.route(x, lay.wr, lay.bias, s.n_group, s.topk_group, K, s.routed_scaling,
                             top_p)
    assert np.array_equal(h(idx_d), ri)
    assert np.array_equal(h(w_d).view(np.uint32), rw.view(np.uint32))
    q, d = oracle.q8_0(x)
    assert np.array_equal(dbg["q"], q)
    assert np.array_equal(dbg["d"].view(np.uint32), d.view(np.uint32))
    g = oracle.group(ri, E)
    for k in UNION:
        assert np.array_equal(dbg[k], g[k]), k
    assert int(dbg["n_active"][0]) == g["n_active"]
    check_dots(lay, q, d, ri, dbg, f"T={T}")
    ref = oracle.layer(x, lay.wr, lay.bias, lay.blob,
                       lay.blob(synth.SHARED_ID) if s.n_shared else None, H=s.hidden, I=s.inter,
                       n_experts=E, n_group=s.n_group, topk_group=s.topk_group, top_k=K,
                       scale=s.routed_scaling, wbits=s.wbits, residual=residual, top_p_value=top_p)
    assert_close_rms(y, ref["y"], 2e-3, "y")
    return y


# ------------------------------------------------------------------ the timed path, every format

@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("T", [1, 2, 4, 8, 12, 16])
def test_layer_dumps_real(dev, fmt, T):
    lay = real_layer(fmt)
    check_layer_dumps(lay, batch(lay.shape, T, synth.SEEDS["verify"] + T), dev)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_layer_dumps_tiny(dev, fmt):
    lay = DeviceLayer(synth.TINY.with_bits(FORMATS[fmt]), synth.SEEDS["tiny"])
    for T in (1, 3, 9, 16, 40):
        check_layer_dumps(lay, synth.tokens(lay.shape, 81, T), dev)


def test_layer_dumps_top_p_and_residual(dev):
    lay = real_layer("int4")
    x = batch(lay.shape, 16, 7)
    check_layer_dumps(lay, x, dev, top_p=0.7, residual=synth.tokens(lay.shape, 8, 16))
    check_layer_dumps(lay, x[:4], dev, top_p=0.5)


@pytest.mark.parametrize("fmt", ["int4", "int8", "fp8"])
def test_layer_dumps_chained_path(dev, fmt):
    """Above 16 tokens the same dumps come from the chained kernels."""
    lay = real_layer(fmt)
    check_layer_dumps(lay, batch(lay.shape, 24, 19), dev)


# ------------------------------------------------------------------ exact router ties

def _route_and_layer(lay, wr, bias, x, dev):
    """moe_route and moe_layer on (wr, bias): idx and w bit-exact vs the oracle."""
    s = lay.shape
    cfg = moe.Config.of(s)
    T = x.shape[0]
    wr_d, bias_d = to_d(wr, dev), to_d(bias, dev)
    ri, rw, _ = oracle.route(x, wr, bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling)
    idx, w = moe.route(cfg, to_d(x, dev), wr_d, bias_d)
    assert np.array_equal(h(idx), ri) and np.array_equal(h(w), rw), "moe_route"
    idx_d = torch.empty((T, s.top_k), dtype=torch.int32, device=dev)
    w_d = torch.empty((T, s.top_k), dtype=torch.float32, device=dev)
    y = moe.layer(cfg, to_d(x, dev), wr_d, bias_d, lay.experts_d, lay.shared_d, idx_out=idx_d,
                  w_out=w_d)
    assert np.array_equal(h(idx_d), ri) and np.array_equal(h(w_d), rw), "moe_layer"
    return ri, rw, h(y)


@pytest.mark.parametrize("T", [1, 16, 40])
def test_ties_zero_input_equal_bias(dev, T):
    """x = 0 and equal biases: every score is sigmoid(0) = 0.5, every group
    ties and every expert ties, so the TG lowest groups are kept and the K
    lowest experts picked, in index order, each weighted 2.5 / K."""
    lay = real_layer("int4")
    s = lay.shape
    bias = np.full(s.n_experts, 0.0625, np.float32)
    x = np.zeros((T, s.hidden), np.float32)
    ri, rw, y = _route_and_layer(lay, lay.wr, bias, x, dev)
    assert np.array_equal(ri, np.tile(np.arange(s.top_k, dtype=np.int32), (T, 1)))
    assert np.all(rw == np.float32(2.5 / s.top_k))
    assert np.all(y == 0.0)  # Q8_0 of zeros is zero; every dot is 0


@pytest.mark.parametrize("T", [1, 16, 40])
def test_ties_duplicated_router_rows(dev, T):
    """Twins with identical router rows and biases have identical scores;
    a group copied onto another ties its group score too.  The lower index
    must come first, on every path, exactly as the oracle orders them."""
    lay = real_layer("int4")
    s = lay.shape
    gs = s.n_experts // s.n_group
    x = synth.tokens(s, 61, T)
    wr, bias = lay.wr.copy(), lay.bias.copy()
    ri, _, _ = oracle.route(x, wr, bias, s.n_group, s.topk_group, s.top_k, s.routed_scaling)
    # expert twins: a lower expert of the same group copies each of a few winners
    winners = sorted({int(e) for e in ri[:, :3].ravel() if e % gs})[:12]
    for e in winners:
        wr[e - 1], bias[e - 1] = wr[e], bias[e]
    # group twins: group 1 becomes a copy of the group holding token 0's top pick
    gtop = int(ri[0, 0]) // gs
    if gtop != 1:
        wr[gs:2 * gs], bias[gs:2 * gs] = wr[gtop * gs:(gtop + 1) * gs], bias[gtop * gs:(gtop + 1) * gs]
    ri2, _, _ = _route_and_layer(lay, wr, bias, x, dev)
    ties = 0
    for row in ri2.tolist():
        for a, b in zip(row, row[1:]):
            if a >= 0 and b >= 0 and np.array_equal(wr[a], wr[b]) and bias[a] == bias[b]:
                assert a < b, row
                ties += 1
    assert ties > 0, "no tie was exercised"


# ------------------------------------------------------------------ every code pattern

def pattern_codes(rng, rows, n, fmt, variant):
    """Code matrices that use every code: per row, cycling over families --
    all lowest code, lowest/highest alternating, every code in turn, uniform
    random, and for MXFP4 blocks of +0/-0 only.  FP8: raw E4M3 bytes (as
    int8), every code but the two NaN ones (0x7F, 0xFF)."""
    wb = FORMATS[fmt]
    if wb == synth.MXFP4:
        lo, hi, allc = 15, 7, np.arange(16)  # raw E2M1 codes: 15 = -6, 7 = +6, 8 = -0
    elif wb == synth.FP8:
        allc = np.array([c for c in range(256) if c & 0x7F != 0x7F]).astype(np.uint8).view(np.int8)
        lo, hi = np.int8(np.uint8(0xFE).view(np.int8)), np.int8(0x7E)  # -448, +448
    else:
        lo, hi = -(1 << (wb - 1)), (1 << (wb - 1)) - 1
        allc = np.arange(lo, hi + 1)
    fam = (np.arange(rows) + variant) % (5 if wb == synth.MXFP4 else 4)
    c = np.empty((rows, n), np.int16)
    k = np.arange(n)
    for f in range(5):
        r = fam == f
        m = int(r.sum())
        if not m:
            continue
        if f == 0:
            c[r] = lo
        elif f == 1:
            c[r] = np.where(k % 2 == 0, lo, hi)[None, :]
        elif f == 2:
            c[r] = allc[(k[None, :] + np.arange(m)[:, None]) % allc.size]
        elif f == 3:
            c[r] = rng.choice(allc, (m, n))
        else:  # MXFP4 zero blocks of both signs
            c[r] = np.where(k % 3 == 0, 8, 0)[None, :]
    return c.astype(np.int8)


def pattern_record(shape, fmt, variant):
    """One expert record (the library's layout) built from pattern codes."""
    rng = np.random.default_rng(1000 + variant)
    H, I = shape.hidden, shape.inter
    wb = FORMATS[fmt]
    mats = [pattern_codes(rng, I, H, fmt, variant), pattern_codes(rng, I, H, fmt, variant + 1),
            pattern_codes(rng, H, I, fmt, variant + 2)]
    packed = [oracle.pack(m.ravel(), wb) for m in mats]
    if wb == synth.FP8:  # one fp32 scale per 128x128 block
        sc = [(rng.uniform(0.5, 1.5, (m.shape[0] // 128) * (m.shape[1] // 128)) * 0.02 / 448)
              .astype(np.float32) for m in mats]
        rec = np.concatenate(packed + [v.view(np.uint8) for v in sc])
    elif wb == synth.MXFP4:
        scales = []
        for m in mats:
            rows, n = m.shape
            # ordinary blocks 2^-27 .. 2^-18, so that h (and its Q8_0 scale) stays
            # small enough for 2^127 times that scale to be finite in fp32
            sb = rng.integers(100, 110, (rows, n // 32)).astype(np.uint8)
            blocks = m.reshape(rows, n // 32, 32)
            zero = np.all((blocks == 0) | (blocks == 8), axis=2)
            # extreme scale bytes on blocks whose every code is +0 or -0
            ext = np.where(np.arange(n // 32)[None, :] % 2 == 0, 254, 0).astype(np.uint8)
            scales.append(np.where(zero, ext, sb).astype(np.uint8).ravel())
        rec = np.concatenate(packed + scales)
    else:
        top = float(1 << (wb - 1))
        sc = [(rng.uniform(0.5, 1.5, m.shape[0]) * 0.02 / top).astype(np.float32) for m in mats]
        rec = np.concatenate(packed + [v.view(np.uint8) for v in sc])
    assert rec.size == synth.blob_bytes(shape)
    return rec


def heavy_tokens(shape, T, seed):
    """Tokens with heavy-tailed magnitudes, one all-constant token (every Q8_0
    code +-127) and one with a single huge element per block.  For MXFP4
    every |x| <= 200: with a scale byte of 254 (2^127) on a block, the
    kernels' fp32 product of the two scales overflows once the activation
    scale exceeds 2 (amax 254), and a +-0 block then gives inf * 0."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, shape.hidden)) *
         np.exp2(rng.standard_normal((T, shape.hidden)) * 3)).astype(np.float32)
    if T > 1:
        x[1] = np.where(np.arange(shape.hidden) % 3 == 0, -1.0, 1.0)
    if T > 2:
        x[2, ::32] *= 1e4
    if shape.wbits == synth.MXFP4:
        x = np.clip(x, -200.0, 200.0).astype(np.float32)
    return x


def install_patterns(lay, x, fmt):
    """Pattern records for every expert the tokens select and the shared one."""
    s = lay.shape
    ri, _, _ = oracle.route(x, lay.wr, lay.bias, s.n_group, s.topk_group, s.top_k,
                            s.routed_scaling)
    recs = [pattern_record(s, fmt, v) for v in range(4)]
    for i, e in enumerate(sorted({int(e) for e in ri.ravel()} | {synth.SHARED_ID})):
        lay.set_record(e, recs[i % 4])


def check_ffn_dumps(lay, x, dev):
    """moe_expert_ffn (GEMV below 17 tokens, MFMA above; int2 always GEMV)
    with every dump against the oracle."""
    s = lay.shape
    cfg = moe.Config.of(s)
    T = x.shape[0]
    ri, _, _ = oracle.route(x, lay.wr, lay.bias, s.n_group, s.topk_group, s.top_k,
                            s.routed_scaling)
    q, d = oracle.q8_0(x)
    dbg_d = moe.debug_buffers(cfg, T, dev)
    moe.expert_ffn(cfg, to_d(q, dev), to_d(d, dev), to_d(ri, dev), lay.experts_d, lay.shared_d,
                   debug=dbg_d)
    check_dots(lay, q, d, ri, {k: h(v) for k, v in dbg_d.items()}, f"ffn T={T}")


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_code_patterns_tiny(dev, fmt):
    shape = synth.TINY.with_bits(FORMATS[fmt])
    lay = DeviceLayer(shape, synth.SEEDS["tiny"])
    for e in list(range(shape.n_experts)) + [synth.SHARED_ID]:
        lay.set_record(e, pattern_record(shape, fmt, e % 5))
    for T in (1, 16, 40):
        x = heavy_tokens(shape, T, 90 + T)
        check_ffn_dumps(lay, x, dev)
        check_layer_dumps(lay, x, dev)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_code_patterns_real(dev, fmt):
    """Real shape: the selected experts' records replaced by pattern records;
    the fused path at 1 and 16 tokens, the GEMV/MFMA expert calls at 1 and
    24.  (The module's layer keeps the patterns: later tests re-read every
    record from the device.)"""
    lay = real_layer(fmt)
    for T, path in ((1, "layer"), (16, "layer"), (1, "ffn"), (24, "ffn")):
        x = heavy_tokens(lay.shape, T, 300 + T)
        install_patterns(lay, x, fmt)
        if path == "layer":
            check_layer_dumps(lay, x, dev)
        else:
            check_ffn_dumps(lay, x, dev)


# ------------------------------------------------------------------ workspace contents

@pytest.mark.parametrize("T", [1, 2, 5, 12, 16, 40])
def test_layer_workspace_contents_do_not_matter(dev, T):
    """A workspace full of garbage gives bit-identical outputs to a zeroed
    one (every byte a call reads, it wrote first), call after call."""
    lay = real_layer("int4")
    cfg = moe.Config.of(lay.shape)
    n = moe.layer_workspace(cfg, T)
    g = torch.Generator(device="cpu").manual_seed(T)
    outs = []
    for ws in (torch.zeros(n, dtype=torch.uint8, device=dev),
               torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g).to(dev),
               torch.full((n,), 0xFF, dtype=torch.uint8, device=dev)):
        for rep in range(2):
            x = to_d(synth.tokens(lay.shape, 400 + rep, T), dev)
            res = to_d(synth.tokens(lay.shape, 500 + rep, T), dev)
            idx = torch.empty((T, lay.shape.top_k), dtype=torch.int32, device=dev)
            y, yn = moe.layer(cfg, x, lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                              residual=res, want_norm=True, idx_out=idx, workspace=ws)
            outs.append((rep, h(y), h(yn), h(idx)))
    for rep, y, yn, idx in outs[2:]:
        r0 = outs[rep]
        assert np.array_equal(y, r0[1]) and np.array_equal(yn, r0[2]) and np.array_equal(idx, r0[3])
    x = synth.tokens(lay.shape, 400, T)
    ref = lay.oracle_layer(x, synth.tokens(lay.shape, 500, T), want_norm=True)
    assert np.array_equal(outs[0][3], ref["idx"])
    assert_close_rms(outs[0][1], ref["y"], 2e-3, "y")


# ------------------------------------------------------------------ records through pointers

@pytest.mark.parametrize("fmt,T", [("int4", 1), ("int4", 8), ("int4", 24), ("fp8", 1),
                                   ("fp8", 4)])
def test_layer_ptrs_host_records_against_oracle(dev, fmt, T):
    """moe_layer_ptrs with the selected experts' records in pinned host memory
    (read over the host link) and the rest in HBM, against the oracle, with
    every dump."""
    lay = real_layer(fmt)
    s = lay.shape
    bb = lay.blob_bytes
    x = batch(s, T, 700 + T)
    ri, _, _ = oracle.route(x, lay.wr, lay.bias, s.n_group, s.topk_group, s.top_k,
                            s.routed_scaling)
    sel = sorted({int(e) for e in ri.ravel()})
    host = torch.empty(len(sel) * bb, dtype=torch.uint8, pin_memory=True)
    for i, e in enumerate(sel):
        host[i * bb:(i + 1) * bb].copy_(torch.from_numpy(lay.blob(e)))
    base = moe.host_device_ptr(host)
    addr = [lay.experts_d.data_ptr() + e * bb for e in range(s.n_experts)]
    for i, e in enumerate(sel):
        addr[e] = base + i * bb
    table = torch.tensor(addr, dtype=torch.int64, device=dev)
    check_layer_dumps(lay, x, dev, table=table)
    del host
