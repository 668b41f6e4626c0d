"""Pins of the CPU oracle against things other than itself.

Each test ties one oracle step to a hand-worked fixture (tests/golden/), a
library routine (numpy, math, scipy), a closed form, an invariant, or brute
force on tiny inputs, so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails here.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _half_away(v):
    v = np.asarray(v, np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


# ------------------------------------------------------------------ packed codes

@pytest.mark.parametrize("wbits", [4, 2, 8])
def test_codes_match_hand_table(wbits):
    for case in _load("packed_codes.json")[f"int{wbits}"]:
        row = np.array([case["byte"]], np.uint8)
        got = oracle.unpack(row, wbits, 8 // wbits).tolist()
        assert got == case["codes"], case["derivation"]


def _code_range(wbits):
    return {8: (-128, 127), 4: (-8, 7), 2: (-2, 1)}[wbits]


@pytest.mark.parametrize("wbits", [4, 2, 8])
def test_pack_unpack_round_trip_exhaustive(wbits):
    per = 8 // wbits
    allbytes = np.arange(256, dtype=np.uint8)
    codes = oracle.unpack(allbytes, wbits, 256 * per)
    assert np.array_equal(oracle.pack(codes, wbits), allbytes)
    lo, hi = _code_range(wbits)
    tuples = np.array(list(itertools.product(range(lo, hi + 1), repeat=per)), np.int8).ravel()
    packed = oracle.pack(tuples, wbits)
    assert np.array_equal(oracle.unpack(packed, wbits, tuples.size), tuples)
    # every byte value appears exactly once: the code map is a bijection
    assert sorted(packed.tolist()) == list(range(256))


@pytest.mark.parametrize("wbits", [4, 2, 8])
def test_generated_record_decodes_to_rounded_weights(wbits):
    """The generator's packed rows, read back by the oracle, equal a numpy
    re-quantisation of the generator's float rows (two independent codes)."""
    shape = synth.TINY.with_bits(wbits)
    H, I = shape.hidden, shape.inter
    blob = synth.expert_blob(shape, 7, 3, 5)
    gate, up, down, sg, su, sd = oracle.blob_view(blob, H, I, wbits)
    qdiv, lo, hi = {4: (7.0, -8, 7), 2: (2.0, -2, 1), 8: (127.0, -127, 127)}[wbits]
    for m, (rows, sc, n) in enumerate([(gate, sg, H), (up, su, H), (down, sd, I)]):
        for r in (0, 1, rows.shape[0] - 1):
            w = synth.weight_row(7, 3, 5, m, n, r)
            s = np.float32(np.max(np.abs(w)) / np.float32(qdiv))
            assert sc[r] == s
            want = np.clip(_half_away(w / s), lo, hi).astype(np.int8)
            assert np.array_equal(oracle.unpack(rows[r], wbits, n), want)


def test_record_size_matches_nineteen_megabytes():
    """~19 MB per int4 expert at hidden 6144 / intermediate 2048 (pages'
    streaming section) -> 3*6144*2048/2 code bytes + fp32 row scales."""
    assert oracle.blob_bytes(6144, 2048, 4) == 18_915_328
    assert oracle.blob_bytes(6144, 2048, 2) == 9_478_144
    assert oracle.blob_bytes(6144, 2048, 8) == 37_789_696  # int8 experts: 3*6144*2048 + scales
    assert synth.blob_bytes(synth.REAL) == 18_915_328
    assert synth.blob_bytes(synth.REAL.with_bits(8)) == 37_789_696


# ------------------------------------------------------------------ integer dots

def test_block_dot_single_product_table():
    """All 16 x 255 products code*q as one-element blocks."""
    for c in range(-8, 8):
        codes = np.zeros(32, np.int8)
        codes[5] = c
        row = oracle.pack(codes, 4)
        for v in range(-127, 128):
            q = np.zeros(32, np.int8)
            q[5] = v
            assert oracle.block_dots(row, 4, q)[0] == c * v


@pytest.mark.parametrize("wbits", [4, 2, 8])
def test_block_dots_vs_numpy_int64(wbits):
    rng = np.random.default_rng(1)
    lo, hi = _code_range(wbits)
    n = 32 * 40
    codes = rng.integers(lo, hi + 1, n).astype(np.int8)
    q = rng.integers(-127, 128, n).astype(np.int8)
    got = oracle.block_dots(oracle.pack(codes, wbits), wbits, q)
    want = (codes.astype(np.int64) * q.astype(np.int64)).reshape(-1, 32).sum(1)
    assert np.array_equal(got, want)


def test_block_dot_extremes():
    row = oracle.pack(np.full(32, -8, np.int8), 4)
    assert oracle.block_dots(row, 4, np.full(32, -127, np.int8))[0] == 32512
    assert oracle.block_dots(row, 4, np.full(32, 127, np.int8))[0] == -32512


# ------------------------------------------------------------------ Q8_0

def test_q8_0_hand_blocks():
    for blk in _load("q8_0_blocks.json")["blocks"]:
        x = np.zeros(32, np.float32)
        for k, v in blk["x"].items():
            x[int(k)] = v
        want = np.zeros(32, np.int8)
        for k, v in blk["q"].items():
            want[int(k)] = v
        q, d = oracle.q8_0(x)
        assert d[0] == np.float32(blk["d"]), blk["name"]
        assert np.array_equal(q, want), blk["name"]


def test_q8_0_invariants_random():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((16, 32 * 24)) * rng.uniform(1e-3, 1e3, (16, 1))).astype(np.float32)
    x[3, 64:96] = 0.0
    q, d = oracle.q8_0(x)
    qb = q.reshape(16, -1, 32).astype(np.int64)
    xb = x.reshape(16, -1, 32).astype(np.float64)
    assert np.all(np.abs(qb) <= 127)
    nz = d > 0
    assert np.all(np.abs(qb).max(-1)[nz] == 127)
    assert not nz[3, 2] and np.all(qb[3, 2] == 0)
    err = np.abs(xb - qb * d[..., None].astype(np.float64))
    assert np.all(err <= d[..., None] * (0.5 + 2e-5))
    # d is the correctly rounded amax/127
    amax = np.abs(x.reshape(16, -1, 32)).max(-1)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float32))


def test_q8_0_integer_grid_is_exact():
    rng = np.random.default_rng(3)
    xi = rng.integers(-127, 128, (5, 32 * 8))
    xi.reshape(5, -1, 32)[:, :, 7] = 127
    q, d = oracle.q8_0(xi.astype(np.float32))
    assert np.all(d == 1.0)
    assert np.array_equal(q.astype(np.int64), xi)


# ------------------------------------------------------------------ router arithmetic

def _ulp(v):
    return np.spacing(np.abs(np.float32(v))).astype(np.float64)


def test_exp_canon_within_two_ulp():
    ys = np.linspace(-87.0, 87.0, 20001, dtype=np.float32)
    got = oracle.exp_canon(ys).astype(np.float64)
    want = np.exp(ys.astype(np.float64))
    ulps = np.abs(got - want) / _ulp(want.astype(np.float32))
    assert ulps.max() <= 2.0
    assert oracle.exp_canon([0.0])[0] == 1.0


def test_sigmoid_canon_closed_forms():
    ls = np.linspace(-20, 20, 4001, dtype=np.float32)
    got = oracle.sigmoid_canon(ls).astype(np.float64)
    want = expit(ls.astype(np.float64))
    assert np.max(np.abs(got - want) / _ulp(want.astype(np.float32))) <= 3.0
    assert oracle.sigmoid_canon([0.0])[0] == 0.5
    sym = got + oracle.sigmoid_canon(-ls).astype(np.float64)
    assert np.max(np.abs(sym - 1.0)) <= 2.5e-7


def test_dot_canon_error_bound():
    rng = np.random.default_rng(4)
    for n in (64, 256, 6144):
        a = rng.standard_normal(n).astype(np.float32)
        b = (rng.standard_normal(n) * 0.02).astype(np.float32)
        exact = math.fsum((a.astype(np.float64) * b.astype(np.float64)).tolist())
        bound = n * 2.0 ** -24 * float(np.sum(np.abs(a.astype(np.float64) * b)))
        assert abs(float(oracle.dot_canon(a, b)) - exact) <= bound


def test_router_scores_match_definition():
    """s = sigmoid(x . W_r[e]) to fp32 accuracy and sb = s + bias, against fp64 numpy."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    wr = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, 8).astype(np.float32)
    s, sb = oracle.router_scores(x, wr, bias)
    ref = expit(x.astype(np.float64) @ wr.astype(np.float64).T)
    assert np.max(np.abs(s - ref)) < 1e-6
    assert np.array_equal(sb, (s + bias).astype(np.float32))


# ------------------------------------------------------------------ selection

def test_select_hand_cases():
    for c in _load("router_cases.json")["cases"]:
        s = np.array([c["s"]], np.float32)
        sb = np.array([c["sb"]], np.float32)
        idx, w, margin = oracle.select(s, sb, c["G"], c["TG"], c["K"], c["scale"])
        assert idx[0].tolist() == c["idx"], c["name"]
        assert np.allclose(w[0], np.array(c["w"], np.float32), rtol=0, atol=1e-7), c["name"]
        if "margin" in c:  # dyadic cases: exact
            want = [math.inf if m == "inf" else m for m in c["margin"]]
            assert margin[0].tolist() == want, c["name"]


@pytest.mark.parametrize("E,G,TG,K", [(8, 2, 1, 2), (16, 4, 2, 3), (256, 8, 4, 8), (12, 3, 3, 4)])
def test_select_margins_vs_sorted_scores(E, G, TG, K):
    """The selection margins against their definition, from sorted lists: the
    K-th largest biased score of the kept groups minus the (K+1)-th, and the
    TG-th largest group score (sum of the group's two largest, fp32) minus
    the (TG+1)-th; +inf when nothing is left out.  Also on grid values with
    many exact ties (margins 0)."""
    rng = np.random.default_rng(E + 7 * K)
    gs = E // G
    for trial in range(100):
        if trial % 2:
            sb = (rng.integers(0, 8, (1, E)) / 8.0).astype(np.float32)
        else:
            sb = rng.uniform(-0.1, 1.1, (1, E)).astype(np.float32)
        s = np.full((1, E), 0.5, np.float32)
        idx, _, margin = oracle.select(s, sb, G, TG, K, 1.0)
        v = sb[0]
        gsc = [np.float32(np.sort(v[g * gs:(g + 1) * gs])[-1] + np.sort(v[g * gs:(g + 1) * gs])[-2])
               for g in range(G)]
        order = sorted(range(G), key=lambda g: (-float(gsc[g]), g))
        kept = order[:TG]
        mg = float(gsc[order[TG - 1]]) - float(gsc[order[TG]]) if TG < G else math.inf
        cand = np.sort(np.concatenate([v[g * gs:(g + 1) * gs] for g in kept]).astype(np.float64))[::-1]
        mp = cand[K - 1] - cand[K] if K < cand.size else math.inf
        assert margin[0, 0] == mp and margin[0, 1] == mg, (trial, margin[0], mp, mg)
        assert margin[0, 0] >= 0 and margin[0, 1] >= 0
        # a zero pick margin means the K-th pick ties a left-out candidate
        if mp == 0:
            assert any(v[e] == v[idx[0, K - 1]] for e in range(E)
                       if e // gs in kept and e not in idx[0])


@pytest.mark.parametrize("E,G,TG,K", [(8, 2, 1, 2), (8, 4, 2, 3), (16, 4, 2, 3), (12, 3, 2, 4)])
def test_select_vs_subset_enumeration(E, G, TG, K):
    """With distinct scores, the kept groups are the TG-subset of largest total
    group score and the picks are the K-subset of largest total biased score."""
    rng = np.random.default_rng(E * 100 + K)
    gs = E // G
    for _ in range(200):
        s = rng.uniform(0.01, 1.0, (1, E)).astype(np.float32)
        sb = (s + rng.uniform(-0.1, 0.1, (1, E)).astype(np.float32)).astype(np.float32)
        idx, w, _ = oracle.select(s, sb, G, TG, K, 2.5)
        v = sb[0].astype(np.float64)
        gscore = [sum(sorted(v[g * gs:(g + 1) * gs])[-2:]) for g in range(G)]
        best_groups = max(itertools.combinations(range(G), TG),
                          key=lambda c: sum(gscore[g] for g in c))
        cands = [e for e in range(E) if e // gs in best_groups]
        best = max(itertools.combinations(cands, K), key=lambda c: sum(v[e] for e in c))
        assert set(idx[0].tolist()) == set(best)
        assert idx[0].tolist() == sorted(best, key=lambda e: (-v[e], e))
        # weights use the unbiased score, normalised, times the scale
        sel = s[0, idx[0]].astype(np.float64)
        assert np.allclose(w[0], sel / sel.sum() * 2.5, rtol=3e-7, atol=0)


def test_select_single_group_is_plain_top_k():
    rng = np.random.default_rng(6)
    for _ in range(100):
        s = rng.uniform(0, 1, (1, 16)).astype(np.float32)
        s[0, 3] = s[0, 9]  # a tie
        idx, _, _ = oracle.select(s, s, 1, 1, 5, 1.0)
        want = np.argsort(-s[0].astype(np.float64), kind="stable")[:5]
        assert idx[0].tolist() == want.tolist()


def test_zero_bias_single_group_is_top_k_of_logits():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    wr = (rng.standard_normal((16, 128)) * 0.1).astype(np.float32)
    idx, _, _ = oracle.route(x, wr, np.zeros(16, np.float32), 1, 1, 4, 1.0)
    logits = x.astype(np.float64) @ wr.astype(np.float64).T
    for t in range(4):
        assert idx[t].tolist() == np.argsort(-logits[t], kind="stable")[:4].tolist()


def test_normalisation_identity():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    wr = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    bias = rng.uniform(-0.1, 0.1, 32).astype(np.float32)
    _, w, _ = oracle.route(x, wr, bias, 4, 2, 8, 2.5)
    # each w_k carries <= 2 roundings, S carries K-1: |sum w - 2.5| <= 2.5 * (K+2) * 2^-24
    assert np.max(np.abs(w.astype(np.float64).sum(1) - 2.5)) <= 2.5 * 10 * 2.0 ** -24
    assert np.all(w > 0)


def test_uniform_bias_shift_keeps_selection_and_weights():
    rng = np.random.default_rng(9)
    for _ in range(50):
        # grid values so that adding 0.125 is exact in fp32
        s = (rng.integers(256, 768, (1, 32)) / 1024.0).astype(np.float32)
        b = (rng.integers(-64, 64, (1, 32)) / 1024.0).astype(np.float32)
        sb = s + b
        idx1, w1, _ = oracle.select(s, sb, 4, 2, 6, 2.5)
        idx2, w2, _ = oracle.select(s, (sb + np.float32(0.125)).astype(np.float32), 4, 2, 6, 2.5)
        assert np.array_equal(idx1, idx2) and np.array_equal(w1, w2)


def test_crafted_tie_rows_pick_lower_index():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((2, 128)).astype(np.float32)
    wr = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    wr[5] = wr[1]  # identical router rows, identical biases
    wr[1] *= 40.0  # make them the winners
    wr[5] = wr[1]
    bias = np.zeros(8, np.float32)
    x[0] = np.abs(x[0]) * np.sign(wr[1])  # positive logit for experts 1 and 5
    idx, _, _ = oracle.route(x[:1], wr, bias, 1, 1, 1, 1.0)
    assert idx[0, 0] == 1


# ------------------------------------------------------------------ adaptive top-p

def _select_top_p(s, sb, G, TG, K, scale, p):
    idx, w, _ = oracle.select(s, sb, G, TG, K, scale)
    return oracle.top_p(s, idx, w, p, scale)


def test_top_p_hand_cases():
    for c in _load("top_p_cases.json")["cases"]:
        s = np.array([c["s"]], np.float32)
        sb = (s + np.array([c["bias"]], np.float32)).astype(np.float32)
        idx, w, kept = _select_top_p(s, sb, 1, 1, c["K"], c["scale"], c["p"])
        assert idx[0].tolist() == c["idx"], c["name"]
        want = np.array([a / b for a, b in c["w_num"]])
        assert np.max(np.abs(w[0] - want)) <= 1e-6, c["name"]
        assert kept[0] == sum(i >= 0 for i in c["idx"]), c["name"]


def test_top_p_vs_exact_prefix_definition():
    """The kept prefix is the shortest one whose exact share of the selected
    unbiased mass reaches p (cases within 1e-5 of the threshold skipped)."""
    rng = np.random.default_rng(21)
    checked = 0
    for _ in range(400):
        E, K = 16, int(rng.integers(1, 9))
        s = rng.uniform(0.01, 1.0, (1, E)).astype(np.float32)
        sb = (s + rng.uniform(-0.1, 0.1, (1, E)).astype(np.float32)).astype(np.float32)
        p = float(np.float32(rng.uniform(0.05, 0.95)))
        idx0, _, _ = oracle.select(s, sb, 4, 2, K, 2.5)
        idx, w, kept = oracle.top_p(s, idx0, np.zeros_like(idx0, np.float32), p, 2.5)
        sel = s[0, idx0[0]].astype(np.float64)
        share = np.cumsum(sel) / sel.sum()
        if np.min(np.abs(share - p)) < 1e-5:
            continue
        n = int(np.argmax(share >= p)) + 1
        assert kept[0] == n
        assert idx[0, :n].tolist() == idx0[0, :n].tolist()
        assert np.all(idx[0, n:] == -1) and np.all(w[0, n:] == 0)
        assert np.allclose(w[0, :n], sel[:n] / sel[:n].sum() * 2.5, rtol=3e-7, atol=0)
        checked += 1
    assert checked > 300


def test_top_p_off_values_keep_plain_selection():
    rng = np.random.default_rng(22)
    s = rng.uniform(0.01, 1.0, (8, 32)).astype(np.float32)
    sb = (s + rng.uniform(-0.1, 0.1, (8, 32)).astype(np.float32)).astype(np.float32)
    idx0, w0, _ = oracle.select(s, sb, 4, 2, 8, 2.5)
    for p in (0.0, 1.0):
        idx, w, kept = oracle.top_p(s, idx0, w0, p, 2.5)
        assert np.array_equal(idx, idx0) and np.array_equal(w, w0) and np.all(kept == 8)


def test_top_p_renormalisation_and_monotone_count():
    rng = np.random.default_rng(23)
    s = rng.uniform(0.01, 1.0, (64, 32)).astype(np.float32)
    sb = (s + rng.uniform(-0.1, 0.1, (64, 32)).astype(np.float32)).astype(np.float32)
    idx0, w0, _ = oracle.select(s, sb, 4, 2, 8, 2.5)
    last = np.ones(64, np.int32)
    for p in (0.1, 0.3, 0.5, 0.7, 0.9, 0.99):
        idx, w, kept = oracle.top_p(s, idx0, w0, p, 2.5)
        assert np.all(kept >= last) and np.all(kept >= 1) and np.all(kept <= 8)
        last = kept
        # kept weights sum to the scale (each carries <= 2 roundings, S_kept K-1)
        assert np.max(np.abs(w.astype(np.float64).sum(1) - 2.5)) <= 2.5 * 10 * 2.0 ** -24
        assert np.array_equal((idx >= 0).sum(1), kept)


def test_group_skips_dropped_slots():
    rng = np.random.default_rng(24)
    for T, K, E in [(1, 8, 256), (16, 8, 256), (37, 3, 10), (2048, 8, 256)]:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
        keep = rng.integers(1, K + 1, T)
        for t in range(T):
            idx[t, keep[t]:] = -1
        g = oracle.group(idx, E)
        flat = idx.ravel()
        valid = np.nonzero(flat >= 0)[0]
        n = valid.size
        assert g["offsets"][E] == n
        assert np.array_equal(g["perm"][:n], valid[np.argsort(flat[valid], kind="stable")])
        assert np.all(g["perm"][n:] == -1)
        assert np.all(g["inv"][flat < 0] == -1)
        assert np.array_equal(g["inv"][g["perm"][:n]], np.arange(n))
        assert np.array_equal(g["counts"], np.bincount(flat[valid], minlength=E))


def test_layer_top_p_identical_experts_closed_form():
    """Kept weights are renormalised, so with identical routed experts the
    layer is still shared(x) + 2.5 * expert(x) whatever top-p drops."""
    shape = synth.TINY
    blob = synth.expert_blob(shape, 100, 0, 0)
    shared = synth.expert_blob(shape, 100, 0, synth.SHARED_ID)
    x = synth.tokens(shape, 100, 6)
    wr = synth.router_weights(shape, 100)
    bias = synth.router_bias_uniform(shape, 100)
    out = oracle.layer(x, wr, bias, lambda e: blob, shared, H=256, I=128, n_experts=8,
                       n_group=2, topk_group=1, top_k=2, scale=2.5, top_p_value=0.5)
    assert np.any(out["idx"] < 0)  # the cut drops something here
    for t in range(6):
        e_y = oracle.expert(blob, 256, 128, 4, out["q"][t], out["d"][t])["y"].astype(np.float64)
        ref = out["shared_out"][t].astype(np.float64) + 2.5 * e_y
        assert np.max(np.abs(out["y"][t] - ref)) <= 1e-6 * np.sqrt(np.mean(ref ** 2)) + 1e-7


# ------------------------------------------------------------------ grouping

def test_group_vs_stable_argsort():
    rng = np.random.default_rng(11)
    for T, K, E in [(1, 8, 256), (4, 2, 8), (16, 8, 256), (2048, 8, 256), (37, 3, 10)]:
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]).astype(np.int32)
        if T >= 4:
            idx[T // 2] = idx[0]  # a duplicated token
        g = oracle.group(idx, E)
        flat = idx.ravel()
        assert np.array_equal(g["perm"], np.argsort(flat, kind="stable"))
        assert np.array_equal(g["counts"], np.bincount(flat, minlength=E))
        assert np.array_equal(g["offsets"], np.concatenate([[0], np.cumsum(g["counts"])]))
        assert np.array_equal(g["inv"][g["perm"]], np.arange(T * K))
        act = np.nonzero(g["counts"])[0]
        assert g["n_active"] == act.size and np.array_equal(g["active"][:act.size], act)
        assert np.all(g["active"][act.size:] == -1)


def test_group_rejects_out_of_range_expert():
    with pytest.raises(ValueError):
        oracle.group(np.array([[0, 9]], np.int32), 8)


# ------------------------------------------------------------------ expert FFN

def _tiny_inputs(seed=12, T=3, wbits=4):
    shape = synth.TINY.with_bits(wbits)
    blob = synth.expert_blob(shape, seed, 0, 1)
    x = synth.tokens(shape, seed, T)
    q, d = oracle.q8_0(x)
    return shape, blob, x, q, d


@pytest.mark.parametrize("wbits", [4, 2, 8])
def test_gate_up_equals_dequantised_matmul(wbits):
    """Integer block dots rescaled == fp64 matmul of dequantised weights and
    dequantised activations (algebraic identity), and h = silu(g) * u."""
    shape, blob, x, q, d = _tiny_inputs(wbits=wbits)
    H, I = shape.hidden, shape.inter
    gate, up, _, sg, su, _ = oracle.blob_view(blob, H, I, wbits)
    Wg = np.stack([oracle.unpack(gate[r], wbits, H) for r in range(I)]).astype(np.float64)
    Wu = np.stack([oracle.unpack(up[r], wbits, H) for r in range(I)]).astype(np.float64)
    Wg *= sg[:, None]
    Wu *= su[:, None]
    for t in range(q.shape[0]):
        a = q[t].astype(np.float64) * np.repeat(d[t].astype(np.float64), 32)
        out = oracle.gate_up(blob, H, I, wbits, q[t], d[t], want_dots=True)
        g_ref, u_ref = Wg @ a, Wu @ a
        assert np.allclose(out["g"], g_ref, rtol=1e-12, atol=1e-15)
        assert np.allclose(out["u"], u_ref, rtol=1e-12, atol=1e-15)
        h_ref = (g_ref * expit(g_ref) * u_ref).astype(np.float32)
        assert np.max(np.abs(out["h"] - h_ref)) <= np.max(np.abs(h_ref)) * 1e-6
        # dots: integer GEMV of the codes against q, blockwise
        codes = np.stack([oracle.unpack(gate[r], wbits, H) for r in range(I)]).astype(np.int64)
        want = (codes * q[t].astype(np.int64)).reshape(I, -1, 32).sum(-1)
        assert np.array_equal(out["gate_dots"], want)


@pytest.mark.parametrize("wbits", [4, 2, 8])
def test_down_equals_dequantised_matmul(wbits):
    shape, blob, x, q, d = _tiny_inputs(wbits=wbits)
    H, I = shape.hidden, shape.inter
    _, _, down, _, _, sd = oracle.blob_view(blob, H, I, wbits)
    Wd = np.stack([oracle.unpack(down[j], wbits, I) for j in range(H)]).astype(np.float64)
    Wd *= sd[:, None]
    h = oracle.gate_up(blob, H, I, wbits, q[0], d[0])["h"]
    qh, dh = oracle.q8_0(h)
    y, dots = oracle.down(blob, H, I, wbits, qh, dh, want_dots=True)
    ref = Wd @ (qh.astype(np.float64) * np.repeat(dh.astype(np.float64), 32))
    assert np.allclose(y, ref.astype(np.float32), rtol=1e-6, atol=1e-9)
    assert dots.shape == (H, I // 32)


def test_expert_chain_quantises_h():
    shape, blob, x, q, d = _tiny_inputs()
    out = oracle.expert(blob, shape.hidden, shape.inter, 4, q[1], d[1])
    qh, dh = oracle.q8_0(out["h"])
    assert np.array_equal(out["qh"], qh) and np.array_equal(out["dh"], dh)
    y, _ = oracle.down(blob, shape.hidden, shape.inter, 4, qh, dh)
    assert np.array_equal(out["y"], y)


def test_grid_exact_ffn_dots_are_textbook_gemv():
    """Integer-valued activations with block amax 127 (d = 1) and unit row
    scales: g equals the plain integer GEMV of the codes."""
    H, I = 256, 64
    rng = np.random.default_rng(13)
    codes = rng.integers(-8, 8, (3, I if True else 0, H)).astype(np.int8)
    gate = np.concatenate([oracle.pack(codes[0, r], 4) for r in range(I)])
    up = np.concatenate([oracle.pack(codes[1, r], 4) for r in range(I)])
    dcodes = rng.integers(-8, 8, (H, I)).astype(np.int8)
    down = np.concatenate([oracle.pack(dcodes[j], 4) for j in range(H)])
    scales = np.ones(2 * I + H, np.float32)
    blob = np.concatenate([gate, up, down, scales.view(np.uint8)])
    xi = rng.integers(-127, 128, H)
    xi.reshape(-1, 32)[:, 0] = 127
    q, d = oracle.q8_0(xi.astype(np.float32))
    out = oracle.gate_up(blob, H, I, 4, q, d)
    assert np.array_equal(out["g"], (codes[0].astype(np.int64) @ xi).astype(np.float64))
    assert np.array_equal(out["u"], (codes[1].astype(np.int64) @ xi).astype(np.float64))


# ------------------------------------------------------------------ combine and layer

def test_combine_vs_numpy():
    rng = np.random.default_rng(14)
    T, K, H = 3, 4, 64
    eo = rng.standard_normal((T, K, H)).astype(np.float32)
    w = rng.uniform(0, 1, (T, K)).astype(np.float32)
    sh = rng.standard_normal((T, H)).astype(np.float32)
    res = rng.standard_normal((T, H)).astype(np.float32)
    y = oracle.combine(eo, w, sh)
    ref = sh.astype(np.float64) + np.einsum("tk,tkh->th", w.astype(np.float64), eo)
    assert np.allclose(y, ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    y2, yn = oracle.combine(eo, w, sh, res, want_norm=True)
    ref2 = ref + res
    assert np.allclose(y2, ref2.astype(np.float32), rtol=1e-6, atol=1e-7)
    ms = np.mean(ref2 ** 2, axis=1, keepdims=True)
    assert np.allclose(yn, ref2 / np.sqrt(ms + 1e-5), rtol=1e-6, atol=1e-7)
    # scale invariance of the norm (eps negligible at this scale)
    assert np.allclose(oracle.rmsnorm(8 * y2), oracle.rmsnorm(y2), rtol=1e-5, atol=1e-6)


def _tiny_layer(blob_of, shared, T=4, seed=100):
    shape = synth.TINY
    x = synth.tokens(shape, seed, T)
    wr = synth.router_weights(shape, seed)
    bias = synth.router_bias_uniform(shape, seed)
    return oracle.layer(x, wr, bias, blob_of, shared, H=shape.hidden, I=shape.inter,
                        n_experts=shape.n_experts, n_group=shape.n_group,
                        topk_group=shape.topk_group, top_k=shape.top_k,
                        scale=shape.routed_scaling)


def test_layer_identical_experts_closed_form():
    """All routed experts identical -> y = shared(x) + 2.5 * expert(x)."""
    blob = synth.expert_blob(synth.TINY, 100, 0, 0)
    shared = synth.expert_blob(synth.TINY, 100, 0, synth.SHARED_ID)
    out = _tiny_layer(lambda e: blob, shared)
    for t in range(4):
        e_y = oracle.expert(blob, 256, 128, 4, out["q"][t], out["d"][t])["y"].astype(np.float64)
        ref = out["shared_out"][t].astype(np.float64) + 2.5 * e_y
        assert np.max(np.abs(out["y"][t] - ref)) <= 1e-6 * np.sqrt(np.mean(ref ** 2)) + 1e-7


def test_layer_zero_routed_experts_gives_shared_only():
    zero = synth.expert_blob(synth.TINY, 100, 0, 0)
    nb = 3 * 256 * 128 // 2
    zero[:nb] = 0  # all codes 0, scales kept
    shared = synth.expert_blob(synth.TINY, 100, 0, synth.SHARED_ID)
    out = _tiny_layer(lambda e: zero, shared)
    assert np.all(out["expert_out"] == 0)
    assert np.array_equal(out["y"], out["shared_out"])


def test_layer_places_each_expert_output_at_its_slot():
    """Distinct routed experts: expert e is expert 0 with its down-row scales
    times 2^e (so its output is exactly 2^e E0(x)).  Then, whatever the
    grouping does, y[t] = S(x_t) + E0(x_t) * sum_k w[t,k] 2^idx[t,k]: an output
    written to another rank's or token's slot breaks the sum.  Also every
    expert_out row is the expert of its (t, k) slot applied to token t."""
    shape = synth.TINY
    H, I, E = shape.hidden, shape.inter, shape.n_experts
    base = synth.expert_blob(shape, 100, 0, 0)
    ds_off = 3 * I * H // 2 + 2 * I * 4  # the down-row scales of an int4 record

    def blob_of(e):
        b = base.copy()
        b[ds_off:].view(np.float32)[:] *= np.float32(2.0 ** e)
        return b

    shared = synth.expert_blob(shape, 100, 0, synth.SHARED_ID)
    x = synth.tokens(shape, 55, 16)
    wr = synth.router_weights(shape, 55)
    bias = synth.router_bias_uniform(shape, 55)
    for p in (0.0, 0.6):
        out = oracle.layer(x, wr, bias, blob_of, shared, H=H, I=I, n_experts=E,
                           n_group=shape.n_group, topk_group=shape.topk_group, top_k=shape.top_k,
                           scale=shape.routed_scaling, top_p_value=p)
        idx, w = out["idx"], out["w"]
        assert len({tuple(r) for r in idx.tolist()}) > 3  # varied placements
        for t in range(16):
            e0 = oracle.expert(base, H, I, 4, out["q"][t], out["d"][t])["y"].astype(np.float64)
            mult = sum(float(w[t, k]) * 2.0 ** idx[t, k] for k in range(shape.top_k) if idx[t, k] >= 0)
            ref = out["shared_out"][t].astype(np.float64) + mult * e0
            assert np.max(np.abs(out["y"][t] - ref)) <= 1e-6 * np.sqrt(np.mean(ref ** 2))
            for k in range(shape.top_k):
                if idx[t, k] < 0:
                    assert np.all(out["expert_out"][t, k] == 0)
                    continue
                assert np.array_equal(out["expert_out"][t, k],
                                      (e0 * 2.0 ** idx[t, k]).astype(np.float32)), (t, k)


def test_layer_groups_cover_every_slot_once():
    shape = synth.TINY
    blobs = {}

    def blob_of(e):
        blobs[e] = blobs.get(e) or 0
        blobs[e] += 1
        return synth.expert_blob(shape, 100, 0, e)

    out = _tiny_layer(blob_of, None)
    g = out["groups"]
    # batch union: every distinct expert is fetched exactly once
    assert sorted(blobs) == sorted(set(out["idx"].ravel().tolist()))
    assert all(v == 1 for v in blobs.values())
    assert g["counts"].sum() == out["idx"].size


# ------------------------------------------------------------------ MXFP4 experts (R16)

MX = oracle.MXFP4


def test_fp4_and_e8m0_hand_values():
    g = _load("mxfp4_codes.json")
    for c in g["fp4"]:
        assert oracle.fp4_value(c["code"]) == c["value"], c
    for c in g["e8m0"]:
        assert oracle.e8m0_value(c["s"]) == c["value"], c
    p = g["packing"]
    assert oracle.pack(np.array(p["codes"], np.int8), MX).tolist() == p["bytes"]
    assert oracle.unpack(np.array(p["bytes"], np.uint8), MX, 4).tolist() == p["codes"]


def test_mx_pack_unpack_exhaustive():
    codes = np.array([(a, b) for a in range(16) for b in range(16)], np.int8).ravel()
    packed = oracle.pack(codes, MX)
    assert np.array_equal(oracle.unpack(packed, MX, codes.size), codes)
    assert np.array_equal(np.sort(packed), np.arange(256))


def _fp4_grid_nearest(v):
    """Nearest FP4 magnitude by direct search; ties to the even mantissa."""
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    best = min(range(8), key=lambda m: (abs(abs(v) - mags[m]), m % 2))
    return best


def test_generated_mx_record_is_the_block_quantisation():
    shape = synth.TINY.with_bits(MX)
    blob = synth.expert_blob(shape, 41, 0, 3)
    assert blob.size == oracle.blob_bytes(256, 128, MX) == synth.blob_bytes(shape)
    gate, up, down, bg, bu, bd = oracle.blob_view(blob, 256, 128, MX)
    for m, (codes, scl, n) in enumerate(((gate, bg, 256), (down, bd, 128))):
        mat = 0 if m == 0 else 2
        for r in (0, 5, codes.shape[0] - 1):
            w = np.empty(n, np.float32)
            synth.lib().synth_weight_row(41, 0, 3, mat, n, r, synth.WEIGHT_SIGMA,
                                         w.ctypes.data)
            c = oracle.unpack(codes[r], MX, n)
            for b in range(n // 32):
                wb = w[32 * b:32 * (b + 1)].astype(np.float64)
                X = int(scl[r, b]) - 127
                amax = np.max(np.abs(wb))
                # the block maximum lands in [4, 8) before rounding (X = floor(log2 amax) - 2)
                assert 4.0 <= amax / 2.0 ** X < 8.0
                for k in range(32):
                    v = wb[k] / 2.0 ** X
                    mag = min(_fp4_grid_nearest(v), 7)
                    want = 0 if mag == 0 else mag | (8 if v < 0 else 0)
                    assert c[32 * b + k] == want, (m, r, b, k, v)


def test_mx_block_dots_vs_numpy():
    rng = np.random.default_rng(15)
    for _ in range(20):
        codes = rng.integers(0, 16, 64).astype(np.int8)
        q = rng.integers(-127, 128, 64).astype(np.int8)
        got = oracle.block_dots(oracle.pack(codes, MX), MX, q)
        twice = np.array([2.0 * oracle.fp4_value(int(c)) for c in codes]).astype(np.int64)
        want = (twice * q.astype(np.int64)).reshape(2, 32).sum(1)
        assert np.array_equal(got, want)


def test_mx_gate_up_equals_dequantised_matmul():
    shape = synth.TINY.with_bits(MX)
    blob = synth.expert_blob(shape, 42, 0, 1)
    x = synth.tokens(shape, 42, 2)
    q, d = oracle.q8_0(x)
    gate, up, down, bg, bu, bd = oracle.blob_view(blob, 256, 128, MX)
    fp4 = np.array([oracle.fp4_value(c) for c in range(16)])
    for t in range(2):
        xq = q[t].astype(np.float64) * np.repeat(d[t].astype(np.float64), 32)
        ref = oracle.gate_up(blob, 256, 128, MX, q[t], d[t])
        for codes, scl, got in ((gate, bg, ref["g"]), (up, bu, ref["u"])):
            W = fp4[np.stack([oracle.unpack(codes[r], MX, 256) for r in range(128)])]
            W = W * np.repeat(2.0 ** (scl.astype(np.float64) - 127), 32, axis=1)
            assert np.max(np.abs(W @ xq - got)) <= 1e-12 * np.max(np.abs(got))


def test_mx_grid_exact_dots():
    """Codes 0..7 with scale 2^0 and integer activations (amax 127 -> d = 1):
    the rows are the textbook dot of the FP4 values with the integers."""
    H, I = 256, 128
    rng = np.random.default_rng(16)
    blob = np.zeros(oracle.blob_bytes(H, I, MX), np.uint8)
    gate, up, down, bg, bu, bd = oracle.blob_view(blob, H, I, MX)
    codes = rng.integers(0, 16, (I, H)).astype(np.int8)
    gate[:] = np.stack([oracle.pack(r, MX) for r in codes])
    bg[:] = 127
    x = rng.integers(-126, 127, (1, H)).astype(np.float32)
    x[0, ::32] = 127.0  # amax 127 in every block
    q, d = oracle.q8_0(x)
    assert np.all(d == 1.0) and np.array_equal(q[0], x[0].astype(np.int8))
    ref = oracle.gate_up(blob, H, I, MX, q[0], d[0], want_dots=True)
    fp4 = np.array([oracle.fp4_value(c) for c in range(16)])
    assert np.array_equal(ref["g"], fp4[codes] @ x[0].astype(np.float64))


# ------------------------------------------------------------------ per-row activations (R17)

ROW = oracle.ACT_ROW


def test_quant_rows_hand_case():
    """Worked by hand: a row of 64 whose amax is 254 has d = 254/127 = 2 and
    id = 0.5; codes are roundf(x/2), halves away from zero, clamped."""
    x = np.zeros(64, np.float32)
    x[:8] = [254.0, -254.0, 1.0, -1.0, 3.0, -5.0, 0.99, 100.5]
    q, d = oracle.quant_act(x, ROW)
    assert d.tolist() == [2.0]
    assert q[:8].tolist() == [127, -127, 1, -1, 2, -3, 0, 50]
    assert not q[8:].any()


def test_quant_rows_invariants():
    rng = np.random.default_rng(21)
    for n in (64, 2048, 6144):
        x = (rng.standard_normal((8, n)) * np.exp2(rng.integers(-20, 20, (8, 1)))).astype(np.float32)
        x[3] = 0.0
        q, d = oracle.quant_act(x, ROW)
        assert d.shape == (8, 1)
        assert np.all(np.abs(q.astype(np.int32)) <= 127)
        for r in range(8):
            if r == 3:
                assert d[r, 0] == 0 and not q[r].any()
                continue
            assert np.abs(q[r].astype(np.int32)).max() == 127
            err = np.abs(x[r].astype(np.float64) - q[r] * np.float64(d[r, 0]))
            assert err.max() <= d[r, 0] / 2 * (1 + 2.0 ** -22)


def test_quant_rows_integer_grid_is_exact():
    rng = np.random.default_rng(22)
    x = rng.integers(-127, 128, (4, 2048)).astype(np.float32)
    x[:, 5] = 127.0
    q, d = oracle.quant_act(x, ROW)
    assert np.all(d == 1.0) and np.array_equal(q, x.astype(np.int8))


def test_quant_rows_of_32_is_q8_0():
    """A row of 32 values is one Q8_0 block: both formats give the same bits."""
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((50, 32)) * 3).astype(np.float32)
    assert all(np.array_equal(a, b) for a, b in zip(oracle.quant_act(x, ROW), oracle.q8_0(x)))


@pytest.mark.parametrize("wbits", [4, 8, 2])
def test_row_dots_are_sums_of_block_dots(wbits):
    """The whole-row integer dot is the sum of the pinned 32-block dots and the
    int64 brute force (no int32 overflow at the real width, extreme codes)."""
    rng = np.random.default_rng(24 + wbits)
    lo, hi = -(1 << (wbits - 1)), (1 << (wbits - 1)) - 1
    for n in (256, 6144):
        codes = rng.integers(lo, hi + 1, n).astype(np.int8)
        codes[:n // 2] = lo  # the largest magnitude
        q = rng.integers(-127, 128, n).astype(np.int8)
        q[:n // 2] = -127
        row = oracle.pack(codes, wbits)
        p_row = oracle.act_dots(row, wbits, q, ROW)
        assert p_row.shape == (1,)
        assert int(p_row[0]) == int(oracle.block_dots(row, wbits, q).astype(np.int64).sum())
        assert int(p_row[0]) == int(codes.astype(np.int64) @ q.astype(np.int64))


@pytest.mark.parametrize("wbits", [4, 8])
def test_row_format_gate_up_and_down_equal_dequantised_matmul(wbits):
    """g = s_r * d * P_row equals the fp64 product of the dequantised weights
    and activations (algebraic identity), as does the down projection."""
    shape = synth.TINY.with_bits(wbits)
    H, I = shape.hidden, shape.inter
    blob = synth.expert_blob(shape, 31, 0, 2)
    gate, up, down, sg, su, sd = oracle.blob_view(blob, H, I, wbits)
    x = synth.tokens(shape, 31, 1)[0]
    q, d = oracle.quant_act(x, ROW)
    xv = q.astype(np.float64) * np.float64(d[0])
    r = oracle.gate_up(blob, H, I, wbits, q, d, want_dots=True, act_block=ROW)
    Wg = np.stack([oracle.unpack(gate[i], wbits, H) for i in range(I)]).astype(np.float64)
    Wu = np.stack([oracle.unpack(up[i], wbits, H) for i in range(I)]).astype(np.float64)
    g_ref = (Wg * sg[:, None].astype(np.float64)) @ xv
    u_ref = (Wu * su[:, None].astype(np.float64)) @ xv
    assert np.allclose(r["g"], g_ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["u"], u_ref, rtol=1e-12, atol=1e-12)
    assert r["gate_dots"].shape == (I, 1)
    assert np.array_equal(r["gate_dots"][:, 0], (Wg @ q.astype(np.float64)).astype(np.int64))
    qh, dh = oracle.quant_act(r["h"], ROW)
    y, dd = oracle.down(blob, H, I, wbits, qh, dh, want_dots=True, act_block=ROW)
    Wd = np.stack([oracle.unpack(down[j], wbits, I) for j in range(H)]).astype(np.float64)
    y_ref = (Wd * sd[:, None].astype(np.float64)) @ (qh.astype(np.float64) * np.float64(dh[0]))
    assert np.allclose(y, y_ref.astype(np.float32), rtol=1e-6, atol=1e-7)
    assert np.array_equal(dd[:, 0], (Wd @ qh.astype(np.float64)).astype(np.int64))


def test_formats_agree_when_every_block_holds_the_row_max():
    """If every 32-block of a row reaches the row's amax, Q8_0 and the per-row
    format give the same codes and scales, and the same gate/up values."""
    shape = synth.TINY
    H, I = shape.hidden, shape.inter
    rng = np.random.default_rng(25)
    x = (rng.standard_normal(H) * 0.3).astype(np.float32)
    x[::32] = np.where(rng.integers(0, 2, H // 32) == 1, 1.75, -1.75)
    qb, db = oracle.q8_0(x)
    qr, dr = oracle.quant_act(x, ROW)
    assert np.array_equal(qb, qr) and np.all(db == dr[0])
    blob = synth.expert_blob(shape, 32, 0, 1)
    a = oracle.gate_up(blob, H, I, 4, qb, db)
    b = oracle.gate_up(blob, H, I, 4, qr, dr, act_block=ROW)
    assert np.allclose(a["g"], b["g"], rtol=1e-13, atol=1e-13)
    assert np.allclose(a["u"], b["u"], rtol=1e-13, atol=1e-13)


def test_layer_row_format_identical_experts_closed_form():
    """All routed experts identical -> y = shared(x) + 2.5 * expert(x), in the
    per-row format too."""
    shape = synth.TINY
    blob = synth.expert_blob(shape, 100, 0, 0)
    shared = synth.expert_blob(shape, 100, 0, synth.SHARED_ID)
    x = synth.tokens(shape, 100, 4)
    out = oracle.layer(x, synth.router_weights(shape, 100), synth.router_bias_uniform(shape, 100),
                       lambda e: blob, shared, H=256, I=128, n_experts=8, n_group=2,
                       topk_group=1, top_k=2, scale=2.5, act_block=ROW)
    assert out["d"].shape == (4, 1)
    for t in range(4):
        e_y = oracle.expert(blob, 256, 128, 4, out["q"][t], out["d"][t], ROW)["y"]
        ref = out["shared_out"][t].astype(np.float64) + 2.5 * e_y.astype(np.float64)
        assert np.max(np.abs(out["y"][t] - ref)) <= 1e-6 * np.sqrt(np.mean(ref ** 2)) + 1e-7


def test_row_format_rejects_mxfp4():
    """MXFP4 keeps per-32 weight scales: only Q8_0 activations pair with it."""
    shape = synth.TINY.with_bits(synth.MXFP4)
    blob = synth.expert_blob(shape, 3, 0, 0)
    q, d = oracle.quant_act(synth.tokens(shape, 3, 1)[0], ROW)
    with pytest.raises(ValueError):
        oracle.gate_up(blob, 256, 128, oracle.MXFP4, q, d, act_block=ROW)


# ---------------------------------------------------------------- R18: FP8 experts

def _torch_e4m3fn(codes):
    import torch
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def test_fp8_values_match_an_independent_decoder():
    """Every E4M3 code against PyTorch's float8_e4m3fn (OCP E4M3), an
    implementation that shares nothing with the oracle: same values, same
    signs of zero, NaN exactly at 0x7F and 0xFF."""
    ref = _torch_e4m3fn(np.arange(256))
    got = np.array([oracle.fp8_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_fp8_hand_values():
    """Values worked out by hand from the format (bias 7, 3 mantissa bits):
    smallest subnormal 2^-9, smallest normal 2^-6, largest 448; the
    positive codes increase strictly."""
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
            0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
            0xB8: -1.0, 0xFE: -448.0}
    for c, v in hand.items():
        assert oracle.fp8_value(c) == v, hex(c)
    pos = [oracle.fp8_value(c) for c in range(0x7F)]
    assert all(b > a for a, b in zip(pos, pos[1:]))


def test_fp8_block_dot_hand_cases():
    """P9 = sum 512 fp8(c) q: ones against 1..32; the largest magnitude
    against 127 everywhere (932,184,064, inside int32); the smallest
    subnormal is 1 unit; a NaN code is refused."""
    q = np.arange(1, 33, dtype=np.int8)
    assert oracle.act_dots(np.full(32, 0x38, np.uint8), oracle.FP8, q).tolist() == [512 * 528]
    big = oracle.act_dots(np.full(32, 0x7E, np.uint8), oracle.FP8, np.full(32, 127, np.int8))
    assert big.tolist() == [448 * 512 * 127 * 32]
    neg = oracle.act_dots(np.full(32, 0xFE, np.uint8), oracle.FP8, np.full(32, 127, np.int8))
    assert neg.tolist() == [-448 * 512 * 127 * 32]
    assert oracle.act_dots(np.full(32, 0x01, np.uint8), oracle.FP8, q).tolist() == [528]
    bad = np.full(32, 0x38, np.uint8)
    bad[5] = 0x7F
    with pytest.raises(ValueError):
        oracle.act_dots(bad, oracle.FP8, q)


def _fp8_record(rng, H, I):
    """Random valid codes (no NaN) and a distinct fp32 scale per 128x128 block."""
    codes = rng.integers(0, 256, size=3 * I * H).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38
    nb = (I // 128) * (H // 128)
    sc = (rng.uniform(0.5, 2.0, 3 * nb) * 1e-3).astype(np.float32)
    return np.concatenate([codes, sc.view(np.uint8)])


def _dequant(codes, scales, rows, cols):
    vals = _torch_e4m3fn(codes).reshape(rows, cols)
    return vals * np.kron(scales.astype(np.float64), np.ones((128, 128)))


def test_fp8_rows_equal_dequantised_matmul():
    """gate/up/down of an FP8 record against the textbook fp64 product of the
    dequantised matrices (PyTorch's decoding, each 128x128 block times its
    own scale) with the dequantised Q8_0 activations: a transposed or
    misplaced block scale, or a wrong 1/512, fails here."""
    rng = np.random.default_rng(18)
    H, I = 256, 384
    blob = _fp8_record(rng, H, I)
    gate, up, down, sg, su, sd = oracle.blob_view(blob, H, I, oracle.FP8)
    assert sg.shape == (I // 128, H // 128) and sd.shape == (H // 128, I // 128)
    x = rng.standard_normal(H).astype(np.float32)
    q, d = oracle.q8_0(x[None])
    xd = q[0].astype(np.float64) * np.repeat(d[0].astype(np.float64), 32)
    ref = oracle.gate_up(blob, H, I, oracle.FP8, q[0], d[0])
    Wg, Wu = _dequant(gate, sg, I, H), _dequant(up, su, I, H)
    assert np.allclose(ref["g"], Wg @ xd, rtol=1e-12, atol=1e-12)
    assert np.allclose(ref["u"], Wu @ xd, rtol=1e-12, atol=1e-12)
    h = rng.standard_normal(I).astype(np.float32)
    qh, dh = oracle.q8_0(h[None])
    y, dots = oracle.down(blob, H, I, oracle.FP8, qh[0], dh[0], want_dots=True)
    hd = qh[0].astype(np.float64) * np.repeat(dh[0].astype(np.float64), 32)
    Wd = _dequant(down, sd, H, I)
    assert np.allclose(y, (Wd @ hd).astype(np.float32), rtol=1e-6, atol=1e-9)
    # and the reported dots are the exact integer sums
    w512 = (_torch_e4m3fn(down) * 512).astype(np.int64).reshape(H, I // 32, 32)
    assert np.array_equal(dots, (w512 * qh[0].astype(np.int64).reshape(I // 32, 32)).sum(-1))


def test_fp8_generated_record_is_the_e4m3_rounding_of_the_weights():
    """The generator's FP8 record (tiny shape): each 128x128 block's scale is
    amax/448 of its float weights, and every code is PyTorch's
    round-to-nearest-even E4M3 conversion of weight / scale (zero as code
    0)."""
    import torch
    shape = synth.TINY.with_bits(synth.FP8)
    H, I = shape.hidden, shape.inter
    blob = synth.expert_blob(shape, 5, 0, 3)
    assert blob.size == oracle.blob_bytes(H, I, oracle.FP8)
    mats = oracle.blob_view(blob, H, I, oracle.FP8)
    for m, (rows, cols) in enumerate(((I, H), (I, H), (H, I))):
        W = np.stack([synth.weight_row(5, 0, 3, m, cols, r) for r in range(rows)])
        codes, sc = mats[m], mats[3 + m]
        for br in range(rows // 128):
            for bc in range(cols // 128):
                blk = W[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128]
                s = np.float32(np.abs(blk).max()) / np.float32(448.0)
                assert sc[br, bc] == s
                want = torch.from_numpy(blk / s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                want = np.where(want == 0x80, 0, want)
                got = codes[br * 128:(br + 1) * 128, bc * 128:(bc + 1) * 128]
                assert np.array_equal(got, want), (m, br, bc)
