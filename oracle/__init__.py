"""CPU oracle for the routed-MoE layer step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never does, and shares
no code with it.  The arithmetic lives in ``oracle.c`` (plain C11, built with
``-O2 -ffp-contract=off -fno-fast-math``); this module only marshals numpy
arrays to it and composes the per-step functions into a whole layer.

Every step cites the pages in ``oracle.c``.  The functions here follow the same
order as the method: router scores -> group-limited top-k -> Q8_0 of the
hidden state -> batch-union grouping -> per-expert gate/up + SwiGLU -> Q8_0 of
h -> down -> weighted combine with the shared expert.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
QBLK = 32

_lib = None


MXFP4 = -4  # weight-format code of MXFP4 experts (reading R16)
FP8 = -8  # weight-format code of FP8 E4M3 experts with 128x128 block scales (reading R18)
F8BLK = 128
ACT_Q8_0, ACT_ROW = 32, -1  # activation formats: Q8_0 blocks of 32 (R6), one scale per row (R17)

def build() -> str:
    """Compile oracle.c into liboracle.so (gcc, plain C11, no fp contraction)."""
    src = os.path.join(_HERE, "oracle.c")
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wno-unknown-pragmas", src, "-o", LIB_PATH + ".tmp",
           "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _p(t):
    return ctypes.POINTER(t)


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    c_i, c_f, c_v = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    L.oracle_code.argtypes = [c_v, c_i, c_i]
    L.oracle_code.restype = c_i
    L.oracle_unpack.argtypes = [c_v, c_i, c_i, c_v]
    L.oracle_unpack.restype = None
    L.oracle_pack.argtypes = [c_v, c_i, c_i, c_v]
    L.oracle_pack.restype = c_i
    L.oracle_q8_0.argtypes = [c_v, ctypes.c_int64, c_i, c_v, c_v]
    L.oracle_q8_0.restype = c_i
    L.oracle_quant_act.argtypes = [c_v, ctypes.c_int64, c_i, c_i, c_v, c_v]
    L.oracle_quant_act.restype = c_i
    L.oracle_act_dots.argtypes = [c_v, c_i, c_v, c_i, c_i, c_v]
    L.oracle_act_dots.restype = c_i
    L.oracle_gate_up_act.argtypes = [c_v, c_i, c_i, c_i, c_i, c_v, c_v, c_v, c_v, c_v, c_v, c_v]
    L.oracle_gate_up_act.restype = c_i
    L.oracle_down_act.argtypes = [c_v, c_i, c_i, c_i, c_i, c_v, c_v, c_v, c_v]
    L.oracle_down_act.restype = c_i
    L.oracle_expert_act.argtypes = [c_v, c_i, c_i, c_i, c_i, c_v, c_v, c_v, c_v, c_v, c_v]
    L.oracle_expert_act.restype = c_i
    L.oracle_dot_canon.argtypes = [c_v, c_v, c_i]
    L.oracle_dot_canon.restype = c_f
    L.oracle_exp_canon.argtypes = [c_f]
    L.oracle_exp_canon.restype = c_f
    L.oracle_sigmoid_canon.argtypes = [c_f]
    L.oracle_sigmoid_canon.restype = c_f
    L.oracle_router_scores.argtypes = [c_i, c_i, c_i, c_v, c_v, c_v, c_v, c_v]
    L.oracle_router_scores.restype = None
    L.oracle_select.argtypes = [c_i, c_i, c_i, c_i, c_i, c_f, c_v, c_v, c_v, c_v, c_v]
    L.oracle_select.restype = c_i
    L.oracle_route.argtypes = [c_i, c_i, c_i, c_i, c_i, c_i, c_f, c_v, c_v, c_v, c_v, c_v, c_v]
    L.oracle_route.restype = c_i
    L.oracle_fp4_value.argtypes = [c_i]
    L.oracle_fp4_value.restype = ctypes.c_double
    L.oracle_e8m0_value.argtypes = [c_i]
    L.oracle_e8m0_value.restype = ctypes.c_double
    L.oracle_fp8_value.argtypes = [c_i]
    L.oracle_fp8_value.restype = ctypes.c_double
    L.oracle_top_p.argtypes = [c_i, c_i, c_i, c_f, c_f, c_v, c_v, c_v, c_v]
    L.oracle_top_p.restype = c_i
    L.oracle_group.argtypes = [c_i, c_i, c_i, c_v, c_v, c_v, c_v, c_v, c_v, c_v]
    L.oracle_group.restype = c_i
    L.oracle_block_dots.argtypes = [c_v, c_i, c_v, c_i, c_v]
    L.oracle_block_dots.restype = c_i
    L.oracle_blob_bytes.argtypes = [c_i, c_i, c_i]
    L.oracle_blob_bytes.restype = ctypes.c_size_t
    L.oracle_gate_up.argtypes = [c_v, c_i, c_i, c_i, c_v, c_v, c_v, c_v, c_v, c_v, c_v]
    L.oracle_gate_up.restype = c_i
    L.oracle_down.argtypes = [c_v, c_i, c_i, c_i, c_v, c_v, c_v, c_v]
    L.oracle_down.restype = c_i
    L.oracle_expert.argtypes = [c_v, c_i, c_i, c_i, c_v, c_v, c_v, c_v, c_v, c_v]
    L.oracle_expert.restype = c_i
    L.oracle_combine.argtypes = [c_i, c_i, c_i, c_v, c_v, c_v, c_v, c_v, c_v, c_f]
    L.oracle_combine.restype = None
    L.oracle_rmsnorm.argtypes = [c_i, c_i, c_v, c_v, c_f]
    L.oracle_rmsnorm.restype = None
    L.oracle_threads.argtypes = []
    L.oracle_threads.restype = c_i
    L.oracle_set_threads.argtypes = [c_i]
    L.oracle_set_threads.restype = None
    _lib = L
    return L


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def threads() -> int:
    """OpenMP threads used by the oracle's parallel loops."""
    return int(lib().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's parallel loops from now on (results do not
    depend on it: each output row is computed by one thread)."""
    lib().oracle_set_threads(int(n))


# ------------------------------------------------------------------ codes

def code(row: np.ndarray, wbits: int, k: int) -> int:
    row = _c(row, np.uint8)
    return lib().oracle_code(_ptr(row), wbits, k)


def _bits(wbits: int) -> int:
    return 4 if wbits == MXFP4 else 8 if wbits == FP8 else wbits


def unpack(row: np.ndarray, wbits: int, n: int) -> np.ndarray:
    row = _c(row, np.uint8)
    assert row.size * (8 // _bits(wbits)) >= n
    out = np.empty(n, np.int8)
    lib().oracle_unpack(_ptr(row), wbits, n, _ptr(out))
    return out


def pack(codes: np.ndarray, wbits: int) -> np.ndarray:
    codes = _c(codes, np.int8)
    out = np.empty(codes.size * _bits(wbits) // 8, np.uint8)
    _check(lib().oracle_pack(_ptr(codes), codes.size, wbits, _ptr(out)), "pack")
    return out


# ------------------------------------------------------------------ Q8_0

def q8_0(x: np.ndarray):
    """Q8_0 of each row (row length a multiple of 32): (int8 codes, fp32 scales)."""
    x = _c(x, np.float32)
    rows, n = (1, x.size) if x.ndim == 1 else (int(np.prod(x.shape[:-1])), x.shape[-1])
    q = np.empty(x.shape, np.int8)
    d = np.empty(x.shape[:-1] + (n // QBLK,), np.float32)
    _check(lib().oracle_q8_0(_ptr(x), rows, n, _ptr(q), _ptr(d)), "q8_0")
    return q, d


def act_len(act_block: int, n: int) -> int:
    """Activation block length of a format on rows of n values."""
    return n if act_block == ACT_ROW else act_block


def quant_act(x: np.ndarray, act_block: int = ACT_Q8_0):
    """Activations of each row in format act_block (R6 Q8_0 or R17 one scale
    per row): (int8 codes, fp32 scales [..., n / block])."""
    x = _c(x, np.float32)
    rows, n = (1, x.size) if x.ndim == 1 else (int(np.prod(x.shape[:-1])), x.shape[-1])
    q = np.empty(x.shape, np.int8)
    d = np.empty(x.shape[:-1] + (n // act_len(act_block, n),), np.float32)
    _check(lib().oracle_quant_act(_ptr(x), rows, n, act_block, _ptr(q), _ptr(d)), "quant_act")
    return q, d


# ------------------------------------------------------------------ router

def dot_canon(a, b) -> np.float32:
    a, b = _c(a, np.float32), _c(b, np.float32)
    return np.float32(lib().oracle_dot_canon(_ptr(a), _ptr(b), a.size))


def exp_canon(y) -> np.ndarray:
    y = np.atleast_1d(np.asarray(y, np.float32))
    L = lib()
    return np.array([L.oracle_exp_canon(float(v)) for v in y], np.float32)


def sigmoid_canon(v) -> np.ndarray:
    v = np.atleast_1d(np.asarray(v, np.float32))
    L = lib()
    return np.array([L.oracle_sigmoid_canon(float(a)) for a in v], np.float32)


def router_scores(x, wr, bias):
    x, wr, bias = _c(x, np.float32), _c(wr, np.float32), _c(bias, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    s = np.empty((T, E), np.float32)
    sb = np.empty((T, E), np.float32)
    lib().oracle_router_scores(T, H, E, _ptr(x), _ptr(wr), _ptr(bias), _ptr(s), _ptr(sb))
    return s, sb


def select(s, sb, n_group, topk_group, top_k, scale):
    """Group-limited top-k on given scores: (idx [T,K] int32, w [T,K] fp32, margins [T,2])."""
    s, sb = _c(s, np.float32), _c(sb, np.float32)
    T, E = s.shape
    idx = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    margin = np.empty((T, 2), np.float64)
    _check(lib().oracle_select(T, E, n_group, topk_group, top_k, scale, _ptr(s), _ptr(sb),
                               _ptr(idx), _ptr(w), _ptr(margin)), "select")
    return idx, w, margin


def top_p(s, idx, w, p, scale):
    """Adaptive expert top-p (R15) on a rank-ordered selection: new (idx, w,
    kept [T]); dropped ranks get idx -1 and w 0.  p = 0 or 1 changes nothing."""
    s = _c(s, np.float32)
    idx, w = np.array(idx, np.int32, order="C"), np.array(w, np.float32, order="C")
    T, E = s.shape
    K = idx.shape[1]
    kept = np.empty(T, np.int32)
    _check(lib().oracle_top_p(T, K, E, p, scale, _ptr(s), _ptr(idx), _ptr(w), _ptr(kept)),
           "top_p")
    return idx, w, kept


def route(x, wr, bias, n_group, topk_group, top_k, scale, top_p_value=0.0):
    """Router for T tokens: (idx [T,K] int32, w [T,K] fp32, margins [T,2] fp64);
    with 0 < top_p_value < 1 the adaptive top-p cut (R15) follows."""
    x, wr, bias = _c(x, np.float32), _c(wr, np.float32), _c(bias, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    idx = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    margin = np.empty((T, 2), np.float64)
    if 0.0 < top_p_value < 1.0:
        s, sb = router_scores(x, wr, bias)
        idx, w, margin = select(s, sb, n_group, topk_group, top_k, scale)
        idx, w, _ = top_p(s, idx, w, top_p_value, scale)
        return idx, w, margin
    _check(lib().oracle_route(T, H, E, n_group, topk_group, top_k, scale, _ptr(x), _ptr(wr),
                              _ptr(bias), _ptr(idx), _ptr(w), _ptr(margin)), "route")
    return idx, w, margin


# ------------------------------------------------------------------ grouping

def group(idx: np.ndarray, n_experts: int):
    """Batch-union grouping: dict of counts, offsets, perm, inv, active, n_active."""
    idx = _c(idx, np.int32)
    T, K = idx.shape
    E = n_experts
    out = dict(counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
               perm=np.empty(T * K, np.int32), inv=np.empty(T * K, np.int32),
               active=np.empty(E, np.int32))
    na = np.zeros(1, np.int32)
    _check(lib().oracle_group(T, K, E, _ptr(idx), _ptr(out["counts"]), _ptr(out["offsets"]),
                              _ptr(out["perm"]), _ptr(out["inv"]), _ptr(out["active"]),
                              _ptr(na)), "group")
    out["n_active"] = int(na[0])
    return out


# ------------------------------------------------------------------ experts

def fp4_value(code: int) -> float:
    return float(lib().oracle_fp4_value(code))


def e8m0_value(s: int) -> float:
    return float(lib().oracle_e8m0_value(s))


def fp8_value(code: int) -> float:
    """R18: value of an FP8 E4M3 code byte (NaN for 0x7F, 0xFF)."""
    return float(lib().oracle_fp8_value(code))


def blob_bytes(H, I, wbits=4) -> int:
    return int(lib().oracle_blob_bytes(H, I, wbits))


def blob_view(blob: np.ndarray, H: int, I: int, wbits: int = 4):
    """Split a packed expert record into (gate, up, down code rows, scales);
    MXFP4: the scales are the per-block E8M0 bytes [rows][n/32]; FP8: the
    fp32 128x128 block scales [rows/128][n/128]."""
    if wbits == FP8:
        gate = blob[: I * H].reshape(I, H)
        up = blob[I * H: 2 * I * H].reshape(I, H)
        down = blob[2 * I * H: 3 * I * H].reshape(H, I)
        sc = blob[3 * I * H:].view(np.float32)
        nb = (I // F8BLK) * (H // F8BLK)
        return (gate, up, down, sc[:nb].reshape(I // F8BLK, H // F8BLK),
                sc[nb:2 * nb].reshape(I // F8BLK, H // F8BLK),
                sc[2 * nb:3 * nb].reshape(H // F8BLK, I // F8BLK))
    if wbits == MXFP4:
        gr, dr = H // 2, I // 2
        gate = blob[: I * gr].reshape(I, gr)
        up = blob[I * gr: 2 * I * gr].reshape(I, gr)
        down = blob[2 * I * gr: 2 * I * gr + H * dr].reshape(H, dr)
        t = blob[2 * I * gr + H * dr:]
        nb, mb = H // QBLK, I // QBLK
        return (gate, up, down, t[:I * nb].reshape(I, nb), t[I * nb:2 * I * nb].reshape(I, nb),
                t[2 * I * nb:2 * I * nb + H * mb].reshape(H, mb))
    gr, dr = H * wbits // 8, I * wbits // 8
    gate = blob[: I * gr].reshape(I, gr)
    up = blob[I * gr: 2 * I * gr].reshape(I, gr)
    down = blob[2 * I * gr: 2 * I * gr + H * dr].reshape(H, dr)
    sc = blob[2 * I * gr + H * dr:].view(np.float32)
    return gate, up, down, sc[:I], sc[I:2 * I], sc[2 * I:2 * I + H]


def block_dots(row, wbits, q):
    row, q = _c(row, np.uint8), _c(q, np.int8)
    out = np.empty(q.size // QBLK, np.int32)
    _check(lib().oracle_block_dots(_ptr(row), wbits, _ptr(q), q.size, _ptr(out)), "block_dots")
    return out


def act_dots(row, wbits, q, act_block=ACT_Q8_0):
    """Exact int32 dots of a packed weight row with int8 activations, one per
    activation block of the format."""
    row, q = _c(row, np.uint8), _c(q, np.int8)
    out = np.empty(q.size // act_len(act_block, q.size), np.int32)
    _check(lib().oracle_act_dots(_ptr(row), wbits, _ptr(q), q.size, act_block, _ptr(out)),
           "act_dots")
    return out


def gate_up(blob, H, I, wbits, q, d, want_dots=False, act_block=ACT_Q8_0):
    """One token through gate/up + SwiGLU: dict(h fp32 [I], g, u fp64 [I], dots
    [I][H / block])."""
    blob, q, d = _c(blob, np.uint8), _c(q, np.int8), _c(d, np.float32)
    nb = H // act_len(act_block, H)
    h = np.empty(I, np.float32)
    g = np.empty(I, np.float64)
    u = np.empty(I, np.float64)
    gd = np.empty((I, nb), np.int32) if want_dots else None
    ud = np.empty((I, nb), np.int32) if want_dots else None
    _check(lib().oracle_gate_up_act(_ptr(blob), H, I, wbits, act_block, _ptr(q), _ptr(d),
                                    _ptr(gd), _ptr(ud), _ptr(g), _ptr(u), _ptr(h)), "gate_up")
    return dict(h=h, g=g, u=u, gate_dots=gd, up_dots=ud)


def down(blob, H, I, wbits, qh, dh, want_dots=False, act_block=ACT_Q8_0):
    """One token through the down matrix: (y fp32 [H], dots [H][I / block] or None)."""
    blob, qh, dh = _c(blob, np.uint8), _c(qh, np.int8), _c(dh, np.float32)
    y = np.empty(H, np.float32)
    dd = np.empty((H, I // act_len(act_block, I)), np.int32) if want_dots else None
    _check(lib().oracle_down_act(_ptr(blob), H, I, wbits, act_block, _ptr(qh), _ptr(dh),
                                 _ptr(dd), _ptr(y)), "down")
    return y, dd


def expert(blob, H, I, wbits, q, d, act_block=ACT_Q8_0):
    """One token through a whole expert: dict(h, qh, dh, y)."""
    blob, q, d = _c(blob, np.uint8), _c(q, np.int8), _c(d, np.float32)
    h = np.empty(I, np.float32)
    qh = np.empty(I, np.int8)
    dh = np.empty(I // act_len(act_block, I), np.float32)
    y = np.empty(H, np.float32)
    _check(lib().oracle_expert_act(_ptr(blob), H, I, wbits, act_block, _ptr(q), _ptr(d), _ptr(h),
                                   _ptr(qh), _ptr(dh), _ptr(y)), "expert")
    return dict(h=h, qh=qh, dh=dh, y=y)


# ------------------------------------------------------------------ combine

def combine(expert_out, w, shared_out=None, residual=None, eps=1e-5, want_norm=False):
    expert_out, w = _c(expert_out, np.float32), _c(w, np.float32)
    T, K, H = expert_out.shape
    shared_out = None if shared_out is None else _c(shared_out, np.float32)
    residual = None if residual is None else _c(residual, np.float32)
    y = np.empty((T, H), np.float32)
    yn = np.empty((T, H), np.float32) if want_norm else None
    lib().oracle_combine(T, H, K, _ptr(expert_out), _ptr(w), _ptr(shared_out), _ptr(residual),
                         _ptr(y), _ptr(yn), eps)
    return (y, yn) if want_norm else y


def rmsnorm(x, eps=1e-5):
    x = _c(x, np.float32)
    T, H = x.shape
    y = np.empty_like(x)
    lib().oracle_rmsnorm(T, H, _ptr(x), _ptr(y), eps)
    return y


# ------------------------------------------------------------------ whole layer

def layer(x, router_w, bias, blob_of, shared_blob, *, H, I, n_experts, n_group, topk_group,
          top_k, scale, wbits=4, residual=None, want_norm=False, eps=1e-5, top_p_value=0.0,
          act_block=ACT_Q8_0):
    """One routed-MoE layer for T tokens, step by step (activations of x and h
    in format act_block: Q8_0, or one scale per row, R17).

    ``blob_of(e)`` returns the packed record of routed expert ``e`` (only the
    experts the router selects are requested); ``shared_blob`` may be None.
    Returns a dict with idx, w, q, d, groups, expert_out [T,K,H], shared_out
    [T,H], y [T,H] (and y_norm when requested).
    """
    x = _c(x, np.float32)
    T = x.shape[0]
    idx, w, margin = route(x, router_w, bias, n_group, topk_group, top_k, scale, top_p_value)
    q, d = quant_act(x, act_block)
    groups = group(idx, n_experts)
    expert_out = np.zeros((T, top_k, H), np.float32)
    for e in groups["active"][: groups["n_active"]]:
        blob = blob_of(int(e))
        lo, hi = groups["offsets"][e], groups["offsets"][e + 1]
        for slot in groups["perm"][lo:hi]:
            t, k = divmod(int(slot), top_k)
            expert_out[t, k] = expert(blob, H, I, wbits, q[t], d[t], act_block)["y"]
    shared_out = None
    if shared_blob is not None:
        shared_out = np.stack([expert(shared_blob, H, I, wbits, q[t], d[t], act_block)["y"]
                               for t in range(T)])
    res = combine(expert_out, w, shared_out, residual, eps, want_norm)
    y, yn = res if want_norm else (res, None)
    return dict(idx=idx, w=w, margin=margin, q=q, d=d, groups=groups, expert_out=expert_out,
                shared_out=shared_out, y=y, y_norm=yn)
