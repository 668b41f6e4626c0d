"""Python binding of libmoe (the routed-MoE layer step for MI355X / gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe.so`` behind the C ABI declared in ``include/moe.h``.  PyTorch supplies
device memory (tensors) and the HIP stream (``torch.cuda.current_stream()``,
which is a HIP stream under PyTorch-ROCm).  There is no fallback: if the
library is not built, or a tensor is not on the GPU, calls raise.

Functions mirror the C entry points: ``route``, ``quant_act``, ``group``,
``expert_ffn``, ``combine``, ``rmsnorm``, ``layer`` (+ workspace queries).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4

EXPORTS = (
    "moe_expert_blob_bytes", "moe_route_workspace", "moe_route", "moe_quant_act", "moe_group",
    "moe_expert_ffn_workspace", "moe_expert_ffn", "moe_combine", "moe_rmsnorm",
    "moe_layer_workspace", "moe_layer", "moe_layer_ptrs", "moe_layer_noalloc",
    "moe_host_device_ptr", "moe_cache_create", "moe_cache_step", "moe_cache_get_stats",
    "moe_cache_prefetch", "moe_cache_publish", "moe_cache_usage", "moe_cache_slot_of", "moe_cache_destroy",
    "moe_cache_simulate",
    "moe_mfma_peak", "moe_read_peak", "moe_strerror", "moe_last_error",
)


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


class MoeCfg(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_group", ctypes.c_int32),
                ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("wbits", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("top_p", ctypes.c_float),
                ("wfmt", ctypes.c_int32), ("act_block", ctypes.c_int32)]


ACT_Q8_0, ACT_ROW = 32, -1  # moe_cfg.act_block: Q8_0 blocks, one scale per row (MOE_ACT_ROW)


MOE_N_STAGES = 8
STAGES = dict(router_scores=0, router_select=1, quant=2, group=3, gate_up=4, down=5, combine=6,
              norm=7)


class MoeEvents(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p * MOE_N_STAGES), ("stop", ctypes.c_void_p * MOE_N_STAGES)]


class MoeFfnDebug(ctypes.Structure):
    _fields_ = [("gate_dots", ctypes.c_void_p), ("up_dots", ctypes.c_void_p),
                ("h", ctypes.c_void_p), ("q_h", ctypes.c_void_p), ("d_h", ctypes.c_void_p),
                ("down_dots", ctypes.c_void_p)]


class MoeLayerDebug(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("counts", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("inv", ctypes.c_void_p),
                ("active", ctypes.c_void_p), ("n_active", ctypes.c_void_p),
                ("ffn", MoeFfnDebug)]


class MoeCacheStats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_uint64), ("routed", ctypes.c_uint64),
                ("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64),
                ("promotions", ctypes.c_uint64), ("completed", ctypes.c_uint64),
                ("bytes_copied", ctypes.c_uint64), ("resident", ctypes.c_int32),
                ("prefetched", ctypes.c_uint64)]


_lib = None


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(there is no fallback implementation)")
    try:  # load PyTorch's HIP runtime first so that libmoe binds to the same one
        import torch  # noqa: F401
    except ImportError:
        pass
    L = ctypes.CDLL(LIB_PATH)
    v, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    pc = ctypes.POINTER(MoeCfg)
    L.moe_expert_blob_bytes.argtypes = [pc]
    L.moe_expert_blob_bytes.restype = sz
    L.moe_route_workspace.argtypes = [pc, i32]
    L.moe_route_workspace.restype = sz
    L.moe_route.argtypes = [pc, i32, v, v, v, v, v, v, sz, v]
    L.moe_route.restype = ctypes.c_int
    L.moe_quant_act.argtypes = [i32, i32, i32, v, v, v, v]
    L.moe_quant_act.restype = ctypes.c_int
    L.moe_group.argtypes = [pc, i32, v, v, v, v, v, v, v, v]
    L.moe_group.restype = ctypes.c_int
    L.moe_expert_ffn_workspace.argtypes = [pc, i32]
    L.moe_expert_ffn_workspace.restype = sz
    L.moe_expert_ffn.argtypes = [pc, i32, v, v, v, v, v, v, v, v, sz,
                                 ctypes.POINTER(MoeFfnDebug), v]
    L.moe_expert_ffn.restype = ctypes.c_int
    L.moe_combine.argtypes = [i32, i32, i32, v, v, v, v, v, v, f32, v]
    L.moe_combine.restype = ctypes.c_int
    L.moe_rmsnorm.argtypes = [i32, i32, v, v, f32, v]
    L.moe_rmsnorm.restype = ctypes.c_int
    L.moe_mfma_peak.argtypes = [i32, i32, v, v]
    L.moe_mfma_peak.restype = ctypes.c_int
    L.moe_read_peak.argtypes = [v, ctypes.c_int64, i32, v, v, v, v]
    L.moe_read_peak.restype = ctypes.c_int
    L.moe_layer_workspace.argtypes = [pc, i32]
    L.moe_layer_workspace.restype = sz
    L.moe_layer.argtypes = [pc, i32, v, v, v, v, v, v, v, v, f32, v, v, v, sz,
                            ctypes.POINTER(MoeEvents), ctypes.POINTER(MoeLayerDebug), v]
    L.moe_layer.restype = ctypes.c_int
    L.moe_layer_ptrs.argtypes = L.moe_layer.argtypes
    L.moe_layer_ptrs.restype = ctypes.c_int
    L.moe_layer_noalloc.argtypes = [pc, i32, v, v, v, v, v, v, v, v, f32, v, v,
                                    ctypes.POINTER(MoeEvents), v]
    L.moe_layer_noalloc.restype = ctypes.c_int
    u64p, i32p = ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_int32)
    L.moe_host_device_ptr.argtypes = [v, ctypes.POINTER(v)]
    L.moe_host_device_ptr.restype = ctypes.c_int
    L.moe_cache_create.argtypes = [pc, i32, i32, i32, i32, ctypes.POINTER(v), v, v, u64p, v,
                                   ctypes.POINTER(v)]
    L.moe_cache_create.restype = ctypes.c_int
    L.moe_cache_step.argtypes = [v, v, i32, i32, v]
    L.moe_cache_step.restype = ctypes.c_int
    L.moe_cache_prefetch.argtypes = [v, v, i32, v]
    L.moe_cache_prefetch.restype = ctypes.c_int
    L.moe_cache_publish.argtypes = [v, v]
    L.moe_cache_publish.restype = ctypes.c_int
    L.moe_cache_get_stats.argtypes = [v, ctypes.POINTER(MoeCacheStats)]
    L.moe_cache_get_stats.restype = ctypes.c_int
    L.moe_cache_usage.argtypes = [v, u64p]
    L.moe_cache_usage.restype = ctypes.c_int
    L.moe_cache_slot_of.argtypes = [v, i32p]
    L.moe_cache_slot_of.restype = ctypes.c_int
    L.moe_cache_destroy.argtypes = [v]
    L.moe_cache_destroy.restype = ctypes.c_int
    L.moe_cache_simulate.argtypes = [i32, i32, i32, i32, u64p, i32p, i32p, i32, i32, i32p, i32p,
                                     i32p]
    L.moe_cache_simulate.restype = ctypes.c_int
    L.moe_strerror.argtypes = [ctypes.c_int]
    L.moe_strerror.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int):
    if rc != MOE_OK:
        L = lib()
        raise MoeError(rc, f"{L.moe_strerror(rc).decode()}: {L.moe_last_error().decode()}")


@dataclass(frozen=True)
class Config:
    hidden: int
    inter: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    n_shared: int = 1
    wbits: int = 4
    routed_scaling: float = 2.5
    top_p: float = 0.0  # adaptive expert top-p; 0 = off
    wfmt: int = 0  # 0: integer codes with fp32 row scales; 1: MXFP4 (wbits 4); 2: FP8 (wbits 8)
    act_block: int = ACT_Q8_0  # activations: Q8_0 blocks of 32, or ACT_ROW (one scale per row)

    @classmethod
    def of(cls, shape, top_p: float = 0.0, act_block: int = ACT_Q8_0) -> "Config":
        # the synthetic shapes' codes: -4 MXFP4 experts, -8 FP8 experts
        wbits, wfmt = {-4: (4, 1), -8: (8, 2)}.get(shape.wbits, (shape.wbits, 0))
        return cls(shape.hidden, shape.inter, shape.n_experts, shape.n_group, shape.topk_group,
                   shape.top_k, shape.n_shared, wbits, shape.routed_scaling, top_p, wfmt,
                   act_block)

    def act_len(self, n: int) -> int:
        """Activation block length on rows of n values."""
        return n if self.act_block == ACT_ROW else 32

    def c(self) -> MoeCfg:
        return MoeCfg(self.hidden, self.inter, self.n_experts, self.n_group, self.topk_group,
                      self.top_k, self.n_shared, self.wbits, self.routed_scaling, self.top_p,
                      self.wfmt, self.act_block)


def _torch():
    import torch
    return torch


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors only")
    return t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def blob_bytes(cfg: Config) -> int:
    return int(lib().moe_expert_blob_bytes(ctypes.byref(cfg.c())))


def route_workspace(cfg: Config, T: int) -> int:
    return int(lib().moe_route_workspace(ctypes.byref(cfg.c()), T))


def expert_ffn_workspace(cfg: Config, T: int) -> int:
    return int(lib().moe_expert_ffn_workspace(ctypes.byref(cfg.c()), T))


def layer_workspace(cfg: Config, T: int) -> int:
    return int(lib().moe_layer_workspace(ctypes.byref(cfg.c()), T))


def _workspace(nbytes, device, ws=None):
    """Caller's workspace, or a new one (its contents do not matter)."""
    torch = _torch()
    if ws is not None:
        return ws
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def route(cfg: Config, x, w_router, bias, idx=None, w=None, workspace=None):
    """moe_route: returns (idx int32 [T,K], w fp32 [T,K])."""
    torch = _torch()
    T = x.shape[0]
    idx = idx if idx is not None else torch.empty((T, cfg.top_k), dtype=torch.int32,
                                                  device=x.device)
    w = w if w is not None else torch.empty((T, cfg.top_k), dtype=torch.float32, device=x.device)
    ws = _workspace(route_workspace(cfg, T), x.device, workspace)
    _check(lib().moe_route(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                           _ptr(idx), _ptr(w), _ptr(ws), ws.numel(), _stream()))
    return idx, w


def quant_act(x, q=None, d=None, block=32):
    """moe_quant_act on the rows of x, blocks of `block` values (32 = Q8_0, or
    the row length = one scale per row): returns (q int8, d fp32 [..., n/block])."""
    torch = _torch()
    n = x.shape[-1]
    rows = x.numel() // n if n else 0
    q = q if q is not None else torch.empty(x.shape, dtype=torch.int8, device=x.device)
    d = d if d is not None else torch.empty(x.shape[:-1] + (n // block,), dtype=torch.float32,
                                            device=x.device)
    _check(lib().moe_quant_act(rows, n, block, _ptr(x), _ptr(q), _ptr(d), _stream()))
    return q, d


def group(cfg: Config, idx):
    """moe_group: dict of counts, offsets, perm, inv, active, n_active (device tensors)."""
    torch = _torch()
    T = idx.shape[0]
    E, S = cfg.n_experts, T * cfg.top_k
    dev = idx.device
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               perm=torch.empty(max(S, 1), dtype=torch.int32, device=dev),
               inv=torch.empty(max(S, 1), dtype=torch.int32, device=dev),
               active=torch.empty(E, dtype=torch.int32, device=dev),
               n_active=torch.empty(1, dtype=torch.int32, device=dev))
    _check(lib().moe_group(ctypes.byref(cfg.c()), T, _ptr(idx), _ptr(out["counts"]),
                           _ptr(out["offsets"]), _ptr(out["perm"]), _ptr(out["inv"]),
                           _ptr(out["active"]), _ptr(out["n_active"]), _stream()))
    return out


def debug_buffers(cfg: Config, T: int, device):
    """Device buffers for every intermediate moe_expert_ffn can report
    (moe_layer's dumps add q, d and the union: ``layer_debug_buffers``)."""
    torch = _torch()
    P = T * cfg.top_k + T * cfg.n_shared
    H, I = cfg.hidden, cfg.inter
    nh, ni = H // cfg.act_len(H), I // cfg.act_len(I)
    return dict(gate_dots=torch.zeros((P, I, nh), dtype=torch.int32, device=device),
                up_dots=torch.zeros((P, I, nh), dtype=torch.int32, device=device),
                h=torch.zeros((P, I), dtype=torch.float32, device=device),
                q_h=torch.zeros((P, I), dtype=torch.int8, device=device),
                d_h=torch.zeros((P, ni), dtype=torch.float32, device=device),
                down_dots=torch.zeros((P, H, ni), dtype=torch.int32, device=device))


def layer_debug_buffers(cfg: Config, T: int, device):
    """Device buffers for every intermediate moe_layer can report."""
    torch = _torch()
    H, E, S = cfg.hidden, cfg.n_experts, T * cfg.top_k
    out = debug_buffers(cfg, T, device)
    i32 = dict(dtype=torch.int32, device=device)
    out.update(q=torch.zeros((T, H), dtype=torch.int8, device=device),
               d=torch.zeros((T, H // cfg.act_len(H)), dtype=torch.float32, device=device),
               counts=torch.zeros(E, **i32), offsets=torch.zeros(E + 1, **i32),
               perm=torch.zeros(S, **i32), inv=torch.zeros(S, **i32),
               active=torch.zeros(E, **i32), n_active=torch.zeros(1, **i32))
    return out


_FFN_DUMPS = ("gate_dots", "up_dots", "h", "q_h", "d_h", "down_dots")
_UNION_DUMPS = ("counts", "offsets", "perm", "inv", "active", "n_active")


def _layer_debug(debug):
    if debug is None:
        return None
    p = lambda k: _ptr(debug[k]) if debug.get(k) is not None else None  # noqa: E731
    return MoeLayerDebug(p("q"), p("d"), *[p(k) for k in _UNION_DUMPS],
                         MoeFfnDebug(*[p(k) for k in _FFN_DUMPS]))


def expert_ffn(cfg: Config, q, d, idx, experts, shared=None, expert_out=None, shared_out=None,
               workspace=None, debug=None):
    """moe_expert_ffn: returns (expert_out [T,K,H], shared_out [T,H] or None)."""
    torch = _torch()
    T = q.shape[0]
    dev = q.device
    H = cfg.hidden
    expert_out = expert_out if expert_out is not None else torch.empty(
        (T, cfg.top_k, H), dtype=torch.float32, device=dev)
    if cfg.n_shared and shared_out is None:
        shared_out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws = _workspace(expert_ffn_workspace(cfg, T), dev, workspace)
    dbg = None
    if debug is not None:
        dbg = MoeFfnDebug(*[(_ptr(debug[k]) if debug.get(k) is not None else None)
                            for k in _FFN_DUMPS])
    _check(lib().moe_expert_ffn(ctypes.byref(cfg.c()), T, _ptr(q), _ptr(d), _ptr(idx),
                                _ptr(experts), _ptr(shared), _ptr(expert_out), _ptr(shared_out),
                                _ptr(ws), ws.numel(), ctypes.byref(dbg) if dbg else None,
                                _stream()))
    return expert_out, shared_out


def combine(expert_out, w, shared_out=None, residual=None, y=None, y_norm=None, eps=1e-5,
            want_norm=False):
    """moe_combine: returns y (and y_norm when want_norm)."""
    torch = _torch()
    T, K, H = expert_out.shape
    y = y if y is not None else torch.empty((T, H), dtype=torch.float32, device=expert_out.device)
    if want_norm and y_norm is None:
        y_norm = torch.empty_like(y)
    _check(lib().moe_combine(T, H, K, _ptr(expert_out), _ptr(w), _ptr(shared_out),
                             _ptr(residual), _ptr(y), _ptr(y_norm), eps, _stream()))
    return (y, y_norm) if want_norm else y


def rmsnorm(x, y=None, eps=1e-5):
    torch = _torch()
    T, H = x.shape
    y = y if y is not None else torch.empty_like(x)
    _check(lib().moe_rmsnorm(T, H, _ptr(x), _ptr(y), eps, _stream()))
    return y


def mfma_peak(n_wg, iters, out):
    """moe_mfma_peak: matrix cores alone; out int32 [n_wg * 256] on the device.
    Returns the int8 operations launched (n_wg * 4 * iters * 8 * 32768)."""
    _check(lib().moe_mfma_peak(n_wg, iters, _ptr(out), _stream()))
    return n_wg * 4 * iters * 8 * 32768


def read_peak(buf, nbytes, n_wg, out, ev_start=None, ev_stop=None):
    """moe_read_peak: a plain streaming read of the first nbytes of the device
    tensor buf; out uint32 (int32 tensor) [n_wg * 4] on the device receives
    one XOR checksum per wave; ev_start / ev_stop: optional hipEvent_t
    handles stamped by the kernel's dispatch."""
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if out.numel() < 4 * n_wg:
        raise ValueError("out needs n_wg * 4 words")
    _check(lib().moe_read_peak(_ptr(buf), nbytes, n_wg, _ptr(out), ev_start, ev_stop,
                               _stream()))


def layer(cfg: Config, x, w_router, bias, experts, shared=None, residual=None, y=None,
          y_norm=None, eps=1e-5, want_norm=False, idx_out=None, w_out=None, workspace=None,
          events=None, debug=None):
    """moe_layer (whole step): returns y (and y_norm when want_norm).

    events: optional MoeEvents (hipEvent_t handles per stage) to receive the
    kernels' own start/stop timestamps; debug: optional dict of device
    buffers (``layer_debug_buffers``, any subset) for the intermediates."""
    torch = _torch()
    T, H = x.shape
    y = y if y is not None else torch.empty((T, H), dtype=torch.float32, device=x.device)
    if want_norm and y_norm is None:
        y_norm = torch.empty_like(y)
    ws = _workspace(layer_workspace(cfg, T), x.device, workspace)
    dbg = _layer_debug(debug)
    _check(lib().moe_layer(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                           _ptr(experts), _ptr(shared), _ptr(residual), _ptr(y), _ptr(y_norm),
                           eps, _ptr(idx_out), _ptr(w_out), _ptr(ws), ws.numel(),
                           ctypes.byref(events) if events is not None else None,
                           ctypes.byref(dbg) if dbg is not None else None, _stream()))
    return (y, y_norm) if want_norm else y


def layer_ptrs(cfg: Config, x, w_router, bias, expert_ptrs, shared=None, residual=None, y=None,
               y_norm=None, eps=1e-5, want_norm=False, idx_out=None, w_out=None,
               workspace=None, events=None, debug=None):
    """moe_layer_ptrs: as layer(), the routed records given by a device int64
    tensor of E record addresses (HBM or device-readable pinned host memory)."""
    torch = _torch()
    T, H = x.shape
    y = y if y is not None else torch.empty((T, H), dtype=torch.float32, device=x.device)
    if want_norm and y_norm is None:
        y_norm = torch.empty_like(y)
    ws = _workspace(layer_workspace(cfg, T), x.device, workspace)
    dbg = _layer_debug(debug)
    _check(lib().moe_layer_ptrs(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router), _ptr(bias),
                                _ptr(expert_ptrs), _ptr(shared), _ptr(residual), _ptr(y),
                                _ptr(y_norm), eps, _ptr(idx_out), _ptr(w_out), _ptr(ws),
                                ws.numel(), ctypes.byref(events) if events is not None else None,
                                ctypes.byref(dbg) if dbg is not None else None, _stream()))
    return (y, y_norm) if want_norm else y


NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def layer_noalloc(cfg: Config, x, w_router, bias, experts, shared=None, residual=None, y=None,
                  y_norm=None, eps=1e-5, want_norm=False, idx_out=None, w_out=None, events=None):
    """moe_layer_noalloc: as layer(), with the library's static device scratch
    instead of a workspace (nothing is allocated by the call; y / y_norm are
    created here only when not given)."""
    torch = _torch()
    T, H = x.shape
    y = y if y is not None else torch.empty((T, H), dtype=torch.float32, device=x.device)
    if want_norm and y_norm is None:
        y_norm = torch.empty_like(y)
    _check(lib().moe_layer_noalloc(ctypes.byref(cfg.c()), T, _ptr(x), _ptr(w_router),
                                   _ptr(bias), _ptr(experts), _ptr(shared), _ptr(residual),
                                   _ptr(y), _ptr(y_norm), eps, _ptr(idx_out), _ptr(w_out),
                                   ctypes.byref(events) if events is not None else None,
                                   _stream()))
    return (y, y_norm) if want_norm else y


def host_device_ptr(host_tensor) -> int:
    """Device-readable address of a pinned host tensor's storage."""
    out = ctypes.c_void_p()
    _check(lib().moe_host_device_ptr(ctypes.c_void_p(host_tensor.data_ptr()), ctypes.byref(out)))
    return int(out.value)


class ExpertCache:
    """One layer's expert cache (moe_cache_*): routed records in pinned host
    memory (``host_records``: a pinned uint8 tensor of E records), ``n_slots``
    of them cached in HBM, and the device table of record pointers that
    ``layer_ptrs`` reads (``self.table``)."""

    def __init__(self, cfg: Config, host_records, n_slots: int, n_pinned: int = 0,
                 max_promote: int = 2, max_pairs: int = 256, usage=None, device="cuda:0"):
        torch = _torch()
        import numpy as np
        self.cfg = cfg
        bb = blob_bytes(cfg)
        E = cfg.n_experts
        assert host_records.is_pinned() and host_records.numel() >= E * bb
        base = host_device_ptr(host_records)
        recs = (ctypes.c_void_p * E)(*[base + e * bb for e in range(E)])
        self.host_records = host_records
        self.slots = torch.empty(max(n_slots, 1) * bb, dtype=torch.uint8, device=device)
        self.table = torch.empty(E, dtype=torch.int64, device=device)
        self.max_pairs = max_pairs
        u = None
        if usage is not None:
            self._usage = np.ascontiguousarray(usage, dtype=np.uint64)
            u = self._usage.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
        h = ctypes.c_void_p()
        _check(lib().moe_cache_create(ctypes.byref(cfg.c()), n_slots, n_pinned, max_promote,
                                      max_pairs, recs, _ptr(self.slots), _ptr(self.table), u,
                                      _stream(), ctypes.byref(h)))
        self._h = h

    def step(self, idx, wait=False):
        _check(lib().moe_cache_step(self._h, _ptr(idx), idx.numel(), int(bool(wait)), _stream()))

    def prefetch(self, idx):
        """moe_cache_prefetch: start promotions of a predicted idx (device)."""
        _check(lib().moe_cache_prefetch(self._h, _ptr(idx), idx.numel(), _stream()))

    def publish(self):
        """moe_cache_publish: the stream waits for this cache's copies in flight
        and their entries point at the slots."""
        _check(lib().moe_cache_publish(self._h, _stream()))

    def stats(self) -> dict:
        s = MoeCacheStats()
        _check(lib().moe_cache_get_stats(self._h, ctypes.byref(s)))
        return {k: getattr(s, k) for k, _ in MoeCacheStats._fields_}

    def usage(self):
        import numpy as np
        out = np.zeros(self.cfg.n_experts, np.uint64)
        _check(lib().moe_cache_usage(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))))
        return out

    def slot_of(self):
        import numpy as np
        out = np.zeros(self.cfg.n_experts, np.int32)
        _check(lib().moe_cache_slot_of(self._h, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
        return out

    def close(self):
        if self._h:
            lib().moe_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cache_simulate(n_experts, n_slots, n_pinned, max_promote, idx, usage=None, pred=None):
    """The cache policy alone (host): per-step hits and misses, final slot_of;
    pred: optional per-step predictions prefetched before each step."""
    import numpy as np
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    pp = None
    if pred is not None:
        pred = np.ascontiguousarray(pred, dtype=np.int32)
        assert pred.shape == idx.shape
        pp = pred.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    n_steps = idx.shape[0]
    n = idx[0].size if n_steps else 0
    hits = np.zeros(n_steps, np.int32)
    misses = np.zeros(n_steps, np.int32)
    slot_of = np.zeros(n_experts, np.int32)
    u = None
    if usage is not None:
        usage = np.ascontiguousarray(usage, dtype=np.uint64)
        u = usage.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))
    i32p = ctypes.POINTER(ctypes.c_int32)
    _check(lib().moe_cache_simulate(n_experts, n_slots, n_pinned, max_promote, u,
                                    idx.ctypes.data_as(i32p), pp, n_steps, n,
                                    hits.ctypes.data_as(i32p), misses.ctypes.data_as(i32p),
                                    slot_of.ctypes.data_as(i32p)))
    return hits, misses, slot_of
