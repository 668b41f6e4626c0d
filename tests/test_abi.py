"""C-ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, answers size queries, and rejects bad arguments with
the documented codes before anything is launched (every call here fails
validation, so no kernel is ever enqueued)."""
import ctypes
import os
import re

import pytest

import int4_routed_expert_moe_amd as moe
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

REAL = moe.Config.of(synth.REAL)
TINY = moe.Config.of(synth.TINY)
A = 0x7F0000000000  # an aligned fake address: only ever passed to calls that must fail validation


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return moe.lib()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert sorted(moe.EXPORTS) == _declared()


def test_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_blob_bytes(L):
    assert moe.blob_bytes(REAL) == 18_915_328
    assert moe.blob_bytes(TINY) == 51_200
    assert moe.blob_bytes(moe.Config.of(synth.REAL.with_bits(2))) == 9_478_144
    assert moe.blob_bytes(REAL) == synth.blob_bytes(synth.REAL)


def test_workspace_queries(L):
    for T in (1, 4, 16, 2048):
        assert moe.route_workspace(REAL, T) >= 2 * 4 * T * 256
        assert moe.expert_ffn_workspace(REAL, T) >= 4 * (T * 8 + T) * 2048
        assert moe.layer_workspace(REAL, T) > moe.expert_ffn_workspace(REAL, T)
        assert moe.layer_workspace(REAL, T) % 256 == 0


@pytest.mark.parametrize("field,value", [
    ("hidden", 100), ("hidden", 0), ("inter", 96), ("n_experts", 1), ("n_experts", 2048),
    ("n_group", 3), ("n_group", 0), ("topk_group", 0), ("topk_group", 9), ("top_k", 0),
    ("top_k", 17), ("n_shared", 2), ("wbits", 3), ("wbits", 16), ("wbits", 1), ("routed_scaling", 0.0),
    ("routed_scaling", float("nan")),
])
def test_bad_cfg_rejected(L, field, value):
    import dataclasses
    cfg = dataclasses.replace(REAL, **{field: value})
    c = cfg.c()
    assert L.moe_expert_blob_bytes(ctypes.byref(c)) == 0
    assert L.moe_layer_workspace(ctypes.byref(c), 1) == 0
    rc = L.moe_route(ctypes.byref(c), 1, A, A, A, A, A, A, 1 << 30, None)
    assert rc == moe.MOE_EINVAL
    assert L.moe_last_error()


@pytest.mark.parametrize("wbits,hidden,inter,ok", [
    (8, 7168, 2048, True), (8, 7424, 2048, False), (8, 6144, 2176, False),
    (4, 8192, 4096, True), (4, 8448, 2048, False), (2, 16384, 8192, True),
])
def test_row_length_limits(L, wbits, hidden, inter, ok):
    import dataclasses
    c = dataclasses.replace(REAL, wbits=wbits, hidden=hidden, inter=inter).c()
    assert (L.moe_expert_blob_bytes(ctypes.byref(c)) > 0) == ok


def test_top_k_above_candidates_rejected(L):
    import dataclasses
    cfg = dataclasses.replace(TINY, top_k=5)  # 1 kept group of 4 experts
    rc = L.moe_group(ctypes.byref(cfg.c()), 1, A, A, A, A, A, A, A, None)
    assert rc == moe.MOE_EINVAL


def test_null_cfg(L):
    assert L.moe_route(None, 1, A, A, A, A, A, A, 1 << 30, None) == moe.MOE_EINVAL
    assert L.moe_expert_blob_bytes(None) == 0


def test_route_errors(L):
    c = REAL.c()
    ws = moe.route_workspace(REAL, 4)
    assert L.moe_route(ctypes.byref(c), -1, A, A, A, A, A, A, ws, None) == moe.MOE_EINVAL
    assert L.moe_route(ctypes.byref(c), 4, None, A, A, A, A, A, ws, None) == moe.MOE_EINVAL
    assert L.moe_route(ctypes.byref(c), 4, A + 4, A, A, A, A, A, ws, None) == moe.MOE_EALIGN
    assert L.moe_route(ctypes.byref(c), 4, A, A, A, A, A, A, ws - 1, None) == moe.MOE_EWORKSPACE
    assert L.moe_route(ctypes.byref(c), 4, A, A, A, A, A, None, ws, None) == moe.MOE_EWORKSPACE
    assert L.moe_route(ctypes.byref(c), 4, A, A, A, A, A, A + 16, ws, None) == moe.MOE_EALIGN
    # T = 0 is a no-op that succeeds without touching any pointer
    assert L.moe_route(ctypes.byref(c), 0, None, None, None, None, None, None, 0, None) == 0


def test_quant_act_errors(L):
    assert L.moe_quant_act(-1, 32, 32, A, A, A, None) == moe.MOE_EINVAL
    assert L.moe_quant_act(2, 48, 32, A, A, A, None) == moe.MOE_EINVAL
    assert L.moe_quant_act(2, 0, 32, A, A, A, None) == moe.MOE_EINVAL
    assert L.moe_quant_act(2, 64, 32, A, None, A, None) == moe.MOE_EINVAL
    assert L.moe_quant_act(2, 64, 32, A, A + 8, A, None) == moe.MOE_EALIGN
    assert L.moe_quant_act(0, 64, 32, None, None, None, None) == 0
    # the block is 32 (Q8_0) or the whole row
    assert L.moe_quant_act(2, 128, 64, A, A, A, None) == moe.MOE_EINVAL
    assert L.moe_quant_act(0, 128, 128, None, None, None, None) == 0


def test_group_errors(L):
    c = REAL.c()
    assert L.moe_group(ctypes.byref(c), -2, A, A, A, A, A, A, A, None) == moe.MOE_EINVAL
    assert L.moe_group(ctypes.byref(c), 2, A, A, A, A, A, A, None, None) == moe.MOE_EINVAL
    assert L.moe_group(ctypes.byref(c), 2, A, A, A + 2, A, A, A, A, None) == moe.MOE_EALIGN
    assert L.moe_group(ctypes.byref(c), 0, None, None, None, None, None, None, None, None) == 0


def test_expert_ffn_errors(L):
    c = REAL.c()
    ws = moe.expert_ffn_workspace(REAL, 2)
    f = L.moe_expert_ffn
    assert f(ctypes.byref(c), 2, A, A, A, A, A, A, A, A, ws - 256, None, None) == moe.MOE_EWORKSPACE
    assert f(ctypes.byref(c), 2, A, A, A, A, None, A, A, A, ws, None, None) == moe.MOE_EINVAL
    assert f(ctypes.byref(c), 2, A, A, A, A, A, A, None, A, ws, None, None) == moe.MOE_EINVAL
    assert f(ctypes.byref(c), 2, A, A, A, A + 16, A, A, A, A, ws, None, None) == moe.MOE_EALIGN
    assert f(ctypes.byref(c), 2, A, A, A, A, A, A, A, A + 16, ws, None, None) == moe.MOE_EALIGN
    dbg = moe.MoeFfnDebug(A, A + 4, None, None, None, None)
    assert f(ctypes.byref(c), 2, A, A, A, A, A, A, A, A, ws, ctypes.byref(dbg), None) == \
        moe.MOE_EALIGN
    assert f(ctypes.byref(c), 0, None, None, None, None, None, None, None, None, 0, None,
             None) == 0


def test_combine_and_layer_errors(L):
    assert L.moe_combine(2, 6144, 17, A, A, None, None, A, None, 1e-5, None) == moe.MOE_EINVAL
    assert L.moe_combine(2, 6146, 8, A, A, None, None, A, None, 1e-5, None) == moe.MOE_EINVAL
    assert L.moe_combine(2, 6144, 8, A, A, None, None, None, None, 1e-5, None) == moe.MOE_EINVAL
    assert L.moe_combine(2, 6144, 8, A, A, A + 4, None, A, None, 1e-5, None) == moe.MOE_EALIGN
    assert L.moe_combine(2, 6144, 8, A, A, None, None, A, None, -1.0, None) == moe.MOE_EINVAL
    assert L.moe_rmsnorm(2, 6144, None, A, 1e-5, None) == moe.MOE_EINVAL
    # outputs may not overlap the row they are computed from (several workgroups per row)
    assert L.moe_rmsnorm(2, 64, A, A + 256, 1e-5, None) == moe.MOE_EINVAL
    assert b"overlaps" in L.moe_last_error()
    assert L.moe_combine(2, 64, 0, None, None, None, None, A, A + 16, 1e-5, None) == moe.MOE_EINVAL
    assert L.moe_mfma_peak(0, 10, A, None) == moe.MOE_EINVAL
    assert L.moe_mfma_peak(4, 0, A, None) == moe.MOE_EINVAL
    assert L.moe_mfma_peak(4, 1 << 21, A, None) == moe.MOE_EINVAL
    assert L.moe_mfma_peak(4, 10, None, None) == moe.MOE_EINVAL
    rp = L.moe_read_peak
    assert rp(A, 0, 4, A, None, None, None) == moe.MOE_EINVAL
    assert rp(A, 17, 4, A, None, None, None) == moe.MOE_EINVAL
    assert rp(A, 256, 0, A, None, None, None) == moe.MOE_EINVAL
    assert rp(A, 256, 1 << 21, A, None, None, None) == moe.MOE_EINVAL
    assert rp(None, 256, 4, A, None, None, None) == moe.MOE_EINVAL
    assert rp(A, 256, 4, None, None, None, None) == moe.MOE_EINVAL
    assert rp(A + 4, 256, 4, A, None, None, None) == moe.MOE_EALIGN
    c = REAL.c()
    ws = moe.layer_workspace(REAL, 1)
    lay = L.moe_layer
    assert lay(ctypes.byref(c), 1, A, A, A, A, A, None, A, None, 1e-5, None, None, A, ws - 1,
               None, None, None) == moe.MOE_EWORKSPACE
    assert lay(ctypes.byref(c), 1, A, A, A, A, None, None, A, None, 1e-5, None, None, A, ws,
               None, None, None) == moe.MOE_EINVAL
    assert lay(ctypes.byref(c), 1, A, A, A, A + 64, A, None, A, None, 1e-5, None, None, A, ws,
               None, None, None) == moe.MOE_EALIGN
    # the union dumps come as a set of six
    part = moe.MoeLayerDebug(None, None, A, A, None, None, None, None)
    assert lay(ctypes.byref(c), 1, A, A, A, A, A, None, A, None, 1e-5, None, None, A, ws,
               None, ctypes.byref(part), None) == moe.MOE_EINVAL
    mis = moe.MoeLayerDebug(A + 4)
    assert lay(ctypes.byref(c), 1, A, A, A, A, A, None, A, None, 1e-5, None, None, A, ws,
               None, ctypes.byref(mis), None) == moe.MOE_EALIGN


def test_layer_noalloc_rejects_batches_beyond_its_scratch(L):
    """The static scratch holds moe_layer's workspace up to its size; a larger
    batch fails with MOE_EWORKSPACE before anything touches a device."""
    c = REAL.c()
    assert moe.layer_workspace(REAL, 96) <= moe.NOALLOC_SCRATCH_BYTES
    big = 4096
    assert moe.layer_workspace(REAL, big) > moe.NOALLOC_SCRATCH_BYTES
    assert L.moe_layer_noalloc(ctypes.byref(c), big, A, A, A, A, A, None, A, None, 1e-5, None,
                               None, None, None) == moe.MOE_EWORKSPACE
    assert b"scratch" in L.moe_last_error()
    assert L.moe_layer_noalloc(ctypes.byref(c), -1, A, A, A, A, A, None, A, None, 1e-5, None,
                               None, None, None) == moe.MOE_EINVAL
    assert L.moe_layer_noalloc(ctypes.byref(c), 0, None, None, None, None, None, None, None,
                               None, 1e-5, None, None, None, None) == moe.MOE_OK


def test_fp8_records(L):
    """FP8 experts (wfmt 2) need byte codes (wbits 8), Q8_0 activations and
    multiples of 128; the record size agrees with the generator's and the
    oracle's layout."""
    import oracle
    f8 = moe.Config.of(synth.REAL.with_bits(synth.FP8))
    assert (f8.wbits, f8.wfmt) == (8, 2)
    H, I = synth.REAL.hidden, synth.REAL.inter
    assert moe.blob_bytes(f8) == 3 * I * H + 3 * (I // 128) * (H // 128) * 4 == 37_757_952
    assert moe.blob_bytes(f8) == synth.blob_bytes(synth.REAL.with_bits(synth.FP8))
    assert moe.blob_bytes(f8) == oracle.blob_bytes(H, I, oracle.FP8)
    for field, value in (("wbits", 4), ("wfmt", 3), ("act_block", moe.ACT_ROW)):
        c = f8.c()
        setattr(c, field, value)
        assert L.moe_expert_blob_bytes(ctypes.byref(c)) == 0, field


def test_per_row_activations_take_int4_or_int8_codes(L):
    for shape in (synth.REAL.with_bits(2), synth.REAL.with_bits(synth.MXFP4)):
        c = moe.Config.of(shape, act_block=moe.ACT_ROW).c()
        assert L.moe_expert_blob_bytes(ctypes.byref(c)) == 0  # rejected
    for bits in (4, 8):
        c = moe.Config.of(synth.REAL.with_bits(bits), act_block=moe.ACT_ROW).c()
        assert L.moe_expert_blob_bytes(ctypes.byref(c)) > 0
    bad = moe.Config.of(synth.REAL, act_block=64).c()
    assert L.moe_expert_blob_bytes(ctypes.byref(bad)) == 0


def test_strerror(L):
    for code in (0, -1, -2, -3, -4):
        assert L.moe_strerror(code)
    assert L.moe_strerror(-99) == b"unknown error"


def test_binding_refuses_host_tensors(L):
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        moe.quant_act(torch.zeros(2, 64))


def test_cache_create_rejects_bad_arguments(L):
    c = REAL.c()
    out = ctypes.c_void_p()
    recs = (ctypes.c_void_p * 256)(*([A] * 256))
    # pinned > slots
    assert L.moe_cache_create(ctypes.byref(c), 4, 5, 1, 8, recs, ctypes.c_void_p(A),
                              ctypes.c_void_p(A), None, None, ctypes.byref(out)) == moe.MOE_EINVAL
    # misaligned host record
    bad = (ctypes.c_void_p * 256)(*([A + 8] * 256))
    assert L.moe_cache_create(ctypes.byref(c), 4, 1, 1, 8, bad, ctypes.c_void_p(A),
                              ctypes.c_void_p(A), None, None, ctypes.byref(out)) == moe.MOE_EALIGN
    assert not out.value
    assert L.moe_cache_step(None, ctypes.c_void_p(A), 8, 0, None) == moe.MOE_EINVAL
    assert L.moe_cache_prefetch(None, ctypes.c_void_p(A), 8, None) == moe.MOE_EINVAL
    assert L.moe_cache_publish(None, None) == moe.MOE_EINVAL


def test_layer_ptrs_rejects_null_table(L):
    c = TINY.c()
    rc = L.moe_layer_ptrs(ctypes.byref(c), 1, A, A, A, None, A, None, A, None, 1e-5, None, None,
                          A, 1 << 30, None, None, None)
    assert rc == moe.MOE_EINVAL
