"""moe_layer_noalloc (the entry point for callers that cannot allocate: its
workspace is the library's static device scratch) against moe_layer with a
workspace: the same kernels, so the outputs must be bit-identical -- on two
calls in a row, the second with a smaller batch (the scratch keeps the first
call's contents), on the small-batch path and the chained path, with and
without the residual / RMSNorm outputs."""
import numpy as np
import pytest
import torch

import int4_routed_expert_moe_amd as moe
import synth
from _inputs import DeviceLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def real(dev):
    return DeviceLayer(synth.REAL, synth.SEEDS["decode"])


def to_d(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def h(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _both(lay, x, dev, norm):
    cfg = moe.Config.of(lay.shape)
    T = x.shape[0]
    res = to_d(synth.tokens(lay.shape, 900 + T, T), dev) if norm else None
    outs = []
    for fn in (moe.layer, moe.layer_noalloc):
        idx = torch.full((T, lay.shape.top_k), -7, dtype=torch.int32, device=dev)
        w = torch.full((T, lay.shape.top_k), -7.0, dtype=torch.float32, device=dev)
        out = fn(cfg, to_d(x, dev), lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                 residual=res, want_norm=norm, idx_out=idx, w_out=w)
        outs.append([h(o) for o in (out if norm else (out,))] + [h(idx), h(w)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("Ts", [(16, 4), (40, 1), (96, 24), (8, 2)])
def test_noalloc_matches_layer_twice(dev, real, Ts):
    for i, T in enumerate(Ts):
        x = synth.tokens_perturbed(synth.REAL, 800 + T, T) if T > 1 else \
            synth.tokens(synth.REAL, 800, 1, start=9)
        _both(real, x, dev, norm=(i == 1))


def test_noalloc_fp8_small_batches(dev):
    """FP8 experts on the small-batch kernels: 4 tokens, then 1."""
    lay = DeviceLayer(synth.REAL.with_bits(synth.FP8), synth.SEEDS["decode"])
    _both(lay, synth.tokens_perturbed(synth.REAL, 804, 4), dev, norm=True)
    _both(lay, synth.tokens(synth.REAL, 801, 1, start=3), dev, norm=False)
    del lay


def test_noalloc_tiny_ragged(dev):
    lay = DeviceLayer(synth.TINY, synth.SEEDS["tiny"])
    for T in (33, 5, 1):
        _both(lay, synth.tokens(synth.TINY, 70 + T, T), dev, norm=T == 5)


def test_noalloc_rejects_a_batch_beyond_its_scratch(dev, real):
    cfg = moe.Config.of(synth.REAL)
    T = 2048
    x = torch.zeros((T, synth.REAL.hidden), dtype=torch.float32, device=dev)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_noalloc(cfg, x, real.wr_d, real.bias_d, real.experts_d, real.shared_d)
    assert e.value.code == moe.MOE_EWORKSPACE
