"""Whole-layer parity at the edges of the supported configurations: the most
experts (1024 in 64 groups) with the largest top-k (16, so T*K reaches 256 at
16 tokens), no shared expert, a single expert per token out of two, and the
longest int4 row (hidden 8192) -- each on the small-batch path and on the
chained path past 16 tokens."""
import numpy as np
import pytest
import torch

import int4_routed_expert_moe_amd as moe
import synth
from _inputs import DeviceLayer, assert_close_rms

pytestmark = pytest.mark.gpu

SHAPES = {
    "e1024_k16": synth.LayerShape(256, 128, 1024, 64, 8, 16),
    "e1024_k16_noshared": synth.LayerShape(256, 128, 1024, 64, 8, 16, n_shared=0),
    "e2_k1": synth.LayerShape(256, 128, 2, 1, 1, 1),
    "h8192": synth.LayerShape(8192, 128, 16, 4, 2, 4),
    "h8192_mxfp4": synth.LayerShape(8192, 128, 16, 4, 2, 4, wbits=synth.MXFP4),
}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


def h(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("name,T", [
    ("e1024_k16", 1), ("e1024_k16", 3), ("e1024_k16", 16), ("e1024_k16", 24),
    ("e1024_k16_noshared", 1), ("e1024_k16_noshared", 5), ("e1024_k16_noshared", 20),
    ("e2_k1", 1), ("e2_k1", 16), ("e2_k1", 17),
    ("h8192", 1), ("h8192", 2), ("h8192", 20),
    ("h8192_mxfp4", 1), ("h8192_mxfp4", 20),
])
def test_layer_at_config_edges(dev, name, T):
    shape = SHAPES[name]
    lay = DeviceLayer(shape, 300 + T, bias="zipf")
    cfg = moe.Config.of(shape)
    x = synth.tokens(shape, 301, T)
    res = synth.tokens(shape, 302, T)
    idx_d = torch.empty((T, shape.top_k), dtype=torch.int32, device=dev)
    w_d = torch.empty((T, shape.top_k), dtype=torch.float32, device=dev)
    y, yn = moe.layer(cfg, torch.from_numpy(x).to(dev), lay.wr_d, lay.bias_d, lay.experts_d,
                      lay.shared_d if shape.n_shared else None,
                      residual=torch.from_numpy(res).to(dev), want_norm=True, idx_out=idx_d,
                      w_out=w_d)
    ref = lay.oracle_layer(x, residual=res, want_norm=True)
    assert np.array_equal(h(idx_d), ref["idx"])
    assert np.array_equal(h(w_d), ref["w"])
    assert_close_rms(h(y), ref["y"], 2e-3, "y")
    assert_close_rms(h(yn), ref["y_norm"], 2e-3, "y_norm")
