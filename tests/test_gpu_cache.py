"""Expert records read through a table of pointers (moe_layer_ptrs), in HBM
and in pinned host memory, and the expert cache that moves them (moe_cache_*):
every output bit-identical to moe_layer on the same record bytes, and the
cache's hit/miss accounting equal to the host policy on the same routing."""
import numpy as np
import pytest
import torch

import int4_routed_expert_moe_amd as moe
import synth
from _inputs import DeviceLayer, assert_close_rms

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


def h(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def hbm_table(lay):
    bb = lay.blob_bytes
    base = lay.experts_d.data_ptr()
    return torch.tensor([base + e * bb for e in range(lay.shape.n_experts)], dtype=torch.int64,
                        device=lay.dev)


def pinned_records(lay):
    host = torch.empty(lay.experts_d.numel(), dtype=torch.uint8, pin_memory=True)
    host.copy_(lay.experts_d.cpu())
    return host


def run_both(lay, x_np, table, dev):
    cfg = moe.Config.of(lay.shape)
    x = torch.from_numpy(x_np).to(dev)
    T, K = x.shape[0], lay.shape.top_k
    i1 = torch.empty((T, K), dtype=torch.int32, device=dev)
    i2 = torch.empty_like(i1)
    w1 = torch.empty((T, K), dtype=torch.float32, device=dev)
    w2 = torch.empty_like(w1)
    y1 = moe.layer(cfg, x, lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d, idx_out=i1,
                   w_out=w1)
    y2 = moe.layer_ptrs(cfg, x, lay.wr_d, lay.bias_d, table, lay.shared_d, idx_out=i2, w_out=w2)
    assert np.array_equal(h(i1), h(i2))
    assert np.array_equal(h(w1).view(np.uint32), h(w2).view(np.uint32))
    assert np.array_equal(h(y1).view(np.uint32), h(y2).view(np.uint32))
    return h(i2)


@pytest.mark.parametrize("T", [1, 4, 40])
def test_table_of_hbm_records_is_bit_identical(dev, T):
    lay = DeviceLayer(synth.TINY, synth.SEEDS["tiny"])
    run_both(lay, synth.tokens(synth.TINY, 31, T), hbm_table(lay), dev)


def test_real_records_half_in_host_memory(dev):
    lay = DeviceLayer(synth.REAL, synth.SEEDS["decode"])
    host = pinned_records(lay)
    hb = moe.host_device_ptr(host)
    bb = lay.blob_bytes
    ptrs = [(hb if e % 2 else lay.experts_d.data_ptr()) + e * bb for e in range(256)]
    table = torch.tensor(ptrs, dtype=torch.int64, device=dev)
    for T, start in ((1, 0), (1, 1), (4, 5), (24, 9)):
        run_both(lay, synth.tokens(synth.REAL, synth.SEEDS["decode"], T, start=start), table,
                 dev)


def test_cache_steps_match_policy(dev):
    """Tiny layer, 3 slots (1 pinned), copies completed within each call:
    outputs bit-identical every step; hits, misses and the final placement
    equal to the host policy run on the same routing."""
    shape = synth.TINY
    lay = DeviceLayer(shape, synth.SEEDS["tiny"], bias="zipf")
    cfg = moe.Config.of(shape)
    host = pinned_records(lay)
    usage = np.array([0, 0, 3, 0, 1, 0, 0, 0], np.uint64)
    cache = moe.ExpertCache(cfg, host, n_slots=3, n_pinned=1, max_promote=1, max_pairs=8,
                            usage=usage)
    idxs = []
    for step in range(30):
        x = synth.tokens(shape, 500 + step, 2)
        idxs.append(run_both(lay, x, cache.table, dev).ravel())
        i_d = torch.from_numpy(idxs[-1]).to(dev)
        cache.step(i_d, wait=True)
    st = cache.stats()
    hits, misses, slot_of = moe.cache_simulate(8, 3, 1, 1, np.stack(idxs), usage=usage)
    assert st["steps"] == 30
    assert st["hits"] == hits.sum() and st["misses"] == misses.sum()
    assert np.array_equal(cache.slot_of(), slot_of)
    assert st["completed"] == st["promotions"]
    assert np.array_equal(cache.usage(), usage + np.bincount(
        np.concatenate([np.unique(i) for i in idxs]), minlength=8).astype(np.uint64))
    cache.close()


def test_cache_async_real_decode(dev):
    """Real layer, 32 slots (8 pinned from a first pass's usage), copies in
    flight across calls: every step still bit-identical."""
    lay = DeviceLayer(synth.REAL, synth.SEEDS["stack"], bias="zipf")
    cfg = moe.Config.of(synth.REAL)
    host = pinned_records(lay)
    warm = [run_both(lay, synth.tokens(synth.REAL, 7, 1, start=s), hbm_table(lay), dev)
            for s in range(20)]
    usage = np.bincount(np.concatenate(warm).ravel(), minlength=256).astype(np.uint64)
    cache = moe.ExpertCache(cfg, host, n_slots=32, n_pinned=8, max_promote=2, max_pairs=8,
                            usage=usage)
    for s in range(60):
        idx = run_both(lay, synth.tokens(synth.REAL, 8, 1, start=s), cache.table, dev)
        cache.step(torch.from_numpy(idx.ravel()).to(dev))
    torch.cuda.synchronize()
    st = cache.stats()
    assert st["hits"] + st["misses"] == st["routed"]
    assert st["completed"] <= st["promotions"] and st["resident"] <= 32
    assert st["hits"] > 0 and st["misses"] > 0
    cache.close()


def test_two_layers_share_the_copy_stream(dev):
    """Two layers' caches used alternately (their promotions share the
    device's copy stream): outputs bit-identical every step; with copies
    completed within each call, each cache's counts and placement equal the
    host policy on its own routing; with copies in flight across calls, the
    counts stay consistent."""
    shape = synth.TINY
    lays = [DeviceLayer(shape, synth.SEEDS["tiny"], layer, bias="zipf") for layer in (0, 1)]
    cfg = moe.Config.of(shape)
    caches = [moe.ExpertCache(cfg, pinned_records(lay), n_slots=3, n_pinned=1, max_promote=1,
                              max_pairs=8, usage=np.array([0, 1, 0, 0, 0, 0, 2, 0], np.uint64))
              for lay in lays]
    idxs = [[], []]
    for step in range(24):
        l = step % 2
        idx = run_both(lays[l], synth.tokens(shape, 700 + step, 2), caches[l].table, dev).ravel()
        idxs[l].append(idx)
        caches[l].step(torch.from_numpy(idx).to(dev), wait=True)
    for l in (0, 1):
        st = caches[l].stats()
        hits, misses, slot_of = moe.cache_simulate(8, 3, 1, 1, np.stack(idxs[l]),
                                                   usage=np.array([0, 1, 0, 0, 0, 0, 2, 0],
                                                                  np.uint64))
        assert st["hits"] == hits.sum() and st["misses"] == misses.sum()
        assert np.array_equal(caches[l].slot_of(), slot_of)
    for step in range(24, 48):
        l = step % 2
        idx = run_both(lays[l], synth.tokens(shape, 700 + step, 2), caches[l].table, dev).ravel()
        caches[l].step(torch.from_numpy(idx).to(dev))
    torch.cuda.synchronize()
    for c in caches:
        st = c.stats()
        assert st["hits"] + st["misses"] == st["routed"]
        assert st["completed"] <= st["promotions"] and st["resident"] <= 3
        c.close()


def test_routing_one_layer_ahead(dev):
    """Three tiny layers in a pre-norm stack, each with a 3-slot cache (no
    pinning): before layer l runs, layer l+1's routing is predicted from
    layer l's input (moe_route with layer l+1's router) and prefetched into
    layer l+1's cache.  The prediction is bit-exact against the oracle's
    routing of that input; every layer output is bit-identical to moe_layer
    on the HBM records, and the first step's against the oracle; the cache
    with prefetch counts its prefetches, and its counts stay consistent."""
    import oracle
    shape = synth.TINY
    L = 3
    lays = [DeviceLayer(shape, synth.SEEDS["tiny"], layer, bias="zipf") for layer in range(L)]
    cfg = moe.Config.of(shape)
    K = shape.top_k

    def run(prefetch):
        caches = [moe.ExpertCache(cfg, pinned_records(lay), n_slots=3, n_pinned=0,
                                  max_promote=2, max_pairs=8) for lay in lays]
        outs = []
        for step in range(16):
            hcur = torch.from_numpy(synth.tokens(shape, 900 + step, 2)).to(dev)
            xn = moe.rmsnorm(hcur)
            for l in range(L):
                lay = lays[l]
                if prefetch and l + 1 < L:
                    nxt = lays[l + 1]
                    pi, _ = moe.route(cfg, xn, nxt.wr_d, nxt.bias_d)
                    ri, _, _ = oracle.route(h(xn), nxt.wr, nxt.bias, shape.n_group,
                                            shape.topk_group, K, shape.routed_scaling)
                    assert np.array_equal(h(pi), ri), (step, l)
                    caches[l + 1].prefetch(pi.view(-1))
                if prefetch:
                    caches[l].publish()
                i1 = torch.empty((2, K), dtype=torch.int32, device=dev)
                y1, yn1 = moe.layer_ptrs(cfg, xn, lay.wr_d, lay.bias_d, caches[l].table,
                                         lay.shared_d, residual=hcur, want_norm=True,
                                         idx_out=i1)
                y2, yn2 = moe.layer(cfg, xn, lay.wr_d, lay.bias_d, lay.experts_d, lay.shared_d,
                                    residual=hcur, want_norm=True)
                assert np.array_equal(h(y1).view(np.uint32), h(y2).view(np.uint32))
                assert np.array_equal(h(yn1).view(np.uint32), h(yn2).view(np.uint32))
                if step == 0:
                    ref = lay.oracle_layer(h(xn), residual=h(hcur), want_norm=True)
                    assert np.array_equal(h(i1), ref["idx"])
                    assert_close_rms(h(y1), ref["y"], 2e-3, f"layer {l}")
                caches[l].step(i1.view(-1), wait=not prefetch)
                outs.append(h(y1))
                hcur, xn = y1, yn1
        stats = [c.stats() for c in caches]
        for c in caches:
            c.close()
        return outs, stats

    outs0, st0 = run(False)
    outs1, st1 = run(True)
    for a, b in zip(outs0, outs1):  # the cache state never changes a result
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    for l in range(L):
        assert st1[l]["hits"] + st1[l]["misses"] == st1[l]["routed"]
        assert st0[l]["prefetched"] == 0
    assert st1[0]["prefetched"] == 0  # nothing routes layer 0 ahead
    assert sum(s["prefetched"] for s in st1[1:]) > 0
