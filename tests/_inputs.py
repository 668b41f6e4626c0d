"""Seeded device inputs for the GPU tests (built from the synth generator)."""
from __future__ import annotations

import numpy as np

import synth


def pairs_of(idx, n_shared):
    """(pair, expert, token) of every routed slot kept and of the shared expert
    (pair t*K + k: slot (t, k); pair T*K + t: the shared expert on token t)."""
    T, K = idx.shape
    out = [(t * K + k, int(idx[t, k]), t) for t in range(T) for k in range(K) if idx[t, k] >= 0]
    if n_shared:
        out += [(T * K + t, synth.SHARED_ID, t) for t in range(T)]
    return out


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def assert_close_rms(got, ref, tol=2e-3, what=""):
    """max |got - ref| <= tol * RMS(ref) (the layer-output bar of the method)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    bound = tol * rms(ref)
    assert err <= bound, f"{what}: max|err| {err:.3e} > {tol} * RMS {rms(ref):.3e}"
    return err / max(rms(ref), 1e-30)


class DeviceLayer:
    """One synthetic MoE layer resident on the GPU, plus host copies on demand.

    Router weights and bias are drawn on the host; expert records are drawn on
    the host for small shapes and by the GPU copy of the generator for the
    real shape (identical bytes either way: the generator test checks it, and
    each such layer re-checks one record against the host generator).  Host
    copies of GPU-drawn records are read back from device memory (no kernel
    of the library writes a record), since drawing 19 MB on the host takes
    ~0.2 s per record."""

    def __init__(self, shape, seed, layer=0, bias="uniform", device="cuda:0", gpu_gen=None):
        import torch
        self.shape, self.seed, self.layer = shape, seed, layer
        self.dev = torch.device(device)
        self.wr = synth.router_weights(shape, seed, layer)
        if bias == "zipf":
            self.bias = synth.router_bias_zipf(shape, seed, layer)
        else:
            self.bias = synth.router_bias_uniform(shape, seed, layer)
        self.wr_d = torch.from_numpy(self.wr).to(self.dev)
        self.bias_d = torch.from_numpy(self.bias).to(self.dev)
        bb = synth.blob_bytes(shape)
        self.blob_bytes = bb
        E = shape.n_experts
        if gpu_gen is None:
            gpu_gen = bb * E > (64 << 20)
        self.experts_d = torch.empty(E * bb, dtype=torch.uint8, device=self.dev)
        self.shared_d = torch.empty(bb, dtype=torch.uint8, device=self.dev)
        self._cache = {}
        self.gpu_gen = gpu_gen
        if gpu_gen:
            stream = torch.cuda.current_stream().cuda_stream
            synth.expert_blobs_gpu(shape, seed, layer, list(range(E)), self.experts_d.data_ptr(),
                                   bb, stream)
            synth.expert_blobs_gpu(shape, seed, layer, [synth.SHARED_ID], self.shared_d.data_ptr(),
                                   bb, stream)
            torch.cuda.synchronize()
            probe = (layer * 37 + 5) % E
            assert np.array_equal(self.blob(probe),
                                  synth.expert_blob(shape, seed, layer, probe)), "generator"
        else:
            host = np.concatenate([self.blob(e) for e in range(E)])
            self.experts_d.copy_(torch.from_numpy(host))
            self.shared_d.copy_(torch.from_numpy(self.blob(synth.SHARED_ID)))

    def _dev_record(self, e: int):
        bb = self.blob_bytes
        return self.shared_d if e == synth.SHARED_ID else self.experts_d[e * bb:(e + 1) * bb]

    def blob(self, e: int) -> np.ndarray:
        if self.gpu_gen:
            return self._dev_record(e).cpu().numpy()
        if e not in self._cache:
            self._cache[e] = synth.expert_blob(self.shape, self.seed, self.layer, e)
        return self._cache[e]

    def set_record(self, e: int, rec: np.ndarray) -> None:
        """Replace expert e's record (or the shared one) on the device and in
        the host copies."""
        import torch
        assert rec.dtype == np.uint8 and rec.size == self.blob_bytes
        self._dev_record(e).copy_(torch.from_numpy(np.ascontiguousarray(rec)))
        torch.cuda.synchronize()
        if not self.gpu_gen:
            self._cache[e] = rec.copy()

    def oracle_layer_on_gpu_qh(self, x, dumps, residual=None, want_norm=False, top_p=0.0,
                               tokens=None, act_block=32):
        """The oracle layer with each down projection taken on the GPU's own
        Q8_0(h) -- after checking that decision: the dumped q_h / d_h
        (moe_layer_debug) are exactly Q8_0 of the dumped h, and h is within the
        fp32 summation bound of the oracle's fp64 h.  Q8_0 of h is an fp32
        decision on a value whose last bits depend on the summation order, so
        where h sits within rounding of a code boundary both codes are
        correct; the down projection of the GPU's codes is then the unique
        comparand.  tokens: row of each x row in the dumps' batch (default
        0..len(x)-1), when x is a sample of a larger batch.  act_block: the
        activation format (Q8_0, or oracle.ACT_ROW: one scale per row, the
        same argument for that row's codes).  Returns oracle.layer's dict plus
        'qh_flips', the pairs whose codes differ from the oracle's own."""
        import oracle
        s = self.shape
        H, I, K, wb = s.hidden, s.inter, s.top_k, s.wbits
        tol_h = max(1e-5, 8 * (H // 32) * 2.0 ** -24)
        x = np.ascontiguousarray(x, np.float32)
        T = x.shape[0]
        rows = np.arange(T) if tokens is None else np.asarray(tokens)
        n_batch = int(dumps["h"].shape[0]) // (K + s.n_shared)
        idx, w, margin = oracle.route(x, self.wr, self.bias, s.n_group, s.topk_group, K,
                                      s.routed_scaling, top_p)
        q, d = oracle.quant_act(x, act_block)
        eo = np.zeros((T, K, H), np.float32)
        so = np.zeros((T, H), np.float32) if s.n_shared else None
        flips = 0
        blobs = {}
        for p, e, t in pairs_of(idx, s.n_shared):
            gp = rows[t] * K + p % K if p < T * K else n_batch * K + rows[t]  # in the dumps
            if e not in blobs:
                blobs[e] = self.blob(e)
            hr = oracle.gate_up(blobs[e], H, I, wb, q[t], d[t], act_block=act_block)["h"]
            hg, qg, dg = dumps["h"][gp], dumps["q_h"][gp], dumps["d_h"][gp]
            assert_close_rms(hg, hr, tol_h, f"h of pair {gp}")
            qc, dc = oracle.quant_act(hg, act_block)
            assert np.array_equal(qg, qc) and np.array_equal(dg, dc), f"codes of h, pair {gp}"
            flips += not np.array_equal(oracle.quant_act(hr, act_block)[0], qg)
            y, _ = oracle.down(blobs[e], H, I, wb, qg, dg, act_block=act_block)
            if p < T * K:
                eo[t, p % K] = y
            else:
                so[t] = y
        res = oracle.combine(eo, w, so, residual, 1e-5, want_norm)
        y, yn = res if want_norm else (res, None)
        return dict(idx=idx, w=w, margin=margin, y=y, y_norm=yn, qh_flips=flips)

    def oracle_layer(self, x, residual=None, want_norm=False, top_p=0.0, act_block=32):
        import oracle
        s = self.shape
        shared = self.blob(synth.SHARED_ID) if s.n_shared else None
        return oracle.layer(x, self.wr, self.bias, self.blob, shared,
                            H=s.hidden, I=s.inter, n_experts=s.n_experts, n_group=s.n_group,
                            topk_group=s.topk_group, top_k=s.top_k, scale=s.routed_scaling,
                            wbits=s.wbits, residual=residual, want_norm=want_norm,
                            top_p_value=top_p, act_block=act_block)
