"""Seeded device inputs for the GPU tests (built from the synth generator)."""
from __future__ import annotations

import numpy as np

import synth


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

    def oracle_layer(self, x, residual=None, want_norm=False, top_p=0.0):
        import oracle
        s = self.shape
        shared = self.blob(synth.SHARED_ID) if s.n_shared else None
        return oracle.layer(x, self.wr, self.bias, self.blob, shared,
                            H=s.hidden, I=s.inter, n_experts=s.n_experts, n_group=s.n_group,
                            topk_group=s.topk_group, top_k=s.top_k, scale=s.routed_scaling,
                            wbits=s.wbits, residual=residual, want_norm=want_norm,
                            top_p_value=top_p)
