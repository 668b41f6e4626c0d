"""The measurement loops do the work they are counted for: moe_mfma_peak
(the matrix-core-only loop bench.py reports beside the published int8
peak) -- every thread's checksum equals the CPU's value of 8 chains x iters
int8 16x16x64 products of the kernel's operands, i.e. no MFMA was elided or
misread; moe_read_peak (the plain streaming read reported beside the HBM
peak) -- the XOR of its per-wave checksums is the XOR of every word of the
buffer, for sizes that end inside the unrolled loop and in its tail."""
import numpy as np
import pytest
import torch

import int4_routed_expert_moe_amd as moe

pytestmark = pytest.mark.gpu


def expected_checksums(iters):
    # operand byte j of lane l, as the kernel builds them
    a = [np.array([(7 * l + 3 * j) & 3 for j in range(16)], np.int64) for l in range(64)]
    b = [np.array([(5 * l + j) % 3 for j in range(16)], np.int64) for l in range(64)]
    # A [16 rows][64 K]: row m, K group g from lane 16 g + m; B [64 K][16 cols] likewise
    A = np.zeros((16, 64), np.int64)
    B = np.zeros((64, 16), np.int64)
    for l in range(64):
        m, g = l % 16, l // 16
        A[m, 16 * g:16 * g + 16] = a[l]
        B[16 * g:16 * g + 16, m] = b[l]
    C = A @ B
    out = np.zeros(256, np.int64)
    for t in range(256):
        l = t % 64
        n, g = l % 16, l // 16
        out[t] = sum(range(8)) + 8 * iters * int(C[4 * g:4 * g + 4, n].sum())
    return out


def test_mfma_peak_checksums():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    n_wg, iters = 3, 5
    out = torch.full((n_wg * 256,), -1, dtype=torch.int32, device=dev)
    ops = moe.mfma_peak(n_wg, iters, out)
    assert ops == n_wg * 4 * iters * 8 * 32768
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(n_wg, 256).astype(np.int64)
    want = expected_checksums(iters)
    for w in range(n_wg):
        assert np.array_equal(got[w], want), w


@pytest.mark.parametrize("nbytes,n_wg", [(16, 1), (16 * 1000, 3), (1 << 20, 7), (96 << 20, 2048)])
def test_read_peak_reads_every_word(nbytes, n_wg):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(nbytes + n_wg)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4 + 8,), generator=g, dtype=torch.int32)
    buf = host.to(dev)  # 8 words past nbytes that must not be read
    out = torch.full((n_wg * 4,), 0x5A5A5A5A, dtype=torch.int32, device=dev)
    moe.read_peak(buf, nbytes, n_wg, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy()[:nbytes // 4].view(np.uint32))
    assert got == want


def test_stale_hip_error_is_not_reported():
    """A failed HIP call of the caller's (here: the elapsed time of two
    events never recorded) leaves HIP's last-error state set; the next
    library call clears it on entry and reports success for its own
    launches."""
    import ctypes
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = torch.device("cuda:0")
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                path = line.split()[-1]
                break
    assert path, "HIP runtime not loaded"
    H = ctypes.CDLL(path)
    H.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    H.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    H.hipEventDestroy.argtypes = [ctypes.c_void_p]
    out = torch.zeros(256, dtype=torch.int32, device=dev)  # before: torch checks the state too
    torch.cuda.synchronize()
    a, b = ctypes.c_void_p(), ctypes.c_void_p()
    assert H.hipEventCreate(ctypes.byref(a)) == 0 and H.hipEventCreate(ctypes.byref(b)) == 0
    ms = ctypes.c_float()
    assert H.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0  # neither was recorded
    moe.mfma_peak(1, 2, out)  # raises MoeError on a non-zero return
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().astype(np.int64), expected_checksums(2))
    H.hipEventDestroy(a)
    H.hipEventDestroy(b)
