"""Host-side checks of bench.py (no GPU): the one-GPU guard, the lookup of
the committed HBM-traffic counters, and the bounds a prefill line reports."""
import hashlib
import importlib.util
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "error" in json.loads(r.stdout.strip().splitlines()[-1])


def test_traffic_lookup_follows_the_source_hash():
    bench = _bench()
    assert bench.measured_traffic("no-such-workload") is None
    path = os.path.join(ROOT, "profiles", "decode_hbm_traffic.md")
    m = re.search(r"src_sha256=([0-9a-f]+) bytes_per_launch=(\d+)", open(path).read())
    assert m, "the decode summary carries its machine-readable line"
    csrc = os.path.join(ROOT, "int4_routed_expert_moe_amd", "csrc")
    src = b"".join(open(os.path.join(csrc, f), "rb").read() for f in bench.TRAFFIC_SOURCES)
    assert hashlib.sha256(src).hexdigest() == bench.sources_sha256()
    assert "decode.h" in bench.TRAFFIC_SOURCES  # the kernels themselves
    got = bench.measured_traffic("decode")
    if hashlib.sha256(src).hexdigest() == m.group(1):
        # counters of these very sources: within 1 % above the algorithmic
        # bytes of one gate/up launch (8 experts of 12,615,680 B + activations)
        assert got == float(m.group(2))
        assert 100.8e6 <= got <= 1.01 * 100.83e6
    else:
        assert got is None  # stale counters are never reported


def test_prefill_gate_up_bounds():
    """The 2048-token layer: with Zipf routing nearly every expert is used and
    the weights (one read of each used expert's gate and up) outweigh the
    matrix-core work; on 8 experts the MFMA bound rules; Q8_0 activations add
    one convert and one multiply-add per (pair, gate or up row, 32-block)."""
    bench = _bench()
    sys.path.insert(0, ROOT)
    import synth
    s = synth.REAL
    T, pairs = 2048, 2048 * s.top_k
    n_pairs = pairs + T * s.n_shared  # 18,432 with the shared expert
    # Zipf: 256 experts used
    b, ops, nbytes, fix = bench.gate_up_bounds(s, T, 256, pairs, True)
    assert ops == 2 * n_pairs * 2 * 2048 * 6144 and fix == 0
    per_expert = 2 * 2048 * 6144 // 2 + 2 * 2048 * 4  # codes + row scales of gate and up
    assert nbytes >= (256 + 1) * per_expert
    assert max(b, key=b.get) == "hbm"
    assert abs(b["mfma"] - ops / 5e15) < 1e-12
    # dense: the same pairs on 8 experts
    b, _, nbytes, _ = bench.gate_up_bounds(s, T, 8, pairs, True)
    assert max(b, key=b.get) == "mfma" and b["hbm"] < b["mfma"] / 4
    # Q8_0: 2 rows (gate, up) x 2048 x 192 blocks per pair
    b, _, _, fix = bench.gate_up_bounds(s, T, 8, pairs, False)
    assert fix == n_pairs * 2 * 2048 * (6144 // 32)
    assert max(b, key=b.get) == "alu"
    assert abs(b["alu"] - 2 * fix / (256 * 4 * 16 * 2.4e9)) < 1e-12


def test_small_phase_bytes_cover_the_step():
    """The step-floor chain reads, per launch of the small-batch step, the
    router matrix, the shared expert's gate/up, the routed experts' gate/up
    and every used expert's down rows: together every weight byte of the
    step once (the records of U routed experts and the shared one, the
    router matrix), and the split at the record's down part."""
    bench = _bench()
    sys.path.insert(0, ROOT)
    import synth
    s = synth.REAL
    bb = 18_915_328  # int4 record at the real shape
    phases = bench.small_phase_bytes(s, 8, bb)
    assert phases == [6144 * 256 * 4, 12_599_296, 8 * 12_599_296, 9 * 6_316_032]
    assert sum(phases) == s.n_experts * s.hidden * 4 + 9 * bb
    # gate/up codes (two I x H/2 matrices) and their 2 I row scales
    assert bench.gate_up_record_bytes(s) == 2 * 2048 * 6144 // 2 + 2 * 2048 * 4
