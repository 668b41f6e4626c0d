"""Host-side checks of bench.py (no GPU): the one-GPU guard and the lookup of
the committed HBM-traffic counters."""
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
