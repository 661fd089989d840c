"""Host-side checks of the benchmark's bookkeeping (no GPU): the visible-pair
count that every TFLOP/s figure divides by, the FLOP convention, the
traffic-record lookup and its source digest, and the refusal of more than
one GPU."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def brute_pairs(B, H, N, causal, kv_len):
    """Count (query, key) pairs whose score is not masked, one by one."""
    q = np.arange(N)[:, None]
    k = np.arange(N)[None, :]
    total = 0
    for b in range(B):
        L = N if kv_len is None else max(0, min(int(kv_len[b]), N))
        vis = np.broadcast_to(k < L, (N, N))
        if causal:
            vis = vis & (k <= q)
        total += int(vis.sum()) * H
    return total


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kv_len", [None, [0, 1, 7, 33, 40, 99]])
def test_pairs_match_brute_force(causal, kv_len):
    B, H, N = (6 if kv_len else 3), 2, 33
    w = SimpleNamespace(B=B, H=H, N=N)
    kv = None if kv_len is None else np.array(kv_len, np.int32)
    assert bench.pairs_per_batch(w, causal, kv) == brute_pairs(B, H, N, causal, kv)


def test_flop_convention_of_the_headline():
    """4 d per pair forward and 10 d backward: the headline's 2199 and 5498
    GFLOP at B=16, H=16, N=4096, d=128 (non-causal)."""
    w = SimpleNamespace(B=16, H=16, N=4096)
    pairs = bench.pairs_per_batch(w, False, None)
    assert pairs == 16 * 16 * 4096 * 4096
    assert 4 * 128 * pairs == 2199023255552
    assert 10 * 128 * pairs == 5497558138880


def test_traffic_record_follows_the_source_digest(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest()
    rec = {"kernel_source_digest": digest, "workloads": {"x:nc": {"fwd_bytes": 1, "bwd_call_bytes": 2}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.stored_traffic("x:nc") == {"fwd_bytes": 1, "bwd_call_bytes": 2}
    assert bench.stored_traffic("y:c") is None
    rec["kernel_source_digest"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.stored_traffic("x:nc") is None


def test_committed_traffic_record_is_current():
    """The committed counter bytes were taken with the current device
    sources, so the bench reports them (null would mean stale counters)."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as fh:
        rec = json.load(fh)
    assert rec["kernel_source_digest"] == bench.kernel_source_digest()
    for key in ("n4096_d128:nc", "n4096_d128:c", "long_16k:c"):
        assert rec["workloads"][key]["fwd_bytes"] > 0 and rec["workloads"][key]["bwd_call_bytes"] > 0


def test_digest_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "io_aware_exact_11_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("int f() {\n  return 1;  // one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_source_digest()
    (src / "k.hip").write_text("// header comment\nint f() {\n\n  return 1;  // another\n}\n")
    assert bench.kernel_source_digest() == d0
    (src / "k.hip").write_text("int f() {\n  return 2;\n}\n")
    assert bench.kernel_source_digest() != d0


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
