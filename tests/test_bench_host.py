"""Host-side logic of bench.py (CPU only): the single-GPU guard and the rule that a recorded HBM
traffic figure is reported only while the kernel sources it was taken on are unchanged."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for a refused run


def test_traffic_is_reported_only_for_unchanged_sources(monkeypatch):
    with open(bench.TRAFFIC_FILE) as fh:
        stored = json.load(fh)["kernels"]
    for kernel in bench.KERNEL_SOURCES:
        rec = stored[kernel]
        monkeypatch.setattr(bench, "source_digest", lambda k, d=rec["source_sha256"]: d)
        assert bench.recorded_traffic(kernel) == rec["bytes_per_launch"] > 0
        monkeypatch.setattr(bench, "source_digest", lambda k: "0" * 64)
        assert bench.recorded_traffic(kernel) is None


def test_source_digest_covers_every_listed_file():
    for kernel, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.isfile(os.path.join(bench.CSRC, f)), (kernel, f)
        assert len(bench.source_digest(kernel)) == 64


def test_pair_counts_match_brute_force():
    """Indexer work counts the causal pairs of rows with t + 1 > k (a row with at most k
    candidates keeps them all); attention work counts min(k, t + 1) pairs per row."""
    for q0, q1, k in [(0, 300, 64), (0, 64, 64), (10, 70, 64), (63, 65, 64), (500, 900, 2048),
                      (2040, 2060, 2048), (0, 1, 1)]:
        assert bench.causal_pairs_range(q0, q1) == sum(t + 1 for t in range(q0, q1))
        assert bench.scored_pairs_range(q0, q1, k) == sum(t + 1 for t in range(q0, q1) if t + 1 > k)
        assert bench.selected_pairs_range(q0, q1, k) == sum(min(k, t + 1) for t in range(q0, q1))
