"""Host logic of bench.py (no GPU): the byte accounting behind its roofline figures and the gate
on the recorded HBM-traffic figure."""
import hashlib
import os

import numpy as np

import bench
import workloads


def test_bytes_per_token_head_matches_the_pool_layout():
    # key and value codes (32 B each) plus fp16 (scale, zero) per group for keys and values
    assert bench.bytes_per_token_head(128) == 72
    assert bench.bytes_per_token_head(64) == 80


def test_history_bytes_of_the_100k_layer():
    wl = workloads.get("qwen3_8b_100k")
    n_hist = 100000 - 320
    pages = -(-n_hist // 64)
    want = 8 * n_hist * 72 + pages * 4 + 8 * 320 * 128 * 2 * 2
    assert bench.history_bytes(wl, [100000]) == want
    # a page table without sharing counts the same bytes
    table = np.arange(pages, dtype=np.int32)[None]
    assert bench.history_bytes(wl, [100000], table) == want


def test_shared_pages_count_once():
    wl = workloads.get("qwen3_8b_100k")
    lengths = [320 + 64 * 10, 320 + 64 * 4 + 5]
    table = np.array([list(range(10)), [0, 1, 2, 3, 10, 0, 0, 0, 0, 0]], dtype=np.int32)
    unique_pages_tokens = 64 * 10 + 5          # pages 0..9 of sequence 0, page 10 with 5 tokens
    want = (8 * 72 * unique_pages_tokens + (10 + 5) * 4
            + 2 * 8 * 320 * 128 * 2 * 2)
    assert bench.history_bytes(wl, lengths, table) == want
    # without the table every sequence's pages count
    assert bench.history_bytes(wl, lengths) == want + 8 * 72 * 64 * 4


def test_recorded_traffic_only_for_its_workload_and_sources(tmp_path, monkeypatch):
    fields = {}
    for line in open(bench.TRAFFIC_FILE):
        key, _, val = line.strip().partition(": ")
        fields[key] = val
    got = bench.recorded_traffic(fields["workload"])
    assert got is None or got == int(fields["traffic_bytes_per_launch"])
    for other in ("qwen3_32b_131k", "qwen3_8b_b64_prefix"):
        assert bench.recorded_traffic(other) is None
    # a figure whose recorded source hash does not match the sources is not reported
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel v1")
    good = hashlib.sha256(b"kernel v1").hexdigest()
    prof = tmp_path / "p.md"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof))
    for sha, want in ((good, 1234), ("0" * 64, None)):
        prof.write_text(f"    workload: w\n    traffic_bytes_per_launch: 1234\n"
                        f"    source_sha256: {sha}\n    sources: {os.path.basename(src)}\n")
        assert bench.recorded_traffic("w") == want
        assert bench.recorded_traffic("x") is None
