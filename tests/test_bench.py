"""Host logic of bench.py (no GPU): the attention flop count, the traffic record of the
dominant kernel, and the refusal of runs on more than one GPU."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench


def _brute_force_valid_keys(sel: np.ndarray, n: int) -> int:
    """Keys of the selected blocks at positions <= t (and < n), counted one by one."""
    total = 0
    B, H, N, K = sel.shape
    for b in range(B):
        for h in range(H):
            for t in range(N):
                for j in sel[b, h, t]:
                    if j < 0:
                        continue
                    total += sum(1 for key in range(64 * j, 64 * j + 64) if key <= t and key < n)
    return total


def test_attention_flops_counts_valid_keys():
    rng = np.random.default_rng(3)
    n, K, group, d = 300, 4, 4, 64
    sel = np.full((2, 1, n, K), -1, dtype=np.int32)
    for b in range(2):
        for t in range(n):
            valid = np.arange(t // 64 + 1)
            pick = rng.choice(valid, size=min(K, len(valid)), replace=False)
            sel[b, 0, t, :len(pick)] = np.sort(pick)
    got = bench.attention_flops(torch.from_numpy(sel), n, group, d)
    assert got == _brute_force_valid_keys(sel, n) * group * 4.0 * d


def _write_record(path, sha: str, fetch: int, write: int) -> None:
    with open(path, "w") as f:
        f.write(f"# traffic\n\nsource_sha256: {sha}\nfetch_bytes_per_call: {fetch}\nwrite_bytes_per_call: {write}\n")


def _sources_sha() -> str:
    h = hashlib.sha256()
    for name in bench.TRAFFIC_SOURCES:
        with open(os.path.join(bench.ROOT, "hierarchical_top_selection_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def test_traffic_record_needs_matching_sources(tmp_path, monkeypatch):
    rec = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    _write_record(rec, _sources_sha(), 100, 23)
    assert bench.attention_traffic("prefill_n262144") == 123
    assert bench.attention_traffic("prefill_n32768") is None          # recorded for the 256K workload only
    _write_record(rec, "0" * 64, 100, 23)
    assert bench.attention_traffic("prefill_n262144") is None         # sources changed since the counters


def test_committed_traffic_record_parses():
    """The committed record has its three fields; it counts only while its hash matches."""
    with open(bench.TRAFFIC_FILE) as f:
        text = f.read()
    for field in ("source_sha256:", "fetch_bytes_per_call:", "write_bytes_per_call:"):
        assert field in text, field
    got = bench.attention_traffic("prefill_n262144")
    assert got is None or got > 0


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(argv):
    res = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), *argv],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
