"""Host logic of bench.py (no GPU): the attention flop count, the per-kernel traffic records,
the byte floors, and the refusal of runs on more than one GPU."""
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


def test_kernel_traffic_needs_matching_sources(tmp_path, monkeypatch):
    """A kernel's counter traffic counts only while the sha256 of its sources matches the record."""
    rec = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    rec.write_text("# traffic\n\n"
                   f"traffic: route_kernel fetch=100 write=23 sha256={bench.source_sha256('route_kernel')}\n"
                   f"traffic: topk_kernel fetch=5 write=6 sha256={'0' * 64}\n"
                   f"traffic: no_such_kernel fetch=5 write=6 sha256={'0' * 64}\n")
    assert bench.kernel_traffic("prefill_n262144") == {"route_kernel": 123}
    assert bench.kernel_traffic("prefill_n32768") == {}                  # recorded for the 256K workload only


def test_committed_traffic_record_parses():
    """Every line of the committed record names a known kernel; entries count only while current."""
    if not os.path.exists(bench.TRAFFIC_FILE):
        pytest.skip("no traffic record committed for the current kernels")
    with open(bench.TRAFFIC_FILE) as f:
        lines = [x for x in f.read().splitlines() if x.startswith("traffic: ")]
    assert lines
    for x in lines:
        assert x.split()[1] in bench.KERNEL_SOURCES, x
    assert all(v > 0 for v in bench.kernel_traffic("prefill_n262144").values())


def test_decode_step_bytes_hand_derived():
    """Decode byte floor at the first step of the 131072-token workload (n = 131073 keys, 13 levels
    2049, 1025, 513, 257, 129, 65, 33, 17, 9, 5, 3, 2, 1), derived by hand: candidates from the root
    1, 2, 3, 5, 9, then 17 at level 8 (scored: 33 children summaries read) and 32 at levels 7..2
    (scored: 64 children each), 32 candidate leaves at the leaf level.  Per (b, kvh) unit:
    summaries (33 + 6 * 64) * 512 B = 213504, leaf keys 32 * 64 * 256 = 524288, selected values
    16 * 64 * 256 = 262144, query and output rows 2 * 4 * 256 = 2048, new key and value read and
    written 1024, the leaf's keys 16384 and the ancestor path read and written 2 * 13 * 512 = 13312:
    1032704 bytes in all, times 64 * 8 units."""
    from hierarchical_top_selection_amd import workloads as W

    w = W.WORKLOADS["decode_b64_ctx131072"]
    assert bench.level_sizes(131073) == [2049, 1025, 513, 257, 129, 65, 33, 17, 9, 5, 3, 2, 1]
    per_unit = 213504 + 524288 + 262144 + 2048 + 1024 + 16384 + 13312
    assert bench.decode_step_bytes(w, 131072) == per_unit * 64 * 8


def test_compulsory_bytes_of_the_256k_selection():
    """Compulsory HBM bytes of the 256K workload's kernels (B = 1, N = 262144, 16 query heads on one
    KV head, d = 128, K = 16, bf16), written out: Q 1 GiB (262144 * 16 * 128 * 2), its packed copy
    as much, the 2K = 32 candidate slots 32 MiB per int32 or float32 array, K 64 MiB, packed K 64 MiB."""
    from hierarchical_top_selection_amd import workloads as W

    b = bench.compulsory_bytes(W.WORKLOADS["prefill_n262144"])
    gib, mib = 1 << 30, 1 << 20
    assert b["route_kernel"] == gib + gib + 32 * mib
    assert b["leaf_lse_kernel"] == gib + 64 * mib + 2 * 32 * mib
    assert b["topk_kernel"] == 2 * 32 * mib + 16 * mib
    assert b["pack_blocks_kernel"] == 64 * mib + 64 * mib
    assert b["pyramid_leaves_kernel"] == 64 * mib + (4096 + 2048 + 1024 + 512) * 512
    assert b["cluster_kernel"] == 2 * 32 * mib + 256 * 4097 * 4


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"]])
def test_more_than_one_gpu_is_refused(argv):
    res = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), *argv],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
