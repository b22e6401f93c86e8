"""CPU checks of bench.py's bookkeeping: the algorithmic work it divides by time, the source
hash that keys the committed counter figures, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import synth
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lists(B, H, M, seed):
    g = np.random.default_rng(seed)
    cnt = np.zeros((B, H, M), np.int32)
    idx = np.zeros((B, H, M, M), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(M):
                js = np.sort(g.choice(M, size=int(g.integers(0, M + 1)), replace=False))
                cnt[b, h, i] = len(js)
                idx[b, h, i, :len(js)] = js
                idx[b, h, i, len(js):] = g.integers(-5, M + 5, size=M - len(js))  # unused entries
    return cnt, idx


@pytest.mark.parametrize("N,block", [(64 * 7 + 13, 64), (128 * 3, 128), (37, 64)])
def test_kept_token_pairs_counts_attended_pairs(N, block):
    """sum over kept (i, j) of n_i n_j equals the number of (query, key) token pairs that
    masked attention attends, counted token by token from the oracle's block partition."""
    M = -(-N // block)
    cnt, idx = _lists(2, 3, M, N + block)
    got = bench.kept_token_pairs(torch.from_numpy(cnt), torch.from_numpy(idx), N, block)
    mask = O.mask_from_lists(cnt, idx, M)
    starts, ends = O.block_partition(N, block)
    tok_block = np.repeat(np.arange(M), np.asarray(ends) - np.asarray(starts))
    want = 0
    for b in range(2):
        for h in range(3):
            tm = mask[b, h][tok_block][:, tok_block]  # [N, N] token-level mask
            want += int(tm.sum())
    assert got == want


def test_kept_token_pairs_all_kept_is_dense():
    N, block = 1000, 64
    M = -(-N // block)
    cnt = torch.full((1, 2, M), M, dtype=torch.int32)
    idx = torch.arange(M, dtype=torch.int32).expand(1, 2, M, M).contiguous()
    assert bench.kept_token_pairs(cnt, idx, N, block) == 2 * N * N


def test_src_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f(int x) { // one\n  return x + 1; /* two */ }\n")
    h1 = bench.src_hash([str(a)])
    a.write_text("int f(int x) {   // changed comment\n\n  return x + 1; /* other */ }\n")
    assert bench.src_hash([str(a)]) == h1
    a.write_text("int f(int x) { return x + 2; }\n")
    assert bench.src_hash([str(a)]) != h1


def test_measured_traffic_needs_matching_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel body\n")
    monkeypatch.setitem(bench.KERNEL_SOURCES, "t", [str(src)])
    table = {"x": {"source": "t", "source_sha": bench.src_hash([str(src)]), "workload": "w1",
                   "bytes_per_launch": 123.0}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(table))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("x", "w1") == 123.0
    assert bench.measured_traffic("x", "w2") is None  # counters taken on another workload
    assert bench.measured_traffic("missing", "w1") is None
    src.write_text("kernel body changed\n")
    assert bench.measured_traffic("x", "w1") is None


def test_committed_traffic_table_names_known_sources():
    table = json.load(open(bench.TRAFFIC_FILE))
    for key, ent in table.items():
        if isinstance(ent, dict):
            assert ent["source"] in bench.KERNEL_SOURCES, key
            assert ent["workload"] in synth.WORKLOADS, key
            assert ent["bytes_per_launch"] > 0, key


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
