"""The seeded input generator: determinism, streaming by head, feature scale, page shapes."""
import json
import os

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_workloads.json")


def test_deterministic_and_streamable_by_head():
    cfg = synth.workload("tiny", grid=(2, 8, 8))
    q1, k1, v1 = synth.make_qkv(cfg)
    q2, k2, v2 = synth.make_qkv(cfg)
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    one = synth.workload("tiny", grid=(2, 8, 8), heads=1)
    q3, _, _ = synth.make_qkv(one)
    assert torch.equal(q3[0, 0], q1[0, 0])
    assert not torch.equal(q1[0, 0], q1[0, 1])
    assert q1.dtype == torch.bfloat16 and q1.shape == (1, 2, 128, 64)


def test_features_unit_rms_and_ragged_prefix():
    phi = synth.positional_features((3, 5, 7)).double()
    assert phi.shape == (105, 64)
    assert torch.allclose((phi ** 2).mean(dim=1), torch.ones(105, dtype=torch.float64), atol=1e-6)
    cfg = synth.workload("tiny", grid=(2, 8, 8))
    q_full, _, _ = synth.make_qkv(cfg)
    q_short, _, _ = synth.make_qkv(cfg, seq=100)
    assert q_short.shape[2] == 100
    assert not torch.equal(q_short[0, 0, :10], q_full[0, 0, 10:20])


def test_workload_shapes_match_pages():
    g = json.load(open(GOLDEN))
    w480 = synth.WORKLOADS["wan14b_480p"]
    assert w480.seq == g["wan14b_480p_seq"]["seq"] == g["wan14b_480p_attention_call"]["seq"]
    assert (w480.batch, w480.heads, w480.head_dim) == (1, 40, 128)
    assert 2 * w480.grid[1] * w480.grid[2] == g["tokens_in_two_480p_frames"]["tokens"]
    assert synth.WORKLOADS["wan14b_720p"].seq == g["wan14b_720p_seq"]["seq"]
    assert synth.WORKLOADS["wan13b_480p"].seq == 32760
    assert synth.WORKLOADS["hunyuan_720p"].seq == 118800
    assert synth.WORKLOADS["wan14b_720p"].num_blocks == 1182
    assert synth.WORKLOADS["hunyuan_720p"].num_blocks == 929


def test_head_params():
    p, c = synth.head_params(synth.WORKLOADS["wan14b_480p"])
    assert p.shape == (40,) and np.all(p >= 0.8) and np.all(p <= 0.97 + 1e-6)
    assert np.all(c >= 0) and np.all(c < 1) and len(set(c.tolist())) == 40
    p, c = synth.head_params(synth.WORKLOADS["wan13b_480p"])
    assert np.all(p == np.float32(0.9)) and np.all(c == 0)


def test_drift_is_small_and_seeded():
    cfg = synth.workload("tiny", grid=(2, 8, 8))
    q, _, _ = synth.make_qkv(cfg)
    q1 = synth.drifted(q, "q", 1)
    q1b = synth.drifted(q, "q", 1)
    assert torch.equal(q1, q1b)
    d = (q1.float() - q.float()).std().item()
    assert 0.03 < d < 0.07


def test_drift_series_matches_single_steps():
    cfg = synth.workload("tiny", grid=(1, 8, 8))
    q, _, _ = synth.make_qkv(cfg)
    series = synth.drift_series(q, "q", 3)
    for s in range(1, 4):
        assert torch.equal(series[s - 1], synth.drifted(q, "q", s))
