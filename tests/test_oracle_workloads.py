"""The oracle on the synthetic workloads: sparsity bands and the block-size trend the pages
report (larger blocks reduce achievable sparsity: CalibAtt page, Fig. S14 and Table S6)."""
import numpy as np
import pytest

import synth
from oracle import oracle as O


def _mask_stats(cfg, p, seq=None):
    q, k, _ = synth.make_qkv(cfg, seq=seq)
    qd, kd = synth.to_f64(q), synth.to_f64(k)
    probs = O.block_scores(qd, kd, cfg.block, cfg.head_dim ** -0.5)
    sel = O.topp_select(probs, p)
    return probs, sel


def test_tiny_sparsity_band_and_kept_mass():
    cfg = synth.WORKLOADS["tiny"]
    probs, sel = _mask_stats(cfg, 0.9)
    sp = O.block_sparsity(sel["count"], cfg.num_blocks)
    assert 0.80 < sp < 0.97, sp
    assert np.all(sel["mass"] >= 0.9)


def test_larger_blocks_reduce_sparsity():
    cfg64 = synth.workload("wan13b_480p", heads=1, grid=(6, 30, 52))
    cfg128 = synth.workload("wan13b_480p", heads=1, grid=(6, 30, 52), block=128)
    _, s64 = _mask_stats(cfg64, 0.9)
    _, s128 = _mask_stats(cfg128, 0.9)
    sp64 = O.block_sparsity(s64["count"], cfg64.num_blocks)
    sp128 = O.block_sparsity(s128["count"], cfg128.num_blocks)
    assert sp128 < sp64, (sp64, sp128)


@pytest.mark.slow
def test_wan13b_head0_sparsity_near_page_level():
    cfg = synth.workload("wan13b_480p", heads=1)
    _, sel = _mask_stats(cfg, 0.9)
    sp = O.block_sparsity(sel["count"], cfg.num_blocks)
    assert 0.85 < sp < 0.96, sp
