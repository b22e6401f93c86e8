"""The refresh identity on the GPU path alone (RECAP Sec. 3.2: the error d_h - d_t of the cached
refinement vanishes at the refresh step t = h). The sparse call on the refresh's own inputs and
kept lists, with the residual R that the dense pass captured added at scale 1, must reproduce
the dense output of that pass, up to the bf16 rounding of R and of the two outputs:

    out = bf16(O_s + bf16(O_d - O_s'))   against   od = bf16(O_d)

O_s' is the capture pass's kept-block accumulator (under the dense running max) and O_s the
sparse call's own result (under its own max). Each rounds its weights to bf16 on its own, and
each is within 2^-8 / (1 - 2^-8) * max_u |v_u - o| of the exact kept attention (a convex
combination whose weights each move by a factor within 1 +- 2^-8). So per element

    |out - od| <= 2^-8 |R| + 2^-8 (|out| + |od|) + 2 * 1.004 * 2^-8 * (max|V_h| + |od|) + 1e-5,

the last terms bounding |O_s - O_s'| (max|v_u - o| <= max|V_h| + |o|, h the head; 1e-5 for the
fp32 sums). That bound is the worst case of two independent roundings; the typical difference
is far smaller, so the test also holds the root-mean-square of the part of |out - od| above
2^-8 |R| + 2^-8 (|out| + |od|) to 1e-3. A key block missing from either side moves whole rows
by its share of the mass (the paired-block walk of the sparse kernel, or the capture pass's
kept-bit mapping attending other keys than the lists name).
"""
import numpy as np
import pytest
import torch

import synth

from gpu_common import DEV, bsa, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu

U = 2.0 ** -8


def _identity(bsa, qd, kd, vd, desc, p, s):
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, _, _ = bsa.recap_topp_mask(desc, probs, p)
    od, rcap = bsa.recap_dense_attn(desc, qd, kd, vd, s, count, idx, capture=True)
    H = desc.heads
    out = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, s, residual=rcap,
                                      res_scale=[1.0] * H)
    torch.cuda.synchronize()
    return od, rcap, out, count


def _check(od, rcap, out, vd, what):
    od, r, o = od.float(), rcap.float(), out.float()
    diff = (o - od).abs()
    tight = U * r.abs() + U * (o.abs() + od.abs())
    vmax = vd.float().abs().amax(dim=(0, 2, 3), keepdim=True)  # per head
    loose = tight + 2.0 * 1.004 * U * (vmax + od.abs()) + 1e-5
    excess = (diff - tight).clamp(min=0)
    rms = excess.square().mean().sqrt().item()
    say(f"[{what}] max|out-od| {diff.max().item():.3e}; above 2^-8|R| + 2^-8(|out|+|od|): "
        f"{(excess > 0).float().mean().item():.2e} of {diff.numel()} elements, max "
        f"{excess.max().item():.3e}, rms {rms:.3e}; worst margin to the full bound "
        f"{(diff - loose).max().item():.3e}")
    assert torch.isfinite(o).all()
    assert bool((diff <= loose).all()), (what, (diff - loose).max().item())
    assert rms <= 1e-3, (what, rms)


CASES = {
    "b64_odd_m_d128": dict(heads=2, head_dim=128, block=64, seq=64 * 37 + 11, p=[0.9, 0.7]),
    "b64_d64_two_batches": dict(batch=2, heads=3, head_dim=64, block=64, seq=64 * 20 + 1,
                                p=[0.95, 0.8, 0.5]),
    "b128_d128": dict(heads=2, head_dim=128, block=128, seq=128 * 13 + 77, p=[0.9, 0.97]),
    "b128_d64": dict(heads=1, head_dim=64, block=128, seq=128 * 9, p=[0.6]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_refresh_identity_small(bsa, case):
    kw = dict(CASES[case])
    p = kw.pop("p")
    seq = kw.pop("seq")
    cfg = synth.workload("tiny", grid=(1, 1, seq), **kw)
    say(f"[case] {case}: B={cfg.batch} H={cfg.heads} D={cfg.head_dim} N={seq} "
        f"block={cfg.block} p={p}")
    q, k, v = synth.make_qkv(cfg)
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    desc = bsa.make_desc(qd, cfg.block)
    od, rcap, out, count = _identity(bsa, qd, kd, vd, desc, p, cfg.head_dim ** -0.5)
    assert int(count.min()) < cfg.num_blocks  # a real sparse set somewhere
    _check(od, rcap, out, vd, case)


def test_refresh_identity_720p(bsa):
    """Every element of every head at the Wan2.1-14B-like 720p refresh (B=1, H=40, D=128,
    N=75,600, block 64, p = 0.95), in the launch configuration the benchmark times."""
    cfg = synth.WORKLOADS["wan14b_720p"]
    say("[case] refresh identity, wan14b_720p: generating inputs")
    q, k, v = synth.make_qkv(cfg)
    p, _ = synth.head_params(cfg)
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    desc = bsa.make_desc(qd, cfg.block)
    od, rcap, out, _ = _identity(bsa, qd, kd, vd, desc, p.tolist(), cfg.head_dim ** -0.5)
    _check(od, rcap, out, vd, "wan14b_720p")
