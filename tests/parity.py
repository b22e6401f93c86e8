"""Comparison rules between the HIP library and the CPU oracle (shared by GPU tests and bench).

Tolerances:
  * block probabilities: |dP| <= 1e-4 * P + 1e-7 elementwise, rows sum to 1 within 1e-5
    (fp32 pooling and fp32 matrix-core dot products against fp64);
  * masks: at least 99.9% of block pairs equal; every row that differs must still be a valid
    top-p set under the oracle's fp64 probabilities within 1e-4 of p: its mass reaches
    p - 1e-4, and dropping its smallest block leaves less than p + 1e-4 (a near-threshold
    flip or a swap of near-equal blocks);
  * attention outputs (bf16 in, fp32 accumulate, bf16 out): max |err| <= 2e-2 and
    relative L2 error <= 5e-3 against the fp64 oracle on the same mask.
"""
from __future__ import annotations

import numpy as np

ATOL_OUT = 2e-2
RTOL_L2 = 5e-3
# Row statistics (log-sum-exp, kept attention mass). The GPU sums exactly the bf16-rounded
# weights its products use: each is within 2^-9 (relative) of the exact weight, so ln l, or a
# ratio of two such sums, moves by at most 1.95e-3; the fp32 sums add at most n * 2^-24
# (relative) for n terms per lane, 2.3e-3 at N = 75,600. 5e-3 absolute covers both.
ATOL_STAT = 5e-3


def check_probs(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got - ref)
    bound = 1e-4 * ref + 1e-7
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} probs out of tolerance; worst {(err - bound).max():.3e}"
    rs = np.abs(got.sum(-1) - 1.0).max()
    assert rs <= 1e-5, rs


def check_lists(count: np.ndarray, idx: np.ndarray, m: int, mask=None):
    """Kept lists are ascending, in range, and agree with the optional uint8 mask."""
    assert count.min() >= 1 and count.max() <= m
    rows = count.reshape(-1)
    lists = idx.reshape(-1, idx.shape[-1])
    for r in range(rows.shape[0]):
        js = lists[r, : rows[r]]
        assert js.min() >= 0 and js.max() < m
        assert np.all(np.diff(js) > 0), "kept indices must be strictly ascending"
    if mask is not None:
        assert np.array_equal(mask.sum(-1), count)


def check_mask(gpu_mask: np.ndarray, ref_probs: np.ndarray, ref_mask: np.ndarray, top_p):
    """The mask agreement rule; returns the fraction of equal block pairs."""
    agree = float(np.mean(gpu_mask == ref_mask))
    assert agree >= 0.999, f"mask agreement {agree:.5f} < 0.999"
    H = ref_probs.shape[1]
    p = np.broadcast_to(np.asarray(top_p, dtype=np.float64), (H,))
    diff_rows = np.argwhere((gpu_mask != ref_mask).any(-1))
    for b, h, i in diff_rows:
        row = ref_probs[b, h, i]
        kept = gpu_mask[b, h, i]
        mass = row[kept].sum()
        if p[h] >= 1.0:
            raise AssertionError("p >= 1 must keep every block")
        assert mass >= p[h] - 1e-4, (b, h, i, mass, p[h])
        assert mass - row[kept].min() < p[h] + 1e-4, (b, h, i, mass, p[h])
    return agree


def check_out(got: np.ndarray, ref: np.ndarray, what: str = "output"):
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert err <= ATOL_OUT and rel <= RTOL_L2, f"{what}: max|err| {err:.3e}, rel-L2 {rel:.3e}"
    return err, rel


def check_row_stat(got: np.ndarray, ref: np.ndarray, what: str):
    """Per-token row statistic: compared where the oracle computed it (not NaN); -inf (an
    empty kept set) must match exactly."""
    got = np.asarray(got, dtype=np.float64)
    sel = ~np.isnan(ref)
    assert sel.any(), what
    g, r = got[sel], ref[sel]
    inf = np.isinf(r)
    assert np.array_equal(np.isinf(g), inf) and np.all(g[inf] == r[inf]), f"{what}: infinities"
    err = np.abs(g[~inf] - r[~inf]).max() if (~inf).any() else 0.0
    assert err <= ATOL_STAT, f"{what}: max |err| {err:.3e} > {ATOL_STAT}"
