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
U_BF16 = 2.0 ** -8   # unit roundoff of bf16 round-to-nearest (8-bit significand)
U_F32 = 2.0 ** -24
# Row statistics (log-sum-exp, kept attention mass). The GPU sums exactly the bf16-rounded
# weights its products use: each is within U_BF16 (relative) of the exact weight, so ln l moves
# by at most ln(1 + 2^-8) = 3.90e-3, and a kept share m = l_kept / l_all (the two sums share the
# kept terms) by at most 2 * 2^-8 * m * (1 - m) <= 1.95e-3; the fp32 sums add at most
# (N / 2) * 2^-24 (relative; each lane sums half of every key tile), 2.25e-3 at N = 75,600.
# 7e-3 absolute covers the worst case of both.
ATOL_STAT = 7e-3


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


def check_captured(ref_sparse: np.ndarray, residual: np.ndarray, ref_dense: np.ndarray,
                   what: str = "sparse + captured residual"):
    """The captured residual R = bf16(O_dense - O_sparse) is the difference of two GPU
    attention outputs, each held to ATOL_OUT / RTOL_L2 against the oracle, rounded once more to
    bf16. So ref_sparse + R must lie within the sum of the two outputs' bounds plus R's own
    rounding (U_BF16 relative) of ref_dense: per element 2 ATOL_OUT + U_BF16 |R|, and in
    relative L2 2 RTOL_L2 + U_BF16 |R| / |ref_dense|."""
    got = ref_sparse + residual
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref_dense)
    bound = 2 * ATOL_OUT + U_BF16 * np.abs(residual)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bound; worst excess " \
                          f"{(err - bound).max():.3e} (max|err| {err.max():.3e})"
    nref = max(np.linalg.norm(ref_dense), 1e-30)
    rel = np.linalg.norm(got - ref_dense) / nref
    lim = 2 * RTOL_L2 + U_BF16 * np.linalg.norm(residual) / nref
    assert rel <= lim, f"{what}: rel-L2 {rel:.3e} > {lim:.3e}"
    return float(err.max()), rel


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


def score_rounding_bound(q: np.ndarray, kbar: np.ndarray, sm_scale: float) -> float:
    """Largest change of sm_scale * q_t . K̄_j over all (t, j) when each block-mean element is
    held as a bf16 pair hi + lo (hi = bf16(x), lo = bf16(x - hi): within U_BF16^2 relative of
    the fp32 mean, plus the fp32 mean's own rounding): sm_scale * (U_BF16^2 + U_F32) *
    sum_d |q_td| |K̄_jd|."""
    worst = 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            worst = max(worst, float((np.abs(q[b, h]) @ np.abs(kbar[b, h]).T).max()))
    return float(sm_scale) * (U_BF16 ** 2 + U_F32) * worst


def coarse_lse_atol(q, kbar, sm_scale) -> float:
    """Coarse-tail log-mass: the rounded block means move each pooled score by at most the
    rounding bound (hence ln of the summed masses by at most that), plus the row-statistics
    bound for the bf16 weights and fp32 sums."""
    return ATOL_STAT + score_rounding_bound(q, kbar, sm_scale)


def variance_lse_atol(q, var, sm_scale) -> float:
    """Moment-refined coarse log-mass: the second-order term (s^2 / 2) sum_d q_d^2 Var_jd is
    formed on the GPU as a bf16 product of bf16(q^2) and bf16((s / 2) Var) with fp32 sums, so
    each factor carries a relative error of at most U_BF16 and every block's term at most
    (2 U_BF16 + U_BF16^2) of itself (plus fp32 sums); ln of the summed masses moves by at most
    the largest such change. Returns that bound over all (t, j)."""
    worst = 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            worst = max(worst, float(((q[b, h] * q[b, h]) @ var[b, h].T).max()))
    return 0.5 * float(sm_scale) ** 2 * (2 * U_BF16 + U_BF16 ** 2 + 64 * U_F32) * worst


def check_rows_within(got: np.ndarray, ref: np.ndarray, atol, what: str):
    """Per-token values (finite reference) within a per-row or scalar bound."""
    got = np.asarray(got, dtype=np.float64)
    sel = np.isfinite(ref)
    atol = np.broadcast_to(np.asarray(atol, dtype=np.float64), ref.shape)
    err = np.abs(got[sel] - ref[sel])
    bad = err > atol[sel]
    assert not bad.any(), f"{what}: {bad.sum()} rows out of bound; worst excess " \
                          f"{(err - atol[sel]).max():.3e}"
    return float(err.max()) if err.size else 0.0


def check_merged(got, ref, w, spread, lse_tol, extra: int, what: str):
    """A log-mass merge out = bf16(w O_s + (1 - w) o_T) of attention-like parts, against the
    oracle's merge. Per row: ATOL_OUT for the convex combination of parts that each meet the
    attention-output rule, plus the final bf16 rounding of the merged value (U_BF16 |out|; the
    parts are fp32), plus ATOL_OUT * (1 - w) for each of `extra` further tail terms whose errors
    do not cancel (a coarse tail taken at another step than the one it is combined with), plus
    the weight error: w (1 - w) * (log-mass error lse_tol) * max_d |O_s - o_T| (`spread`).
    Relative L2 error within RTOL_L2. got, ref: [B,H,N,D]; w, spread: [B,H,N] from the oracle."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    bound = ATOL_OUT * (1.0 + extra * (1.0 - w)) + w * (1.0 - w) * lse_tol * spread \
        + U_BF16 * np.abs(ref).max(axis=-1)
    err = np.abs(got - ref).max(axis=-1)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} rows out of bound; worst excess " \
                          f"{(err - bound).max():.3e}"
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= RTOL_L2, f"{what}: rel-L2 {rel:.3e}"
    return float(err.max()), rel


# ---- FP8 (MXFP8) products -------------------------------------------------------------------
U_E4M3 = 2.0 ** -4  # unit roundoff of E4M3 round-to-nearest (4-bit significand)


def fp8_weight_bounds(q, k, v, mask, block: int, sm_scale: float, out_ref, rows=None):
    """Error bounds of attention whose weights are rounded to E4M3 (relative error <= u each,
    unbiased, variance <= u^2 / 3), on inputs already quantised (q, k, v dequantised):
      per element: |dO_d| <= u / (1 - u) * max_j |v_jd - o_d| over the attended keys j (the
      output stays a convex combination of the attended values with each weight moved by a
      factor in [1 - u, 1 + u]), plus 1e-3 of that spread for weights in E4M3's subnormal range
      (below 2^-13 of their 32-key block's largest);
      expected squared error: (u^2 / 3) * sum_j w_j^2 (v_jd - o_d)^2 (first order, independent
      roundings). rows: optional (b, h, i) query blocks (default all). Returns (per-element
      bound [B,H,N,D], zero outside rows; total expected squared error over rows)."""
    B, H, N, D = q.shape
    bound = np.zeros((B, H, N, D))
    exp_sq = 0.0
    nblk = -(-N // block)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(nblk)]
    for b, h, i in rows:
        lo, hi = i * block, min(N, (i + 1) * block)
        js = np.nonzero(mask[b, h, i])[0]
        toks = np.concatenate([np.arange(j * block, min(N, (j + 1) * block)) for j in js])
        vv = v[b, h, toks]
        o = out_ref[b, h, lo:hi]
        spread = np.maximum(vv.max(0)[None, :] - o, o - vv.min(0)[None, :])
        bound[b, h, lo:hi] = (U_E4M3 / (1 - U_E4M3) + 1e-3) * spread
        sc = sm_scale * q[b, h, lo:hi] @ k[b, h, toks].T
        w = np.exp(sc - sc.max(-1, keepdims=True))
        w /= w.sum(-1, keepdims=True)
        w2 = w * w
        var = w2 @ (vv * vv) - 2 * o * (w2 @ vv) + o * o * w2.sum(-1, keepdims=True)
        exp_sq += float(np.maximum(var, 0).sum()) * U_E4M3 ** 2 / 3
    return bound, exp_sq


def check_fp8_out(got, ref, bound, exp_sq, what: str):
    """FP8 attention output against the oracle on the quantised inputs: every element within
    ATOL_OUT (bf16 output rounding and fp32 sums, as for the bf16 path) plus its weight-rounding
    bound; relative L2 error within RTOL_L2 plus three times the expected relative error of the
    weight rounding."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    err = np.abs(got - ref)
    bad = err > ATOL_OUT + bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bound; worst excess " \
                          f"{(err - ATOL_OUT - bound).max():.3e}"
    nref = max(np.linalg.norm(ref), 1e-30)
    rel = np.linalg.norm(got - ref) / nref
    lim = RTOL_L2 + 3 * np.sqrt(exp_sq) / nref
    assert rel <= lim, f"{what}: rel-L2 {rel:.3e} > {lim:.3e}"
    return float(err.max()), rel, lim
