"""Checks that pin the CPU oracle to facts outside itself.

Each `check_*` function raises AssertionError when the oracle (the module `oracle.oracle`,
looked up at call time so that a test can plant a mistake in it) disagrees with a closed form,
an invariant, a library routine or the scalar brute force. `test_oracle_pins.py` runs every
check on the real oracle; `test_oracle_mutants.py` plants plausible mistakes in the oracle and
requires that at least one check fails for each.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import brute
from oracle import oracle as O


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).normal(0.0, scale, size=shape)


# ----------------------------------------------------------------------------- pooling
def check_pool_block_constant():
    """A block-constant input pools to that constant, including the short last block."""
    n, b, d = 200, 64, 3  # blocks of 64, 64, 64, 8
    x = np.zeros((1, 1, n, d))
    vals = [1.5, -2.25, 7.0, 0.125]
    for j, v in enumerate(vals):
        x[0, 0, j * b:(j + 1) * b, :] = v
    pooled = O.block_mean_pool(x, b)
    assert pooled.shape == (1, 1, 4, d)
    assert np.array_equal(pooled[0, 0, :, 0], np.array(vals)), pooled[0, 0, :, 0]


def check_pool_closed_form_ragged():
    """X_t[d] = t + 10 d: block mean over [s, e) is (s + e - 1)/2 + 10 d (arithmetic series)."""
    n, b, d = 150, 32, 4  # last block has 22 tokens
    t = np.arange(n, dtype=np.float64)[:, None]
    x = (t + 10.0 * np.arange(d)[None, :])[None, None]
    pooled = O.block_mean_pool(x, b)[0, 0]
    for j in range(pooled.shape[0]):
        s, e = j * b, min(n, (j + 1) * b)
        want = (s + e - 1) / 2.0 + 10.0 * np.arange(d)
        assert np.allclose(pooled[j], want, rtol=0, atol=1e-12), (j, pooled[j], want)


def check_pool_mass_invariant():
    """sum_j n_j * X̄_j equals sum_t X_t (pooling preserves the total)."""
    n, b = 333, 64
    x = _rand((2, 3, n, 5), 7)
    pooled = O.block_mean_pool(x, b)
    s, e = O.block_partition(n, b)
    nj = (e - s).astype(np.float64)
    lhs = np.einsum("bhjd,j->bhd", pooled, nj)
    assert np.allclose(lhs, x.sum(axis=2), rtol=1e-12, atol=1e-10)


# ----------------------------------------------------------------------------- scores
def _two_block_case(a0, a1, x0, x1, b=8):
    """D = 1; query blocks are constant a0, a1; key blocks are constant x0, x1."""
    q = np.zeros((1, 1, 2 * b, 1))
    k = np.zeros((1, 1, 2 * b, 1))
    q[0, 0, :b, 0], q[0, 0, b:, 0] = a0, a1
    k[0, 0, :b, 0], k[0, 0, b:, 0] = x0, x1
    return q, k


def check_scores_closed_form():
    """Two blocks: P̄[i,0] = 1 / (1 + exp(s * a_i * (x1 - x0))) (logistic of the logit gap)."""
    a0, a1, x0, x1, s = 0.7, -1.9, 0.4, 2.3, 0.5
    q, k = _two_block_case(a0, a1, x0, x1)
    p = O.block_scores(q, k, 8, s)[0, 0]
    for i, a in enumerate((a0, a1)):
        p0 = 1.0 / (1.0 + math.exp(s * a * (x1 - x0)))
        assert abs(p[i, 0] - p0) < 1e-14 and abs(p[i, 1] - (1.0 - p0)) < 1e-14, (i, p[i], p0)


def check_scores_rows_and_degenerate():
    """Rows sum to 1; a single block gives 1; identical key blocks give uniform 1/M."""
    q = _rand((1, 2, 300, 16), 3)
    k = _rand((1, 2, 300, 16), 4)
    p = O.block_scores(q, k, 64, 0.25)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-14)
    one = O.block_scores(q[:, :, :40], k[:, :, :40], 64, 0.25)
    assert one.shape == (1, 2, 1, 1) and np.all(one == 1.0)
    kc = np.tile(_rand((1, 2, 64, 16), 5), (1, 1, 5, 1))  # every key block is the same block
    pu = O.block_scores(q[:, :, :320], kc, 64, 0.25)
    assert np.allclose(pu, 0.2, atol=1e-15)


def check_scores_scale_and_shift():
    """softmax(2L) = P^2 / sum P^2 (the scale multiplies the logits); adding one vector to
    every key leaves each row unchanged (a per-row constant logit shift)."""
    q = _rand((1, 1, 256, 8), 11)
    k = _rand((1, 1, 256, 8), 12)
    p1 = O.block_scores(q, k, 32, 0.3)
    p2 = O.block_scores(q, k, 32, 0.6)
    sq = p1 ** 2
    assert np.allclose(p2, sq / sq.sum(-1, keepdims=True), rtol=1e-12, atol=1e-15)
    shift = _rand((1, 1, 1, 8), 13) * 3.0
    p3 = O.block_scores(q, k + shift, 32, 0.3)
    assert np.allclose(p3, p1, rtol=1e-11, atol=1e-15)
    p0 = O.block_scores(q, k, 32, 0.0)
    assert np.allclose(p0, 1.0 / 8.0, atol=1e-15)


def check_scores_vs_brute():
    """Vectorised scores equal the scalar loop spelling on a tiny ragged input."""
    n, b, d, s = 45, 8, 5, 0.37
    q = _rand((1, 1, n, d), 21)
    k = _rand((1, 1, n, d), 22)
    got = O.block_scores(q, k, b, s)[0, 0]
    want = np.array(brute.scores(q[0, 0].tolist(), k[0, 0].tolist(), n, b, d, s))
    assert np.allclose(got, want, rtol=0, atol=1e-13), np.abs(got - want).max()


# ----------------------------------------------------------------------------- top-p
def check_topp_inclusive_dyadic():
    """Dyadic probabilities: p = 0.75 is reached exactly by {0, 1}; the crossing block is kept."""
    probs = np.array([0.5, 0.25, 0.125, 0.125])[None, None, None, :]
    probs = np.repeat(probs, 4, axis=2)
    r = O.topp_select(probs, 0.75)
    assert np.all(r["count"] == 2) and np.all(r["mask"][0, 0, :, :2]) and not r["mask"][..., 2:].any()
    assert np.all(r["mass"] == 0.75)
    r = O.topp_select(probs, 0.7500001)
    assert np.all(r["count"] == 3)


def check_topp_ties_lower_index():
    """Equal probabilities are taken in ascending key-block order; p = 0 keeps the argmax."""
    probs = np.full((1, 1, 1, 4), 0.25)
    r = O.topp_select(probs, 0.5)
    assert r["mask"][0, 0, 0].tolist() == [True, True, False, False]
    probs2 = np.array([0.1, 0.4, 0.1, 0.4])[None, None, None, :]
    r = O.topp_select(probs2, 0.0)
    assert r["mask"][0, 0, 0].tolist() == [False, True, False, False]
    r = O.topp_select(probs2, 0.45)
    assert r["mask"][0, 0, 0].tolist() == [False, True, False, True]
    r = O.topp_select(probs2, 0.85)
    assert r["mask"][0, 0, 0].tolist() == [True, True, False, True]


def _random_prob_rows(m, rows, seed, temp=1.5):
    g = np.random.default_rng(seed)
    logits = g.normal(0.0, temp, size=(1, 1, rows, m))
    return O.softmax_rows(logits)


def check_topp_invariants():
    """Kept mass >= p; dropping the smallest kept block falls below p (minimality); sets nest
    in p; p >= 1 keeps every block; p = 0 keeps exactly one block."""
    probs = _random_prob_rows(37, 50, 31)
    prev = None
    for p in (0.0, 0.3, 0.6, 0.9, 0.97, 1.0):
        r = O.topp_select(probs, p)
        mask = r["mask"]
        mass = (probs * mask).sum(-1)
        assert np.all(mass >= p - 1e-12)
        assert np.allclose(mass, r["mass"], atol=1e-12)
        assert np.array_equal(mask.sum(-1), r["count"])
        if p < 1.0:
            smallest = np.where(mask, probs, np.inf).min(-1)
            assert np.all((r["count"] == 1) | (mass - smallest < p)), p
        if prev is not None:
            assert np.all(~prev | mask), "kept sets must grow with p"
        prev = mask
    assert np.all(O.topp_select(probs, 1.0)["count"] == 37)
    assert np.all(O.topp_select(probs, 0.0)["count"] == 1)
    am = O.topp_select(probs, 0.0)["mask"].argmax(-1)
    assert np.array_equal(am, probs.argmax(-1))


def check_topp_vs_subset_search():
    """For M <= 9: k* is the fewest blocks of any subset reaching p, and the kept set has the
    largest mass among subsets of that size (exhaustive enumeration, no sorting)."""
    probs = _random_prob_rows(9, 12, 41, temp=1.0)
    for p in (0.35, 0.8, 0.95):
        r = O.topp_select(probs, p)
        for i in range(probs.shape[2]):
            row = probs[0, 0, i].tolist()
            kstar, best = brute.min_cardinality_subsets(row, p)
            assert r["count"][0, 0, i] == kstar, (p, i, r["count"][0, 0, i], kstar)
            assert abs(r["mass"][0, 0, i] - best) < 1e-12


def check_topp_per_head_threshold():
    """Thresholds apply per head: head h uses p[h]."""
    probs = np.repeat(_random_prob_rows(20, 6, 51), 2, axis=1)
    r = O.topp_select(probs, np.array([0.0, 1.0]))
    assert np.all(r["count"][:, 0] == 1) and np.all(r["count"][:, 1] == 20)


# ----------------------------------------------------------------------------- attention
def _sdpa64(q, k, v, scale, mask=None):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a)) for a in (q, k, v))
    am = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    return o.numpy()


def _token_mask(block_mask, n, b):
    tb = np.arange(n) // b
    return block_mask[:, :, tb][:, :, :, tb]


def check_dense_vs_sdpa():
    """All blocks kept == dense == torch SDPA in float64 (library routine)."""
    n, b, d, s = 150, 32, 16, 0.2
    q, k, v = (_rand((2, 2, n, d), 60 + i) for i in range(3))
    m = -(-n // b)
    dense = O.dense_attention(q, k, v, s, block=b)
    allkept = O.masked_attention(q, k, v, b, s, np.ones((2, 2, m, m), bool))
    ref = _sdpa64(q, k, v, s)
    assert np.allclose(dense, ref, rtol=0, atol=1e-12), np.abs(dense - ref).max()
    assert np.array_equal(dense, allkept)


def check_masked_vs_sdpa():
    """Block mask expanded to tokens == torch SDPA with that boolean mask (float64)."""
    n, b, d, s = 173, 32, 8, 0.35
    q, k, v = (_rand((1, 3, n, d), 70 + i) for i in range(3))
    m = -(-n // b)
    g = np.random.default_rng(77)
    mask = g.random((1, 3, m, m)) < 0.4
    mask[..., np.arange(m), (np.arange(m) * 3) % m] = True  # at least one block per row
    got = O.masked_attention(q, k, v, b, s, mask)
    ref = _sdpa64(q, k, v, s, _token_mask(mask, n, b))
    assert np.allclose(got, ref, rtol=0, atol=1e-12), np.abs(got - ref).max()


def check_masked_vs_brute():
    """Vectorised masked attention equals the scalar loops on a tiny ragged input."""
    n, b, d, s = 21, 4, 3, 0.8
    q, k, v = (_rand((1, 1, n, d), 80 + i) for i in range(3))
    m = -(-n // b)
    rows = [{0}, {0, 1}, {2, 5}, {1, 3}, {4}, {0, 5}]
    mask = np.zeros((1, 1, m, m), bool)
    for i, js in enumerate(rows):
        mask[0, 0, i, list(js)] = True
    got = O.masked_attention(q, k, v, b, s, mask)[0, 0]
    want = np.array(brute.masked_attention(q[0, 0].tolist(), k[0, 0].tolist(),
                                           v[0, 0].tolist(), n, b, s, rows))
    assert np.allclose(got, want, rtol=0, atol=1e-12), np.abs(got - want).max()


def check_attention_hull_and_single_token():
    """Each output lies in the box of its kept value rows; a row whose only kept block holds
    one valid token returns that value row exactly; kept-list order does not matter."""
    n, b, d, s = 129, 64, 6, 0.5  # last block holds one token (index 128)
    q, k, v = (_rand((1, 1, n, d), 90 + i) for i in range(3))
    mask = np.zeros((1, 1, 3, 3), bool)
    mask[0, 0, 0, [0, 1]] = True
    mask[0, 0, 1, 2] = True
    mask[0, 0, 2, [1, 2]] = True
    o = O.masked_attention(q, k, v, b, s, mask)[0, 0]
    assert np.array_equal(o[64:128], np.repeat(v[0, 0, 128:129], 64, axis=0))
    lo, hi = v[0, 0, :128].min(0), v[0, 0, :128].max(0)
    assert np.all(o[:64] >= lo - 1e-12) and np.all(o[:64] <= hi + 1e-12)
    count, idx = O.kept_lists(mask)
    rev = idx.copy()
    rev[0, 0, 0, :2] = rev[0, 0, 0, :2][::-1]
    assert np.array_equal(O.mask_from_lists(count, rev, 3), mask)


# ----------------------------------------------------------------------------- epilogue
def check_epilogue_identities():
    """c = 0 gives the sparse output; c = 1 with R captured on the same inputs gives the dense
    output (refresh-step identity); the output is linear in c and c acts per head."""
    n, b, d, s = 200, 32, 8, 0.3
    q, k, v = (_rand((1, 2, n, d), 100 + i) for i in range(3))
    m = -(-n // b)
    probs = O.block_scores(q, k, b, s)
    mask = O.topp_select(probs, 0.6)["mask"]
    assert mask.sum() < mask.size
    o_s = O.masked_attention(q, k, v, b, s, mask)
    o_d, r = O.dense_with_capture(q, k, v, b, s, mask)
    assert np.array_equal(O.residual_epilogue(o_s, r, [0.0, 0.0]), o_s)
    assert np.allclose(O.residual_epilogue(o_s, r, [1.0, 1.0]), o_d, rtol=0, atol=1e-12)
    mixed = O.residual_epilogue(o_s, r, [0.0, 1.0])
    assert np.array_equal(mixed[:, 0], o_s[:, 0])
    assert np.allclose(mixed[:, 1], o_d[:, 1], rtol=0, atol=1e-12)
    half = O.residual_epilogue(o_s, r, [0.5, 0.5])
    assert np.allclose(half, 0.5 * (o_s + o_d), rtol=0, atol=1e-12)
    ref = _sdpa64(q, k, v, s)
    assert np.allclose(o_d, ref, rtol=0, atol=1e-12)
    _, r_all = O.dense_with_capture(q, k, v, b, s, np.ones((1, 2, m, m), bool))
    assert np.all(r_all == 0.0)


def check_lse_closed_forms():
    """Zero queries score every key 0, so lse = ln(number of attended keys): ln N dense, and
    ln(sum of the kept blocks' token counts) under a mask (ragged last block included). With
    every key equal to k0, lse_t = s * q_t . k0 + ln n. Shifting every key by c shifts the
    dense lse of query t by s * q_t . c."""
    n, b, d, s = 150, 32, 8, 0.7  # blocks of 32, 32, 32, 32, 22
    m = -(-n // b)
    q0 = np.zeros((1, 1, n, d))
    k = _rand((1, 1, n, d), 301)
    assert np.allclose(O.attention_lse(q0, k, b, s), math.log(n), rtol=0, atol=1e-13)
    mask = np.zeros((1, 1, m, m), bool)
    mask[0, 0, :, 0] = True
    mask[0, 0, 1, 4] = True
    mask[0, 0, 3, 2:5] = True
    sizes = np.array([32, 32, 32, 32, 22])
    lse = O.attention_lse(q0, k, b, s, mask)
    for i in range(m):
        want = math.log(sizes[mask[0, 0, i]].sum())
        assert np.allclose(lse[0, 0, i * b:min(n, (i + 1) * b)], want, rtol=0, atol=1e-13)
    q = _rand((1, 1, n, d), 302)
    k0 = _rand((d,), 303)
    keq = np.broadcast_to(k0, (1, 1, n, d)).copy()
    want = s * (q[0, 0] @ k0) + math.log(n)
    assert np.allclose(O.attention_lse(q, keq, b, s)[0, 0], want, rtol=0, atol=1e-12)
    c = _rand((d,), 304)
    shifted = O.attention_lse(q, k + c, b, s) - O.attention_lse(q, k, b, s)
    assert np.allclose(shifted[0, 0], s * (q[0, 0] @ c), rtol=0, atol=1e-12)


def check_lse_vs_brute():
    """Vectorised lse equals a scalar Python loop (dense and masked) on tiny inputs."""
    n, b, d, s = 37, 8, 4, 0.9
    m = -(-n // b)
    q, k = _rand((1, 2, n, d), 311), _rand((1, 2, n, d), 312)
    mask = np.zeros((1, 2, m, m), bool)
    mask[0, 0, :, 0] = True
    mask[0, 0, 2, 3] = True
    mask[0, 1] = np.eye(m, dtype=bool)
    mask[0, 1, 4, 1] = True
    dense, masked = O.attention_lse(q, k, b, s), O.attention_lse(q, k, b, s, mask)
    for h in range(2):
        for t in range(n):
            i = t // b
            toks = [u for u in range(n) if mask[0, h, i, u // b]]
            assert abs(dense[0, h, t] - brute.lse_row(q[0, h, t], list(k[0, h]), s)) < 1e-12
            assert abs(masked[0, h, t] -
                       brute.lse_row(q[0, h, t], [k[0, h, u] for u in toks], s)) < 1e-12


def check_kept_mass_identities():
    """Kept mass: 1 with every block kept; equals exp(lse_kept - lse_dense); the dense output
    is the kept-mass mixture of the sparse output and the output over the other keys; grows
    with p (nested kept sets) and stays in [0, 1]."""
    n, b, d, s = 200, 32, 8, 0.4
    m = -(-n // b)
    q, k, v = (_rand((1, 2, n, d), 320 + i) for i in range(3))
    probs = O.block_scores(q, k, b, s)
    lo = O.topp_select(probs, 0.3)["mask"]
    hi = O.topp_select(probs, 0.6)["mask"]
    assert np.all(hi >= lo) and lo.sum() < hi.sum() < hi.size
    ones = np.ones((1, 2, m, m), bool)
    assert np.allclose(O.kept_attention_mass(q, k, b, s, ones), 1.0, rtol=0, atol=1e-14)
    km_lo, km_hi = (O.kept_attention_mass(q, k, b, s, mk) for mk in (lo, hi))
    assert np.all((km_lo > 0) & (km_lo <= km_hi + 1e-15) & (km_hi <= 1 + 1e-15))
    assert np.any(km_hi < 1 - 1e-6)
    lse_d = O.attention_lse(q, k, b, s)
    for mk, km in ((lo, km_lo), (hi, km_hi)):
        assert np.allclose(km, np.exp(O.attention_lse(q, k, b, s, mk) - lse_d), rtol=0,
                           atol=1e-12)
    o_d = O.dense_attention(q, k, v, s)
    o_s = O.masked_attention(q, k, v, b, s, lo)
    rows = [(0, h, i) for h in range(2) for i in range(m) if not lo[0, h, i].all()]
    o_r = O.masked_attention(q, k, v, b, s, ~lo, rows=rows)
    for _, h, i in rows:
        sl = slice(i * b, min(n, (i + 1) * b))
        w = km_lo[0, h, sl][:, None]
        assert np.allclose(w * o_s[0, h, sl] + (1 - w) * o_r[0, h, sl], o_d[0, h, sl],
                           rtol=0, atol=1e-12)


def check_candidate_scores():
    """Restricted scores: with every block a candidate they are the block scores; otherwise
    the block scores renormalised over the candidates (zero elsewhere, rows sum to 1), and a
    scalar loop agrees on a tiny case."""
    n, b, d, s = 300, 32, 8, 0.8
    m = -(-n // b)
    q, k = _rand((1, 2, n, d), 330, 2.0), _rand((1, 2, n, d), 331, 2.0)
    full = O.block_scores(q, k, b, s)
    every = np.ones((1, 2, m, m), bool)
    assert np.allclose(O.candidate_scores(q, k, b, s, every), full, rtol=0, atol=1e-15)
    rng = np.random.default_rng(332)
    cand = rng.random((1, 2, m, m)) < 0.4
    cand[..., 0] = True
    pc = O.candidate_scores(q, k, b, s, cand)
    assert np.all(pc[~cand] == 0.0)
    assert np.allclose(pc.sum(-1), 1.0, rtol=0, atol=1e-14)
    ren = np.where(cand, full, 0.0)
    ren /= ren.sum(-1, keepdims=True)
    assert np.allclose(pc, ren, rtol=1e-12, atol=1e-15)
    qs, ks = q[0, 1, :70].tolist(), k[0, 1, :70].tolist()
    tiny = brute.scores(qs, ks, 70, 16, d, s)  # 5 blocks
    c5 = np.zeros((1, 1, 5, 5), bool)
    c5[0, 0] = [[1, 0, 1, 0, 1], [0, 1, 1, 0, 0], [1, 1, 1, 1, 1], [0, 0, 0, 1, 0],
                [1, 0, 0, 1, 1]]
    pc5 = O.candidate_scores(q[:, 1:, :70], k[:, 1:, :70], 16, s, c5)
    for i in range(5):
        js = [j for j in range(5) if c5[0, 0, i, j]]
        tot = sum(tiny[i][j] for j in js)
        for j in js:
            assert abs(pc5[0, 0, i, j] - tiny[i][j] / tot) < 1e-12


def check_candidate_topp():
    """Restricted top-p keeps only candidates; with every block a candidate it is top-p; when
    the candidates contain the full top-p set at p, the restricted search at p / S (S the
    candidates' share of the full mass) returns that same set; p = 1 keeps every candidate."""
    rows = _random_prob_rows(24, 16, 340)  # [1, 1, 16, 24]
    every = np.ones(rows.shape, bool)
    for p in (0.3, 0.75, 0.95):
        a = O.topp_select_candidates(rows, every, p)
        bm = O.topp_select(rows, p)
        assert np.array_equal(a["mask"], bm["mask"]) and np.array_equal(a["count"], bm["count"])
    base = O.topp_select(rows, 0.6)["mask"]
    rng = np.random.default_rng(341)
    cand = base | (rng.random(rows.shape) < 0.3)
    S = (rows * cand).sum(-1)
    pc = np.where(cand, rows, 0.0) / S[..., None]
    for r in range(rows.shape[2]):
        got = O.topp_select_candidates(pc[:, :, r:r + 1], cand[:, :, r:r + 1],
                                       0.6 / S[0, 0, r])["mask"]
        assert np.array_equal(got[0, 0, 0], base[0, 0, r])
    one = O.topp_select_candidates(pc, cand, 1.0)
    assert np.array_equal(one["mask"], cand)
    half = O.topp_select_candidates(pc, cand, 0.5)
    assert np.all(half["mask"] <= cand) and np.all((pc * half["mask"]).sum(-1) >= 0.5 - 1e-12)


def check_mean_drift():
    """Drift is 0 for identical means, exactly eps for a (1 + eps) scaling, separate for Q̄
    and K̄, and the Frobenius ratio of a hand-sized case."""
    qb, kb = _rand((2, 3, 5, 4), 350), _rand((2, 3, 5, 4), 351)
    assert np.all(O.mean_drift(qb, kb, qb, kb) == 0.0)
    dr = O.mean_drift(qb * 1.25, kb, qb, kb)
    assert np.allclose(dr[..., 0], 0.25, rtol=0, atol=1e-14) and np.all(dr[..., 1] == 0.0)
    dr = O.mean_drift(qb, kb * 0.5, qb, kb)
    assert np.all(dr[..., 0] == 0.0) and np.allclose(dr[..., 1], 0.5, rtol=0, atol=1e-14)
    x = np.zeros((1, 1, 2, 2))
    xr = x.copy()
    xr[0, 0] = [[3.0, 0.0], [0.0, 4.0]]  # norm 5
    x[0, 0] = [[3.0, 1.0], [0.0, 4.0]]   # difference norm 1
    assert np.allclose(O.mean_drift(x, xr, xr, xr)[0, 0], [0.2, 0.0], rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- coarse tail
def _tail_case(n=200, b=32, d=8, seed=400, heads=2):
    q, k, v = (_rand((1, heads, n, d), seed + i) for i in range(3))
    m = -(-n // b)
    rng = np.random.default_rng(seed + 9)
    mask = rng.random((1, heads, m, m)) < 0.45
    mask[..., 0] = True  # every row keeps block 0 and omits the (possibly short) last block
    mask[..., -1] = False
    return q, k, v, mask


def check_tail_block_constant_keys():
    """With every key and value constant over its block (a short last block included) the
    block-mean estimate is exact: coarse tail == exact tail, log-mass and output. The per-token
    query is kept: two queries of one block get different tails."""
    n, b, d = 200, 32, 8  # blocks of 32 x 6 and a last block of 8
    q, k, v, mask = _tail_case(n, b, d, 410)
    kb = O.block_mean_pool(k, b)
    vb = O.block_mean_pool(v, b)
    st, en = O.block_partition(n, b)
    for j in range(len(st)):
        k[:, :, st[j]:en[j]] = kb[:, :, j:j + 1]
        v[:, :, st[j]:en[j]] = vb[:, :, j:j + 1]
    s = 0.9
    cl, co = O.coarse_tail(q, k, v, b, s, mask)
    el, eo = O.exact_tail(q, k, v, b, s, mask)
    assert np.allclose(cl, el, rtol=0, atol=1e-12), np.abs(cl - el).max()
    assert np.allclose(co, eo, rtol=0, atol=1e-12), np.abs(co - eo).max()
    assert abs(cl[0, 0, 0] - cl[0, 0, 1]) > 1e-3


def check_tail_closed_forms():
    """One omitted block j: log-mass ln n_j + s * q . K̄_j and output V̄_j. Two omitted blocks:
    output weights n_j e^{a_j} / (n_0 e^{a_0} + n_1 e^{a_1}) (a logistic in a_1 - a_0)."""
    n, b, d = 150, 32, 4  # last block (index 4) has 22 tokens
    q, k, v, _ = _tail_case(n, b, d, 420, heads=1)
    m = 5
    kb = O.block_mean_pool(k, b)[0, 0]
    vb = O.block_mean_pool(v, b)[0, 0]
    s = 0.7
    mask = np.ones((1, 1, m, m), bool)
    mask[0, 0, 2, 4] = False  # row 2 omits only the short last block
    mask[0, 0, 1, [0, 3]] = False
    cl, co = O.coarse_tail(q, k, v, b, s, mask)
    for t in range(64, 96):
        a = s * q[0, 0, t] @ kb[4]
        assert abs(cl[0, 0, t] - (math.log(22.0) + a)) < 1e-12
        assert np.allclose(co[0, 0, t], vb[4], rtol=0, atol=1e-12)
    for t in range(32, 64):
        a0, a1 = s * q[0, 0, t] @ kb[0], s * q[0, 0, t] @ kb[3]
        w1 = 1.0 / (1.0 + math.exp(a0 - a1))  # both blocks hold 32 tokens
        assert np.allclose(co[0, 0, t], (1 - w1) * vb[0] + w1 * vb[3], rtol=0, atol=1e-12)
        assert abs(cl[0, 0, t] - (math.log(32.0) + np.logaddexp(a0, a1))) < 1e-12
    assert np.all(np.isneginf(cl[0, 0, :32])) and np.all(co[0, 0, :32] == 0.0)


def check_tail_vs_brute():
    """Coarse tail against the scalar brute force on a ragged tiny case."""
    n, b, d = 70, 16, 5  # 5 blocks, the last of 6 tokens
    q, k, v, mask = _tail_case(n, b, d, 430, heads=1)
    s = 0.6
    cl, co = O.coarse_tail(q, k, v, b, s, mask)
    qs, ks, vs = q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()
    for t in range(0, n, 3):
        tail = [j for j in range(5) if not mask[0, 0, t // b, j]]
        bl, bo = brute.coarse_tail_row(qs[t], ks, vs, n, b, tail, s)
        assert abs(cl[0, 0, t] - bl) < 1e-12, (t, cl[0, 0, t], bl)
        assert np.allclose(co[0, 0, t], bo, rtol=0, atol=1e-12)


def check_tail_key_shift():
    """Adding a vector c to every key shifts each query's score by s * q_t . c: both tail
    log-masses move by exactly that per-token amount and the outputs do not change."""
    n, b, d = 130, 32, 6
    q, k, v, mask = _tail_case(n, b, d, 440)
    c = _rand((d,), 441, 0.5)
    s = 0.8
    shift = s * q @ c  # [1, H, N]
    for fn in (O.coarse_tail, O.exact_tail):
        l0, o0 = fn(q, k, v, b, s, mask)
        l1, o1 = fn(q, k + c, v, b, s, mask)
        assert np.allclose(l1 - l0, shift, rtol=0, atol=1e-11), fn.__name__
        assert np.allclose(o1, o0, rtol=0, atol=1e-11), fn.__name__


def check_tail_partition_identity():
    """The kept and the omitted key sets partition the keys: merging the block-sparse output
    and log-sum-exp with the exact tail gives dense attention and the dense log-sum-exp."""
    n, b, d = 200, 32, 8
    q, k, v, mask = _tail_case(n, b, d, 450)
    s = 0.5
    o_s = O.masked_attention(q, k, v, b, s, mask)
    l_s = O.attention_lse(q, k, b, s, mask)
    l_t, o_t = O.exact_tail(q, k, v, b, s, mask)
    out, lse = O.merge_attention(o_s, l_s, o_t, l_t)
    assert np.allclose(out, _sdpa64(q, k, v, s), rtol=0, atol=1e-12)
    sc = s * np.einsum("bhnd,bhmd->bhnm", q, k)
    mx = sc.max(-1)
    assert np.allclose(lse, mx + np.log(np.exp(sc - mx[..., None]).sum(-1)), rtol=0, atol=1e-12)


def check_tail_refresh_identity():
    """At the refresh step the discrepancy makes the reconstruction exact (its error d_h - d_t
    vanishes at t = h): sparse output merged with coarse tail + d equals dense attention. At
    later inputs the reconstructed tail misses the exact one by exactly d_h - d_t."""
    n, b, d = 200, 32, 8
    q, k, v, mask = _tail_case(n, b, d, 460)
    s = 0.5
    cl, co = O.coarse_tail(q, k, v, b, s, mask)
    el, eo = O.exact_tail(q, k, v, b, s, mask)
    dl, do = O.tail_discrepancy(el, eo, cl, co)
    o_s = O.masked_attention(q, k, v, b, s, mask)
    l_s = O.attention_lse(q, k, b, s, mask)
    rec = O.tail_reconstruction(o_s, l_s, cl, co, dl, do)
    assert np.allclose(rec, _sdpa64(q, k, v, s), rtol=0, atol=1e-12)
    q2, k2, v2 = (x + _rand(x.shape, 470 + i, 0.1) for i, x in enumerate((q, k, v)))
    cl2, co2 = O.coarse_tail(q2, k2, v2, b, s, mask)
    el2, eo2 = O.exact_tail(q2, k2, v2, b, s, mask)
    dl2, do2 = O.tail_discrepancy(el2, eo2, cl2, co2)
    assert np.allclose((cl2 + dl) - el2, dl - dl2, rtol=0, atol=1e-12)
    assert np.allclose((co2 + do) - eo2, do - do2, rtol=0, atol=1e-12)
    coarse_only = O.tail_reconstruction(o_s, l_s, cl, co)
    assert np.abs(coarse_only - rec).max() > 1e-6  # the cached discrepancy matters here


def check_tail_empty_and_merge():
    """Every block kept: no tail (-inf, 0), zero discrepancy, and the reconstruction is the
    sparse output itself. merge_attention weighs parts by e^lse: lse ln 3 against ln 1 gives
    3/4 and 1/4, and a part with lse -inf has no weight."""
    n, b, d = 96, 32, 4
    q, k, v, _ = _tail_case(n, b, d, 480)
    every = np.ones((1, 2, 3, 3), bool)
    cl, co = O.coarse_tail(q, k, v, b, 0.5, every)
    el, eo = O.exact_tail(q, k, v, b, 0.5, every)
    assert np.all(np.isneginf(cl)) and np.all(co == 0.0) and np.all(np.isneginf(el))
    dl, do = O.tail_discrepancy(el, eo, cl, co)
    assert np.all(dl == 0.0) and np.all(do == 0.0)
    o_s = O.dense_attention(q, k, v, 0.5, block=b)
    l_s = O.attention_lse(q, k, b, 0.5)
    assert np.array_equal(O.tail_reconstruction(o_s, l_s, cl, co, dl, do), o_s)
    oa, ob = np.full((1, 1, 1, 2), 4.0), np.full((1, 1, 1, 2), -8.0)
    out, lse = O.merge_attention(oa, np.full((1, 1, 1), math.log(3.0)), ob, np.zeros((1, 1, 1)))
    assert np.allclose(out, 1.0, rtol=0, atol=1e-15) and abs(lse[0, 0, 0] - math.log(4.0)) < 1e-15
    out, _ = O.merge_attention(oa, np.full((1, 1, 1), -np.inf), ob, np.zeros((1, 1, 1)))
    assert np.array_equal(out, ob)


# ----------------------------------------------------------------- coarse tail: moment refinements
def check_moment_stats():
    """Block key variance and the pooled value-key covariance against numpy's population
    variance and covariance (ddof 0 / bias=True) per block, the pooled one weighted by n_j / N
    over a ragged partition; and a two-token block k = K̄ +- d, v = V̄ +- w, where the variance is
    d^2 per dimension and the covariance is exactly w d^T."""
    n, b, d = 70, 16, 3  # blocks of 16 x 4 and 6
    k = _rand((1, 2, n, d), 600)
    v = _rand((1, 2, n, d), 601)
    var = O.block_key_variance(k, b)
    cov = O.pooled_value_key_covariance(k, v, b)
    st, en = O.block_partition(n, b)
    want = np.zeros((d, d))
    for j, (a, e) in enumerate(zip(st, en)):
        assert np.allclose(var[0, 1, j], np.var(k[0, 1, a:e], axis=0), rtol=0, atol=1e-13)
        both = np.cov(np.concatenate([v[0, 1, a:e], k[0, 1, a:e]], axis=1).T, bias=True)
        want += (e - a) / n * both[:d, d:]
    assert np.allclose(cov[0, 1], want, rtol=0, atol=1e-13)
    kd, vw = np.array([0.5, -1.0, 2.0]), np.array([3.0, 0.25, -1.5])
    k2 = np.stack([1.0 + kd, 1.0 - kd])[None, None]
    v2 = np.stack([-2.0 + vw, -2.0 - vw])[None, None]
    assert np.allclose(O.block_key_variance(k2, 2)[0, 0, 0], kd * kd, rtol=0, atol=1e-15)
    assert np.allclose(O.pooled_value_key_covariance(k2, v2, 2)[0, 0], np.outer(vw, kd),
                       rtol=0, atol=1e-15)


def _two_key_case(kd, vw, q_rows):
    """One block of two keys K̄ +- kd with values V̄ +- vw, omitted by its only query block."""
    kbar, vbar = np.array([0.3, -0.2, 0.1]), np.array([1.0, -1.0, 0.5])
    k = np.stack([kbar + kd, kbar - kd])[None, None]
    v = np.stack([vbar + vw, vbar - vw])[None, None]
    q = np.asarray(q_rows, dtype=np.float64)[None, None]
    return q, k, v, np.zeros((1, 1, 1, 1), bool), kbar, vbar


def check_tail_moments_two_key_block():
    """Two keys K̄ +- d in one omitted block: the exact log-mass is ln 2 + s q.K̄ + ln cosh(x)
    with x = s q.d, the exact output V̄ + w tanh(x). With d along one dimension the refined
    log-mass is ln 2 + s q.K̄ + x^2 / 2 (the second-order term of ln cosh) and the refined
    output V̄ + w x (the first-order term of tanh), so they miss the exact values by at most
    x^4 / 12 and |w| |x|^3 / 3. With d along two dimensions the refined log-mass takes the
    per-dimension variances only: ln 2 + s q.K̄ + (s^2 / 2)(q_0^2 d_0^2 + q_1^2 d_1^2)."""
    s = 0.4
    kd, vw = np.array([0.9, 0.0, 0.0]), np.array([0.5, -0.25, 1.0])
    q, k, v, mask, kbar, vbar = _two_key_case(kd, vw, [[1.2, -0.7, 0.4], [-0.5, 2.0, 1.0]])
    lse, out = O.coarse_tail(q, k, v, 2, s, mask, moments=True)
    for t in range(2):
        x = s * q[0, 0, t] @ kd
        base = math.log(2.0) + s * q[0, 0, t] @ kbar
        assert abs(lse[0, 0, t] - (base + x * x / 2)) < 1e-14
        assert abs(lse[0, 0, t] - (base + math.log(math.cosh(x)))) <= x ** 4 / 12 + 1e-15
        assert np.allclose(out[0, 0, t], vbar + vw * x, rtol=0, atol=1e-14)
        assert np.all(np.abs(out[0, 0, t] - (vbar + vw * math.tanh(x)))
                      <= np.abs(vw) * abs(x) ** 3 / 3 + 1e-15)
    kd2 = np.array([0.9, -0.6, 0.0])
    q, k, v, mask, kbar, _ = _two_key_case(kd2, vw, [[1.2, -0.7, 0.4], [0.3, 0.3, 0.3]])
    lse, _ = O.coarse_tail(q, k, v, 2, s, mask, moments=True)
    qt = q[0, 0, 0]
    want = math.log(2.0) + s * qt @ kbar + 0.5 * s * s * (qt[0] ** 2 * 0.81 + qt[1] ** 2 * 0.36)
    assert abs(lse[0, 0, 0] - want) < 1e-14


def check_tail_moments_vanish_and_brute():
    """Keys and values constant over each block: no variance, no covariance, so the refined
    tail equals the zeroth-order one and the exact tail. On a ragged random case the refined
    tail agrees with the scalar brute force."""
    n, b, d = 200, 32, 8
    q, k, v, mask = _tail_case(n, b, d, 610)
    kb, vb = O.block_mean_pool(k, b), O.block_mean_pool(v, b)
    st, en = O.block_partition(n, b)
    for j in range(len(st)):
        k[:, :, st[j]:en[j]] = kb[:, :, j:j + 1]
        v[:, :, st[j]:en[j]] = vb[:, :, j:j + 1]
    l1, o1 = O.coarse_tail(q, k, v, b, 0.9, mask, moments=True)
    l0, o0 = O.coarse_tail(q, k, v, b, 0.9, mask)
    el, eo = O.exact_tail(q, k, v, b, 0.9, mask)
    assert np.allclose(l1, l0, rtol=0, atol=1e-13) and np.allclose(o1, o0, rtol=0, atol=1e-13)
    assert np.allclose(l1, el, rtol=0, atol=1e-12) and np.allclose(o1, eo, rtol=0, atol=1e-12)
    n, b, d = 70, 16, 5
    q, k, v, mask = _tail_case(n, b, d, 620, heads=1)
    s = 0.6
    cl, co = O.coarse_tail(q, k, v, b, s, mask, moments=True)
    qs, ks, vs = q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist()
    for t in range(0, n, 3):
        tail = [j for j in range(5) if not mask[0, 0, t // b, j]]
        bl, bo = brute.coarse_tail_moments_row(qs[t], ks, vs, n, b, tail, s)
        assert abs(cl[0, 0, t] - bl) < 1e-12, (t, cl[0, 0, t], bl)
        assert np.allclose(co[0, 0, t], bo, rtol=0, atol=1e-12)


def check_tail_moments_order():
    """The refinements raise the order of the estimate in the score scale s. Keys K̄_j + e_u and
    values V̄_j + W e_u with the same symmetric, axis-aligned deviations e_u in every block (so
    every block's value-key covariance is the pooled one and its key covariance is diagonal):
    halving s divides the zeroth-order log-mass error
    by about 4 (it is O(s^2)) and the refined one by about 16 (O(s^4): the third cumulant of
    symmetric deviations vanishes); the zeroth-order output error by about 2 (O(s)) and the
    refined one by about 4 (O(s^2))."""
    n, b, d = 128, 16, 4
    rng = np.random.default_rng(630)
    # each token deviates along one axis (+- a_d e_d, twice each): mean zero, symmetric, and a
    # diagonal key covariance, so the per-dimension variances hold the whole second cumulant
    amp = rng.uniform(0.5, 1.5, size=d)
    dev = np.concatenate([np.diag(sg * amp) for sg in (1.0, -1.0, 1.0, -1.0)])
    W = rng.normal(size=(d, d))
    kbar = rng.normal(size=(n // b, d))
    vbar = rng.normal(size=(n // b, d))
    k = np.concatenate([kbar[j] + dev for j in range(n // b)])[None, None]
    v = np.concatenate([vbar[j] + dev @ W.T for j in range(n // b)])[None, None]
    q = rng.normal(size=(1, 1, n, d))
    mask = np.zeros((1, 1, n // b, n // b), bool)
    mask[0, 0, :, 0] = True

    def errs(s):
        el, eo = O.exact_tail(q, k, v, b, s, mask)
        out = []
        for mom in (False, True):
            cl, co = O.coarse_tail(q, k, v, b, s, mask, moments=mom)
            out.append((np.abs(cl - el).max(), np.abs(co - eo).max()))
        return out

    e1, e2 = errs(0.02), errs(0.01)
    (l0a, o0a), (l1a, o1a) = e1
    (l0b, o0b), (l1b, o1b) = e2
    assert 3.5 < l0a / l0b < 4.5, l0a / l0b
    assert l1a / l1b > 12.0, l1a / l1b
    assert 1.7 < o0a / o0b < 2.3, o0a / o0b
    assert o1a / o1b > 3.5, o1a / o1b
    assert l1a < 0.1 * l0a and o1a < 0.1 * o0a


def check_tail_moments_shifts():
    """A vector c added to every key leaves the variances and the covariance unchanged and
    moves the refined log-mass by s * q_t . c; one added to every value moves the refined
    output by c."""
    n, b, d = 130, 32, 6
    q, k, v, mask = _tail_case(n, b, d, 640)
    c = _rand((d,), 641, 0.5)
    s = 0.8
    l0, o0 = O.coarse_tail(q, k, v, b, s, mask, moments=True)
    l1, o1 = O.coarse_tail(q, k + c, v, b, s, mask, moments=True)
    assert np.allclose(l1 - l0, s * q @ c, rtol=0, atol=1e-11)
    assert np.allclose(o1, o0, rtol=0, atol=1e-11)
    l2, o2 = O.coarse_tail(q, k, v + c, b, s, mask, moments=True)
    tail = np.isfinite(l0)
    assert np.allclose(l2, l0, rtol=0, atol=1e-12)
    assert np.allclose(o2[tail], (o0 + c)[tail], rtol=0, atol=1e-11)


# ----------------------------------------------------------------------------- FP8 (MX)
def _e4m3_grid():
    return np.array(sorted({brute.e4m3_value(c) for c in range(256)
                            if not math.isnan(brute.e4m3_value(c))}))


def check_e4m3_rounding_vs_brute():
    """E4M3 rounding against an exhaustive nearest-code search over the bit layout: every
    finite value maps to itself, every midpoint between neighbours goes to the even mantissa,
    quarter points go to the nearer value, and random values agree."""
    grid = _e4m3_grid()
    assert len(grid) == 253 and grid.max() == 448.0 and grid.min() == -448.0
    assert np.array_equal(O.e4m3_round(grid), grid)
    mids = (grid[1:] + grid[:-1]) / 2
    quarters = grid[:-1] + (grid[1:] - grid[:-1]) / 4
    rng = np.random.default_rng(500)
    rand = np.concatenate([rng.uniform(-460, 460, 300), rng.normal(0, 0.02, 300)])
    for xs in (mids, quarters, rand):
        got = O.e4m3_round(xs)
        want = np.array([brute.e4m3_nearest(float(x)) for x in xs])
        assert np.array_equal(got, want), xs[np.argmax(got != want)]


def check_mx_scale_closed_forms():
    """Block exponents: max magnitude 1 -> -7, 255 -> 0, 256 -> 1, 2^-3 -> -10; an all-zero
    block -> -127; blocks of 32 along the axis with a ragged last block; every block's largest
    scaled magnitude lies in [128, 256)."""
    x = np.zeros((2, 70))
    x[0, :32] = 0.5
    x[0, 3] = -1.0
    x[0, 32:64] = 255.0
    x[0, 64:] = 256.0
    x[1, 5] = 0.125
    e = O.mx_scale_exponents(x)
    assert e.shape == (2, 3)
    assert np.array_equal(e, [[-7, 0, 1], [-10, -127, -127]]), e
    y = _rand((4, 3, 96), 510, 3.0)
    ey = O.mx_scale_exponents(y, axis=-1)
    top = np.abs(y).reshape(4, 3, 3, 32).max(-1) / np.exp2(ey)
    assert np.all((top >= 128) & (top < 256))
    ez = O.mx_scale_exponents(np.moveaxis(y, -1, 0), axis=0)
    assert np.array_equal(ez, ey)
    # the 32 elements share one scale: next to 192 (E = 0) a value 0.001 lies below 2^-6 and
    # lands on the subnormal spacing 2^-9 of that scale (0.001 -> 2^-9, 0.0004 -> 0)
    b = np.full(32, 0.001)
    b[:16] = 192.0
    b[20] = 0.0004
    qb = O.mx_quantize(b)
    assert qb[0] == 192.0 and qb[16] == 2.0 ** -9 and qb[20] == 0.0


def _on_mx_grid(shape, axis, seed):
    """A tensor that MX quantisation along `axis` leaves unchanged: in each block of 32, E4M3
    values with the largest magnitude in [128, 240], times a random power of two per block."""
    rng = np.random.default_rng(seed)
    g = _e4m3_grid()
    x = np.moveaxis(rng.choice(g[np.abs(g) <= 240], size=shape), axis, -1).copy()
    n = x.shape[-1]
    for lo in range(0, n, 32):
        x[..., lo] = rng.choice([-1.0, 1.0], size=x.shape[:-1]) * rng.choice(g[(g >= 128) & (g <= 240)], size=x.shape[:-1])
        x[..., lo:lo + 32] *= np.exp2(rng.integers(-12, 3, size=x.shape[:-1] + (1,)))
    return np.moveaxis(x, -1, axis)


def check_mx_quantize_invariants():
    """MX quantisation keeps 4 significant bits (relative error <= 2^-4 above the block's
    subnormal edge, absolute <= 2^E * 2^-10 below it), commutes with power-of-two scaling,
    keeps signs, maps a tensor already on the MX grid of its axis onto itself, and agrees with a
    scalar per-block spelling on a ragged case."""
    x = _rand((3, 5, 100), 520, 2.0)
    qx = O.mx_quantize(x)
    sc = np.exp2(np.repeat(O.mx_scale_exponents(x), 32, axis=-1)[..., :100])
    normal = np.abs(x) >= sc * 2.0 ** -6
    assert np.all(np.abs(qx - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal] + 1e-300)
    assert np.all(np.abs(qx - x)[~normal] <= sc[~normal] * 2.0 ** -10)
    assert np.array_equal(O.mx_quantize(x * 8.0), qx * 8.0)
    assert np.array_equal(O.mx_quantize(-x), -qx)
    on = _on_mx_grid((2, 3, 96, 64), 2, 521)
    assert np.array_equal(O.mx_quantize(on, 2), on)
    assert not np.array_equal(O.mx_quantize(on, -1), on)
    row = x[1, 2].tolist()
    want = []
    for lo in range(0, 100, 32):
        want += brute.mx_quantize_group(row[lo:lo + 32])
    assert np.array_equal(qx[1, 2], np.array(want))


def check_attention_mx_definition():
    """The FP8 attention is plain masked attention on MX-quantised Q, K (blocks along the head
    dimension) and V (blocks along the tokens): inputs already on those grids give the bf16-path
    definition exactly, and quantising along the wrong axis does not."""
    q, k, v, mask = _tail_case(192, 32, 64, 530)
    s = 0.125
    qq, kk = _on_mx_grid(q.shape, -1, 531) * 2.0 ** -7, _on_mx_grid(k.shape, -1, 532) * 2.0 ** -7
    vv = _on_mx_grid(v.shape, 2, 533)
    ref = O.masked_attention(qq, kk, vv, 32, s, mask)
    got = O.masked_attention_mx(qq, kk, vv, 32, s, mask)
    assert np.array_equal(got, ref)
    assert np.abs(O.masked_attention(qq, kk, O.mx_quantize(vv, -1), 32, s, mask) - ref).max() > 0
    assert np.abs(O.masked_attention(O.mx_quantize(qq, 2), kk, vv, 32, s, mask) - ref).max() > 0
    raw = O.masked_attention(q, k, v, 32, s, mask)
    err = np.abs(O.masked_attention_mx(q, k, v, 32, s, mask) - raw).max()
    assert 1e-4 < err < 0.5, err  # FP8 inputs move the output, but boundedly


# ----------------------------------------------------------------------------- work counts
def check_kept_flops_and_sparsity():
    """Kept FLOPs are 4 D n_i n_j per kept block pair (one QK^T and one PV product per attended
    (query, key) token pair): every block kept gives the dense count 4 D N^2 per head, one kept
    pair pairing a full block with the short last block gives 4 D b n_last, and a random mask
    gives 4 D times the number of attended token pairs counted token by token. Block sparsity
    is the skipped share of block pairs: 0 with every block kept, 1 - 1/M with one per row."""
    n, b, d = 200, 64, 16  # blocks of 64, 64, 64, 8
    m = 4
    full = np.ones((1, 3, m, m), dtype=bool)
    assert O.kept_flops(full, n, b, d) == 4.0 * d * n * n * 3
    one = np.zeros((1, 1, m, m), dtype=bool)
    one[0, 0, 1, m - 1] = True
    assert O.kept_flops(one, n, b, d) == 4.0 * d * 64 * 8
    rnd = np.random.default_rng(11).random((2, 2, m, m)) < 0.4
    tok_block = np.repeat(np.arange(m), [64, 64, 64, 8])
    pairs = sum(int(rnd[i, h][tok_block][:, tok_block].sum()) for i in range(2) for h in range(2))
    assert O.kept_flops(rnd, n, b, d) == 4.0 * d * pairs
    assert O.block_sparsity(np.full((1, 2, m), m), m) == 0.0
    assert O.block_sparsity(np.ones((1, 2, m)), m) == 1.0 - 1.0 / m


ALL_CHECKS = [
    check_pool_block_constant,
    check_pool_closed_form_ragged,
    check_pool_mass_invariant,
    check_scores_closed_form,
    check_scores_rows_and_degenerate,
    check_scores_scale_and_shift,
    check_scores_vs_brute,
    check_topp_inclusive_dyadic,
    check_topp_ties_lower_index,
    check_topp_invariants,
    check_topp_vs_subset_search,
    check_topp_per_head_threshold,
    check_dense_vs_sdpa,
    check_masked_vs_sdpa,
    check_masked_vs_brute,
    check_attention_hull_and_single_token,
    check_epilogue_identities,
    check_lse_closed_forms,
    check_lse_vs_brute,
    check_kept_mass_identities,
    check_candidate_scores,
    check_candidate_topp,
    check_mean_drift,
    check_tail_block_constant_keys,
    check_tail_closed_forms,
    check_tail_vs_brute,
    check_tail_key_shift,
    check_tail_partition_identity,
    check_tail_refresh_identity,
    check_tail_empty_and_merge,
    check_moment_stats,
    check_tail_moments_two_key_block,
    check_tail_moments_vanish_and_brute,
    check_tail_moments_order,
    check_tail_moments_shifts,
    check_e4m3_rounding_vs_brute,
    check_mx_scale_closed_forms,
    check_mx_quantize_invariants,
    check_attention_mx_definition,
    check_kept_flops_and_sparsity,
]


def failing_checks():
    """Names of the checks that fail against the oracle as it currently stands."""
    bad = []
    for chk in ALL_CHECKS:
        try:
            chk()
        except (AssertionError, ValueError, IndexError) as exc:  # noqa: PERF203
            bad.append((chk.__name__, repr(exc)[:120]))
    return bad


__all__ = ["ALL_CHECKS", "failing_checks"] + [c.__name__ for c in ALL_CHECKS]
