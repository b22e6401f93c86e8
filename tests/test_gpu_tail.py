"""RECAP tail reconstruction on the GPU (coarse tail from block means, discrepancy at a dense
refresh, log-mass merge at a sparse step) against the CPU oracle, through the C ABI.

The kept lists come from the GPU's own top-p (both sides then use the same kept set). Bounds:
  * coarse log-mass: the row-statistics bound plus the largest score change that bf16 block
    means can cause (computed from the data, parity.coarse_lse_atol);
  * discrepancy d_lse: the coarse bound, plus the bf16-weight bound of the exact tail, plus the
    fp32 summation bound of the dense pass amplified by 1 / (tail share), since the exact tail
    is the dense sums minus the kept sums;
  * outputs (coarse fp32 output, discrepancy d_o on rows with a tail share >= 1e-2, the
    refresh-step reconstruction against dense attention): the attention-output rule of
    parity.check_out;
  * merges at other inputs: parity.check_merged, the attention-output rule per merged part
    plus the coarse-tail terms that do not cancel and the merge-weight error.
"""
import math

import numpy as np
import pytest
import torch

import parity
import synth
from gpu_common import bsa, f64, say, to_dev  # noqa: F401
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _check_inf_pattern(got, ref, what):
    g, r = np.isneginf(got), np.isneginf(ref)
    assert np.array_equal(g, r), f"{what}: -inf pattern differs on {int((g != r).sum())} rows"


def _drift(x, name):
    return synth.drifted(x, name, 1)


def _merge_weights(o_s, l_s, l_t, o_t):
    """Oracle weight w of the sparse part in the log-mass merge and max_d |O_s - o_T| per row."""
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.where(np.isneginf(l_t), 1.0, 1.0 / (1.0 + np.exp(l_t - l_s)))
    spread = np.where(np.isneginf(l_t)[..., None], 0.0, np.abs(o_s - o_t)).max(axis=-1)
    return w, spread


TAIL = {
    "tiny": dict(),
    "ragged_d128_b64_bnhd": dict(batch=2, heads=3, head_dim=128, seq=1000, layout="bnhd",
                                 top_p=[0.5, 0.9, 0.99]),
    "b128_short_last_block": dict(heads=2, head_dim=128, block=128, seq=128 * 5 + 20),
    "d64_b128": dict(heads=2, head_dim=64, block=128, seq=2000),
    "one_token_last_block": dict(heads=1, head_dim=64, seq=129),
    # 131 pooled keys: three 64-key tiles in the coarse pass, the last one ragged
    "several_pooled_tiles": dict(heads=1, head_dim=64, seq=64 * 130 + 10, top_p=0.6),
    "single_block_no_tail": dict(heads=2, head_dim=128, seq=37),
    "p_one_no_tail": dict(heads=2, head_dim=128, seq=700, top_p=1.0),
}


@pytest.mark.parametrize("mom", [False, True], ids=["zeroth", "moments"])
@pytest.mark.parametrize("case", list(TAIL))
def test_tail_case(bsa, case, mom):
    kw = dict(TAIL[case])
    seq = kw.pop("seq", None)
    layout = kw.pop("layout", "bhnd")
    top_p = kw.pop("top_p", None)
    grid = synth.WORKLOADS["tiny"].grid if seq is None else (1, 1, seq)
    cfg = synth.workload("tiny", grid=grid, **kw)
    q, k, v = synth.make_qkv(cfg)
    q2, k2, v2 = _drift(q, "q"), _drift(k, "k"), _drift(v, "v")
    N = q.shape[2]
    M = -(-N // cfg.block)
    p_def, _ = synth.head_params(cfg)
    p = p_def if top_p is None else np.broadcast_to(np.asarray(top_p, float), (cfg.heads,))
    s = cfg.head_dim ** -0.5
    say(f"[test] tail {case}: B={cfg.batch} H={cfg.heads} D={cfg.head_dim} N={N} "
        f"block={cfg.block} layout={layout} p={np.round(p, 3).tolist()} moments={mom}")
    qd, kd, vd, q2d, k2d, v2d = (to_dev(x, layout) for x in (q, k, v, q2, k2, v2))
    desc = bsa.make_desc(qd, cfg.block)
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, _, _ = bsa.recap_topp_mask(desc, probs, p.tolist())
    c_lse, c_o = bsa.recap_tail_estimate(desc, qd, kd, vd, count, idx, s, moments=mom)
    out_d, d_lse, d_o = bsa.recap_dense_attn_tail(desc, qd, kd, vd, count, idx, s, moments=mom)
    out_h = bsa.recap_block_sparse_attn_tail(desc, qd, kd, vd, count, idx, s, d_lse, d_o,
                                             moments=mom)
    out_c = bsa.recap_block_sparse_attn_tail(desc, qd, kd, vd, count, idx, s, moments=mom)
    out_2 = bsa.recap_block_sparse_attn_tail(desc, q2d, k2d, v2d, count, idx, s, d_lse, d_o,
                                             moments=mom)
    od_cap, _ = bsa.recap_dense_attn(desc, qd, kd, vd, s, count, idx, capture=True)
    o_sp = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, s)
    torch.cuda.synchronize()
    # the refresh's dense output comes from the same capture pass (extra writes only)
    assert torch.equal(out_d, od_cap)

    cnt, ix = count.cpu().numpy(), idx.cpu().numpy()
    gmask = O.mask_from_lists(cnt, ix, M)
    q64, k64, v64 = (synth.to_f64(x) for x in (q, k, v))
    q2_64, k2_64, v2_64 = (synth.to_f64(x) for x in (q2, k2, v2))
    cl, co = O.coarse_tail(q64, k64, v64, cfg.block, s, gmask, moments=mom)
    el, eo = O.exact_tail(q64, k64, v64, cfg.block, s, gmask)
    dl, do = O.tail_discrepancy(el, eo, cl, co)
    ref_d = O.dense_attention(q64, k64, v64, s, block=cfg.block)
    o_s = O.masked_attention(q64, k64, v64, cfg.block, s, gmask)
    l_s = O.attention_lse(q64, k64, cfg.block, s, gmask)
    lse_d = O.attention_lse(q64, k64, cfg.block, s)

    # coarse tail
    g_cl = c_lse.cpu().numpy().astype(np.float64)
    _check_inf_pattern(g_cl, cl, "coarse lse")
    kbar = O.block_mean_pool(k64, cfg.block)
    tol_c = parity.coarse_lse_atol(q64, kbar, s)
    if mom:
        tol_c += parity.variance_lse_atol(q64, O.block_key_variance(k64, cfg.block), s)
    parity.check_rows_within(g_cl, cl, tol_c, "coarse lse")
    parity.check_out(c_o.cpu().numpy().astype(np.float64), co, "coarse output")

    # discrepancy at the refresh
    g_dl = d_lse.cpu().numpy().astype(np.float64)
    notail = np.isneginf(cl) & np.isneginf(el)
    assert np.all(g_dl[notail] == 0.0), "d_lse must be exactly 0 without a tail"
    with np.errstate(invalid="ignore"):
        share = np.exp(el - lse_d)  # exact tail share of the dense mass (0 without a tail)
    sel = share >= 1e-6
    assert np.all(np.isfinite(g_dl[sel])), "d_lse not finite on rows with a tail"
    bound = tol_c + math.log1p(parity.U_BF16) + (N / 2) * parity.U_F32 / np.where(sel, share, 1)
    parity.check_rows_within(np.where(sel, g_dl, np.nan), np.where(sel, dl, np.nan), bound,
                             "discrepancy d_lse")
    big = share >= 1e-2
    if big.any():
        parity.check_out(f64(d_o)[big], do[big], "discrepancy d_o")

    # merges: at the refresh inputs the reconstruction is the dense output
    parity.check_out(f64(out_h), ref_d, "refresh-step reconstruction vs dense")
    lse_tol = 2 * parity.ATOL_STAT + 2 * tol_c
    w, spread = _merge_weights(o_s, l_s, cl, co)
    parity.check_merged(f64(out_c), O.tail_reconstruction(o_s, l_s, cl, co), w, spread, lse_tol,
                        0, "coarse-only merge")
    o_s2 = O.masked_attention(q2_64, k2_64, v2_64, cfg.block, s, gmask)
    l_s2 = O.attention_lse(q2_64, k2_64, cfg.block, s, gmask)
    cl2, co2 = O.coarse_tail(q2_64, k2_64, v2_64, cfg.block, s, gmask, moments=mom)
    if mom:  # the drifted step's own variance term
        tol_c = max(tol_c, parity.coarse_lse_atol(q2_64, O.block_mean_pool(k2_64, cfg.block), s)
                    + parity.variance_lse_atol(q2_64, O.block_key_variance(k2_64, cfg.block), s))
        lse_tol = 2 * parity.ATOL_STAT + 2 * tol_c
    # the coarse tails of this step and of the refresh both enter (their errors do not cancel)
    w2, spread2 = _merge_weights(o_s2, l_s2, cl2 + dl, co2 + do)
    parity.check_merged(f64(out_2), O.tail_reconstruction(o_s2, l_s2, cl2, co2, dl, do), w2,
                        spread2, lse_tol, 2, "next-step reconstruction")

    if not (~gmask).any():  # no tail anywhere: the merge is the sparse output itself
        assert np.all(np.isneginf(g_cl)) and np.all(g_dl == 0.0)
        assert torch.count_nonzero(d_o) == 0
        assert torch.equal(out_h, o_sp) and torch.equal(out_c, o_sp)


def _rows_of(blocks, block, n):
    return [(0, 0, i) for i in blocks], [(i * block, min(n, (i + 1) * block)) for i in blocks]


@pytest.mark.parametrize("mom", [False, True], ids=["zeroth", "moments"])
def test_full_size_tail(bsa, mom):
    """Wan2.1-14B 720p layer (B=1, H=40, D=128, N=75,600, block 64): refresh with the tail
    discrepancy, the reconstruction at the refresh inputs, and a drifted step that reuses the
    refresh's kept lists and discrepancy; sampled heads and query blocks against the oracle;
    with and without the moment refinements."""
    cfg = synth.WORKLOADS["wan14b_720p"]
    heads = [0, 21]
    say("[test] full-size tail wan14b_720p: generating inputs")
    q, k, v = synth.make_qkv(cfg)
    q1, k1, v1 = _drift(q, "q"), _drift(k, "k"), _drift(v, "v")
    p, _ = synth.head_params(cfg)
    s = cfg.head_dim ** -0.5
    N, blk, M = cfg.seq, cfg.block, cfg.num_blocks
    qd, kd, vd, q1d, k1d, v1d = (to_dev(x) for x in (q, k, v, q1, k1, v1))
    desc = bsa.make_desc(qd, blk)
    say("[gpu] scores, top-p, tail estimate, dense refresh with discrepancy, merges")
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, _, _ = bsa.recap_topp_mask(desc, probs, p.tolist())
    del probs
    c_lse, c_o = bsa.recap_tail_estimate(desc, qd, kd, vd, count, idx, s, moments=mom)
    out_d, d_lse, d_o = bsa.recap_dense_attn_tail(desc, qd, kd, vd, count, idx, s, moments=mom)
    out_h = bsa.recap_block_sparse_attn_tail(desc, qd, kd, vd, count, idx, s, d_lse, d_o,
                                             moments=mom)
    out_1 = bsa.recap_block_sparse_attn_tail(desc, q1d, k1d, v1d, count, idx, s, d_lse, d_o,
                                             moments=mom)
    torch.cuda.synchronize()
    for h in heads:
        blocks = sorted({0, M - 1} | set(np.random.default_rng(300 + h).choice(M, 2, False).tolist()))
        sel, spans = _rows_of(blocks, blk, N)
        say(f"[check] head {h} blocks {blocks}")
        cnt, ix = count[:, h:h + 1].cpu().numpy(), idx[:, h:h + 1].cpu().numpy()
        m_h = O.mask_from_lists(cnt, ix, M)
        q64, k64, v64 = (synth.to_f64(x[:, h:h + 1]) for x in (q, k, v))
        cl, co = O.coarse_tail(q64, k64, v64, blk, s, m_h, rows=sel, moments=mom)
        el, eo = O.exact_tail(q64, k64, v64, blk, s, m_h, rows=sel)
        dl, do = O.tail_discrepancy(el, eo, cl, co)
        ref_d = O.dense_attention(q64, k64, v64, s, rows=sel, block=blk)
        lse_d = O.attention_lse(q64, k64, blk, s, rows=sel)
        q_rows = np.concatenate([q64[:, :, lo:hi] for lo, hi in spans], axis=2)
        tol_c = parity.coarse_lse_atol(q_rows, O.block_mean_pool(k64, blk), s)
        if mom:
            tol_c += parity.variance_lse_atol(q_rows, O.block_key_variance(k64, blk), s)
        g = {name: t[:, h:h + 1].cpu().numpy().astype(np.float64)
             for name, t in (("cl", c_lse), ("co", c_o), ("dl", d_lse), ("do", d_o))}
        g.update({name: f64(t[:, h:h + 1]) for name, t in (("out_d", out_d), ("out_h", out_h),
                                                             ("out_1", out_1))})
        q1_64, k1_64, v1_64 = (synth.to_f64(x[:, h:h + 1]) for x in (q1, k1, v1))
        o_s1 = O.masked_attention(q1_64, k1_64, v1_64, blk, s, m_h, rows=sel)
        l_s1 = O.attention_lse(q1_64, k1_64, blk, s, m_h, rows=sel)
        cl1, co1 = O.coarse_tail(q1_64, k1_64, v1_64, blk, s, m_h, rows=sel, moments=mom)
        if mom:
            q1_rows = np.concatenate([q1_64[:, :, lo:hi] for lo, hi in spans], axis=2)
            tol_c = max(tol_c, parity.coarse_lse_atol(q1_rows, O.block_mean_pool(k1_64, blk), s)
                        + parity.variance_lse_atol(q1_rows, O.block_key_variance(k1_64, blk), s))
        ref_1 = O.tail_reconstruction(o_s1, l_s1, cl1, co1, dl, do)
        w1, spread1 = _merge_weights(o_s1, l_s1, cl1 + dl, co1 + do)
        with np.errstate(invalid="ignore"):
            share = np.exp(el - lse_d)
        for lo, hi in spans:
            r = slice(lo, hi)
            _check_inf_pattern(g["cl"][:, :, r], cl[:, :, r], f"h{h} coarse lse")
            parity.check_rows_within(g["cl"][:, :, r], cl[:, :, r], tol_c, f"h{h} coarse lse")
            parity.check_out(g["co"][:, :, r], co[:, :, r], f"h{h} coarse output")
            sh = share[:, :, r]
            ok = sh >= 1e-6
            bound = tol_c + math.log1p(parity.U_BF16) + (N / 2) * parity.U_F32 / np.where(ok, sh, 1)
            parity.check_rows_within(np.where(ok, g["dl"][:, :, r], np.nan),
                                     np.where(ok, dl[:, :, r], np.nan), bound, f"h{h} d_lse")
            big = sh >= 1e-2
            if big.any():
                parity.check_out(g["do"][:, :, r][big], do[:, :, r][big], f"h{h} d_o")
            parity.check_out(g["out_d"][:, :, r], ref_d[:, :, r], f"h{h} dense")
            parity.check_out(g["out_h"][:, :, r], ref_d[:, :, r], f"h{h} refresh reconstruction")
            parity.check_merged(g["out_1"][:, :, r], ref_1[:, :, r], w1[:, :, r],
                                spread1[:, :, r], 2 * parity.ATOL_STAT + 2 * tol_c, 2,
                                f"h{h} step-1 reconstruction")
