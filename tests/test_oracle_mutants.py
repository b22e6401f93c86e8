"""Plant plausible mistakes in the CPU oracle and require that the pins catch every one.

Each mutant replaces one function of `oracle.oracle` (on the CPU, for the duration of one
test) with a version carrying a single typical slip: a dropped term, a wrong sign or index, a
transposed operand, a wrong axis, an off-by-one or a different tie rule. The pins in
`pins.py` must fail for each, which shows they constrain the oracle beyond its own spelling.
"""
import numpy as np
import pytest

import pins
from oracle import oracle as O

_REAL = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _pool_divides_by_block(x, block):
    x = np.asarray(x, dtype=np.float64)
    s, e = O.block_partition(x.shape[2], block)
    out = np.empty(x.shape[:2] + (len(s), x.shape[3]))
    for j, (a, b) in enumerate(zip(s, e)):
        out[:, :, j] = x[:, :, a:b].sum(axis=2) / float(block)
    return out


def _pool_first_token(x, block):
    x = np.asarray(x, dtype=np.float64)
    s, _ = O.block_partition(x.shape[2], block)
    return x[:, :, s, :]


def _scores_with(transform):
    def f(q, k, block, sm_scale):
        qb = O.block_mean_pool(q, block)
        kb = O.block_mean_pool(k, block)
        return transform(qb, kb, block, sm_scale, q.shape[2])
    return f


def _transposed(qb, kb, block, s, n):
    return O.softmax_rows(s * np.matmul(kb, np.swapaxes(qb, -1, -2)))


def _no_scale(qb, kb, block, s, n):
    return O.softmax_rows(np.matmul(qb, np.swapaxes(kb, -1, -2)))


def _column_softmax(qb, kb, block, s, n):
    lg = s * np.matmul(qb, np.swapaxes(kb, -1, -2))
    return np.swapaxes(O.softmax_rows(np.swapaxes(lg, -1, -2)), -1, -2)


def _log_block_size(qb, kb, block, s, n):
    st, en = O.block_partition(n, block)
    lg = s * np.matmul(qb, np.swapaxes(kb, -1, -2)) + np.log((en - st).astype(float))
    return O.softmax_rows(lg)


def _topp_variant(strict=False, ties_high=False, ascending=False, off_by_one=False,
                  head0=False):
    def f(probs, top_p):
        probs = np.asarray(probs, dtype=np.float64)
        B, H, _, M = probs.shape
        p = np.broadcast_to(np.asarray(top_p, dtype=np.float64), (H,)).copy()
        if head0:
            p[:] = p[0]
        idx = np.broadcast_to(np.arange(M), probs.shape)
        tie = -idx if ties_high else idx
        order = np.lexsort((tie, probs if ascending else -probs), axis=-1)
        csum = np.cumsum(np.take_along_axis(probs, order, axis=-1), axis=-1)
        reached = csum > p[None, :, None, None] if strict else csum >= p[None, :, None, None]
        first = np.where(reached.any(-1), reached.argmax(-1) + (0 if off_by_one else 1), M)
        first = np.maximum(first, 1)
        count = np.where(p[None, :, None] >= 1.0, M, first)
        rank = np.empty_like(order)
        np.put_along_axis(rank, order, np.broadcast_to(np.arange(M), order.shape), axis=-1)
        mask = rank < count[..., None]
        mass = np.take_along_axis(csum, (count - 1)[..., None], axis=-1)[..., 0]
        return {"mask": mask, "count": count, "mass": mass, "order": order}
    return f


def _attend_no_scale(qt, kt, vt, s):
    return _REAL["_attend"](qt, kt, vt, 1.0)


def _attend_keys_as_values(qt, kt, vt, s):
    return _REAL["_attend"](qt, kt, kt[:, : vt.shape[1]] if kt.shape[1] >= vt.shape[1] else vt, s)


def _attend_wrong_axis(qt, kt, vt, s):
    lg = s * (qt @ kt.T)
    lg -= lg.max(axis=0, keepdims=True)
    w = np.exp(lg)
    w /= w.sum(axis=0, keepdims=True)
    return w @ vt


def _masked_ignores_mask(q, k, v, block, sm_scale, mask, rows=None):
    return _REAL["masked_attention"](q, k, v, block, sm_scale, np.ones_like(mask), rows=rows)


def _epilogue_minus(o, r, c):
    return _REAL["residual_epilogue"](o, -np.asarray(r), c)


def _epilogue_heads_reversed(o, r, c):
    return _REAL["residual_epilogue"](o, r, np.asarray(c, dtype=float)[::-1])


def _capture_sign(q, k, v, block, sm_scale, mask, rows=None):
    o_d, r = _REAL["dense_with_capture"](q, k, v, block, sm_scale, mask, rows=rows)
    return o_d, -r


def _lse_log2(q, k, block, sm_scale, mask=None, rows=None):
    return _REAL["attention_lse"](q, k, block, sm_scale, mask, rows) / np.log(2.0)


def _lse_no_scale(q, k, block, sm_scale, mask=None, rows=None):
    return _REAL["attention_lse"](q, k, block, 1.0, mask, rows)


def _lse_ignores_mask(q, k, block, sm_scale, mask=None, rows=None):
    return _REAL["attention_lse"](q, k, block, sm_scale, None, rows)


def _kept_mass_renormalised(q, k, block, sm_scale, mask, rows=None):
    km = _REAL["kept_attention_mass"](q, k, block, sm_scale, mask, rows)
    return np.where(np.isnan(km), km, 1.0)


def _kept_mass_complement(q, k, block, sm_scale, mask, rows=None):
    return 1.0 - _REAL["kept_attention_mass"](q, k, block, sm_scale, mask, rows)


def _cand_scores_over_all(q, k, block, sm_scale, cand):
    return np.where(cand, O.block_scores(q, k, block, sm_scale), 0.0)


def _cand_topp_keeps_all_at_one(probs_c, cand, top_p):
    res = _REAL["topp_select_candidates"](probs_c, cand, top_p)
    if np.all(np.asarray(top_p) >= 1.0):
        res["mask"] = np.ones_like(res["mask"])
    return res


def _cand_topp_unrenormalised(probs_c, cand, top_p):
    return _REAL["topp_select"](probs_c, top_p)


def _drift_squared(qbar, kbar, qref, kref):
    return _REAL["mean_drift"](qbar, kbar, qref, kref) ** 2


def _drift_swapped(qbar, kbar, qref, kref):
    return _REAL["mean_drift"](qbar, kbar, qref, kref)[..., ::-1]


def _coarse_variant(no_count=False, full_count=False, pooled_query=False, with_kept=False):
    def f(q, k, v, block, sm_scale, mask, rows=None, moments=False):  # zeroth order only
        q = np.asarray(q, dtype=np.float64)
        B, H, N, D = q.shape
        st, en = O.block_partition(N, block)
        M = len(st)
        kb, vb = O.block_mean_pool(k, block), O.block_mean_pool(v, block)
        qb = O.block_mean_pool(q, block)
        n = np.full(M, float(block)) if full_count else (en - st).astype(np.float64)
        lse, out = np.full((B, H, N), np.nan), np.full((B, H, N, D), np.nan)
        for b in range(B):
            for h in range(H):
                for i in range(M):
                    qs = slice(st[i], en[i])
                    js = np.arange(M) if with_kept else np.nonzero(~mask[b, h, i])[0]
                    if len(js) == 0:
                        lse[b, h, qs], out[b, h, qs] = -np.inf, 0.0
                        continue
                    qq = np.broadcast_to(qb[b, h, i], q[b, h, qs].shape) if pooled_query \
                        else q[b, h, qs]
                    lw = sm_scale * (qq @ kb[b, h, js].T)
                    if not no_count:
                        lw = lw + np.log(n[js])[None, :]
                    mx = lw.max(-1, keepdims=True)
                    w = np.exp(lw - mx)
                    lse[b, h, qs] = mx[:, 0] + np.log(w.sum(-1))
                    out[b, h, qs] = (w @ vb[b, h, js]) / w.sum(-1)[:, None]
        return lse, out
    return f


def _exact_tail_of_kept(q, k, v, block, sm_scale, mask, rows=None):
    return _REAL["exact_tail"](q, k, v, block, sm_scale, ~np.asarray(mask, dtype=bool) | (
        np.arange(mask.shape[-1]) == 0), rows)


def _discrepancy_sign(lse_t, o_t, lse_bar, o_bar):
    dl, do = _REAL["tail_discrepancy"](lse_t, o_t, lse_bar, o_bar)
    return -dl, -do


def _merge_swapped(o_a, lse_a, o_b, lse_b):
    return _REAL["merge_attention"](o_b, lse_a, o_a, lse_b)


def _merge_linear_weights(o_a, lse_a, o_b, lse_b):
    la, lb = np.asarray(lse_a, dtype=np.float64), np.asarray(lse_b, dtype=np.float64)
    wa = np.where(np.isneginf(la), 0.0, np.abs(la))
    wb = np.where(np.isneginf(lb), 0.0, np.abs(lb))
    tot = np.where(wa + wb > 0, wa + wb, 1.0)
    out = (wa / tot)[..., None] * o_a + (wb / tot)[..., None] * o_b
    return out, np.logaddexp(la, lb)


def _reconstruction_without_lse_shift(o_s, lse_s, lse_bar, o_bar, d_lse=None, d_o=None):
    return _REAL["tail_reconstruction"](o_s, lse_s, lse_bar, o_bar,
                                        None if d_lse is None else np.zeros_like(d_lse), d_o)


def _e4m3_variant(away=False, bits=3, sub_floor=-6.0):
    def f(y):
        y = np.asarray(y, dtype=np.float64)
        a = np.abs(y)
        if np.any(a >= 464.0):
            raise ValueError("value outside the E4M3 range")
        e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), sub_floor)
        step = np.exp2(e - bits)
        q = (np.floor(a / step + 0.5) if away else np.round(a / step)) * step
        return np.where(y < 0, -q, q)
    return f


def _mx_exp_offset(off):
    def f(x, axis=-1, group=32):
        x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
        n = x.shape[-1]
        g = -(-n // group)
        pad = np.zeros(x.shape[:-1] + (g * group - n,))
        a = np.abs(np.concatenate([x, pad], axis=-1)).reshape(x.shape[:-1] + (g, group)).max(-1)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))) - off
        return np.where(a > 0, np.clip(e, -127.0, 127.0), -127.0)
    return f


def _mx_group16(x, axis=-1, group=32):
    return _REAL["mx_quantize"](x, axis, 16)


def _attention_mx_v_wrong_axis(q, k, v, block, sm_scale, mask, rows=None):
    return O.masked_attention(O.mx_quantize(q, -1), O.mx_quantize(k, -1), O.mx_quantize(v, -1),
                              block, sm_scale, mask, rows=rows)


def _kept_flops_full_blocks(count_or_mask, n_tokens, block, head_dim):
    mask = np.asarray(count_or_mask, dtype=np.float64)
    return float(4.0 * head_dim * block * block * mask.sum())


def _kept_flops_one_product(count_or_mask, n_tokens, block, head_dim):
    return 0.5 * _REAL["kept_flops"](count_or_mask, n_tokens, block, head_dim)


def _sparsity_kept_share(count, m):
    return float(np.mean(count)) / float(m)


def _moments_variant(half=0.5, s_power=2, full_quad=False, transposed=False, comp_scale=True,
                     sample_var=False, raw_cov=False):
    """coarse_tail with moments, written out with one planted slip in a refinement."""
    def f(q, k, v, block, sm_scale, mask, rows=None, moments=False):
        if not moments:
            return _REAL["coarse_tail"](q, k, v, block, sm_scale, mask, rows)
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, N, D = q.shape
        st, en = O.block_partition(N, block)
        M = len(st)
        kb, vb = O.block_mean_pool(k, block), O.block_mean_pool(v, block)
        n = (en - st).astype(np.float64)
        var = np.empty((B, H, M, D))
        cov = np.zeros((B, H, D, D))
        sig = [None] * M
        for j in range(M):
            dk = k[:, :, st[j]:en[j]] - kb[:, :, j:j + 1]
            dv = v[:, :, st[j]:en[j]] - (0.0 if raw_cov else vb[:, :, j:j + 1])
            var[:, :, j] = (dk * dk).sum(2) / (max(n[j] - 1, 1) if sample_var else n[j])
            sig[j] = np.einsum("bhnd,bhne->bhde", dk, dk) / n[j]
            cov += np.einsum("bhnv,bhnk->bhvk", dv, dk if not raw_cov else k[:, :, st[j]:en[j]])
        cov /= N
        if transposed:
            cov = np.swapaxes(cov, -1, -2)
        s = float(sm_scale)
        lse, out = np.full((B, H, N), np.nan), np.full((B, H, N, D), np.nan)
        for b in range(B):
            for h in range(H):
                for i in range(M):
                    qs = slice(st[i], en[i])
                    js = np.nonzero(~np.asarray(mask[b, h, i], dtype=bool))[0]
                    if len(js) == 0:
                        lse[b, h, qs], out[b, h, qs] = -np.inf, 0.0
                        continue
                    qt = q[b, h, qs]
                    lw = s * (qt @ kb[b, h, js].T) + np.log(n[js])[None, :]
                    if full_quad:
                        quad = np.stack([np.einsum("td,de,te->t", qt, sig[j][b, h], qt)
                                         for j in js], axis=1)
                    else:
                        quad = (qt * qt) @ var[b, h, js].T
                    lw = lw + half * s ** s_power * quad
                    mx = lw.max(-1, keepdims=True)
                    w = np.exp(lw - mx)
                    lse[b, h, qs] = mx[:, 0] + np.log(w.sum(-1))
                    out[b, h, qs] = (w @ vb[b, h, js]) / w.sum(-1)[:, None]
                    out[b, h, qs] += (s if comp_scale else 1.0) * (qt @ cov[b, h].T)
        return lse, out
    return f


MUTANTS = {
    "pool divides by the full block size": ("block_mean_pool", _pool_divides_by_block),
    "pool takes the first token": ("block_mean_pool", _pool_first_token),
    "scores transposed (keys x queries)": ("block_scores", _scores_with(_transposed)),
    "scores drop the scale": ("block_scores", _scores_with(_no_scale)),
    "softmax over query blocks": ("block_scores", _scores_with(_column_softmax)),
    "log block size added to logits": ("block_scores", _scores_with(_log_block_size)),
    "strict threshold": ("topp_select", _topp_variant(strict=True)),
    "ties prefer higher index": ("topp_select", _topp_variant(ties_high=True)),
    "keeps the smallest blocks": ("topp_select", _topp_variant(ascending=True)),
    "count off by one": ("topp_select", _topp_variant(off_by_one=True)),
    "head 0 threshold for all heads": ("topp_select", _topp_variant(head0=True)),
    "attention drops the scale": ("_attend", _attend_no_scale),
    "attention uses keys as values": ("_attend", _attend_keys_as_values),
    "attention softmax over queries": ("_attend", _attend_wrong_axis),
    "attention ignores the mask": ("masked_attention", _masked_ignores_mask),
    "epilogue subtracts the residual": ("residual_epilogue", _epilogue_minus),
    "epilogue scales reversed across heads": ("residual_epilogue", _epilogue_heads_reversed),
    "captured residual has the wrong sign": ("dense_with_capture", _capture_sign),
    "lse in base 2": ("attention_lse", _lse_log2),
    "lse drops the scale": ("attention_lse", _lse_no_scale),
    "lse ignores the mask": ("attention_lse", _lse_ignores_mask),
    "kept mass renormalised over the kept keys": ("kept_attention_mass", _kept_mass_renormalised),
    "kept mass of the complement": ("kept_attention_mass", _kept_mass_complement),
    "candidate scores not renormalised": ("candidate_scores", _cand_scores_over_all),
    "candidate top-p at p = 1 keeps every block": ("topp_select_candidates",
                                                   _cand_topp_keeps_all_at_one),
    "candidate top-p ignores the candidates": ("topp_select_candidates",
                                               _cand_topp_unrenormalised),
    "drift without the square root": ("mean_drift", _drift_squared),
    "drift of Q and K swapped": ("mean_drift", _drift_swapped),
    "coarse tail without block token counts": ("coarse_tail", _coarse_variant(no_count=True)),
    "coarse tail counts a full last block": ("coarse_tail", _coarse_variant(full_count=True)),
    "coarse tail scores the pooled query": ("coarse_tail", _coarse_variant(pooled_query=True)),
    "coarse tail includes the kept blocks": ("coarse_tail", _coarse_variant(with_kept=True)),
    "exact tail over the kept blocks": ("exact_tail", _exact_tail_of_kept),
    "discrepancy coarse minus exact": ("tail_discrepancy", _discrepancy_sign),
    "merge pairs weights with the wrong outputs": ("merge_attention", _merge_swapped),
    "merge weighs by lse, not e^lse": ("merge_attention", _merge_linear_weights),
    "reconstruction drops the log-mass discrepancy": ("tail_reconstruction",
                                                      _reconstruction_without_lse_shift),
    "E4M3 ties away from zero": ("e4m3_round", _e4m3_variant(away=True)),
    "E4M3 with two mantissa bits": ("e4m3_round", _e4m3_variant(bits=2)),
    "E4M3 subnormal spacing one binade too low": ("e4m3_round", _e4m3_variant(sub_floor=-7.0)),
    "MX block exponent offset 8 (overflows E4M3)": ("mx_scale_exponents", _mx_exp_offset(8)),
    "MX block exponent offset 6": ("mx_scale_exponents", _mx_exp_offset(6)),
    "MX blocks of 16": ("mx_quantize", _mx_group16),
    "variance term without the 1/2": ("coarse_tail", _moments_variant(half=1.0)),
    "variance term scaled by s, not s^2": ("coarse_tail", _moments_variant(s_power=1)),
    "full key covariance instead of per-dimension variance": ("coarse_tail",
                                                              _moments_variant(full_quad=True)),
    "sample (n - 1) key variance": ("coarse_tail", _moments_variant(sample_var=True)),
    "value compensation with the transposed covariance": ("coarse_tail",
                                                           _moments_variant(transposed=True)),
    "value compensation without the scale": ("coarse_tail", _moments_variant(comp_scale=False)),
    "covariance of raw, uncentred tokens": ("coarse_tail", _moments_variant(raw_cov=True)),
    "kept FLOPs count full blocks": ("kept_flops", _kept_flops_full_blocks),
    "kept FLOPs count one product": ("kept_flops", _kept_flops_one_product),
    "sparsity is the kept share": ("block_sparsity", _sparsity_kept_share),
    "FP8 attention quantises V along the head dimension": ("masked_attention_mx",
                                                           _attention_mx_v_wrong_axis),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, repl = MUTANTS[name]
    monkeypatch.setattr(O, attr, repl)
    # a planted mistake may produce empty tails and NaN ratios; the pins fail on them, quietly
    with np.errstate(all="ignore"):
        failed = pins.failing_checks()
    assert failed, f"no pin caught the planted mistake: {name}"


def test_real_oracle_passes_every_pin():
    assert pins.failing_checks() == []
