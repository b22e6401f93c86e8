"""Scalar pure-Python brute force for tiny inputs (test infrastructure, like the rest of the oracle).

Every quantity is computed element by element with Python floats and `math`, without numpy
vectorisation, so that the vectorised oracle can be checked against an independent spelling
of the same definitions. The top-p check here does not sort at all: it enumerates every subset
of key blocks, which characterises the top-p set without reference to an ordering.
"""
from __future__ import annotations

import itertools
import math


def pool(x, n_tokens, block, dim):
    """x: nested list [N][D] -> [M][D] block means over valid tokens."""
    m = -(-n_tokens // block)
    out = []
    for j in range(m):
        lo, hi = j * block, min(n_tokens, (j + 1) * block)
        row = []
        for d in range(dim):
            acc = 0.0
            for t in range(lo, hi):
                acc += x[t][d]
            row.append(acc / (hi - lo))
        out.append(row)
    return out


def scores(q, k, n_tokens, block, dim, sm_scale):
    """[M][M] block-pair softmax of s * (mean q_i . mean k_j)."""
    qb = pool(q, n_tokens, block, dim)
    kb = pool(k, n_tokens, block, dim)
    m = len(qb)
    out = []
    for i in range(m):
        logits = []
        for j in range(m):
            dot = 0.0
            for d in range(dim):
                dot += qb[i][d] * kb[j][d]
            logits.append(sm_scale * dot)
        mx = max(logits)
        ex = [math.exp(v - mx) for v in logits]
        tot = sum(ex)
        out.append([e / tot for e in ex])
    return out


def min_cardinality_subsets(prob_row, p):
    """Exhaustive search: (k*, best mass) where k* is the fewest blocks reaching mass >= p and
    best mass is the largest mass over all subsets of that size. p >= 1 -> all blocks."""
    m = len(prob_row)
    if p >= 1.0:
        return m, sum(prob_row)
    for size in range(1, m + 1):
        best = None
        for sub in itertools.combinations(range(m), size):
            mass = sum(prob_row[j] for j in sub)
            if best is None or mass > best:
                best = mass
        if best >= p:
            return size, best
    return m, sum(prob_row)


def attention_row(qt, keys, values, sm_scale):
    """One query against a list of keys/values: softmax(s q.k) weighted sum, scalar loops."""
    logits = []
    for kr in keys:
        dot = 0.0
        for a, b in zip(qt, kr):
            dot += a * b
        logits.append(sm_scale * dot)
    mx = max(logits)
    w = [math.exp(v - mx) for v in logits]
    tot = sum(w)
    dim = len(values[0])
    out = [0.0] * dim
    for wi, vr in zip(w, values):
        for d in range(dim):
            out[d] += wi / tot * vr[d]
    return out


def masked_attention(q, k, v, n_tokens, block, sm_scale, mask_rows):
    """q, k, v: [N][D] lists; mask_rows[i] = set of kept key blocks for query block i."""
    out = []
    for t in range(n_tokens):
        i = t // block
        toks = [u for u in range(n_tokens) if (u // block) in mask_rows[i]]
        out.append(attention_row(q[t], [k[u] for u in toks], [v[u] for u in toks], sm_scale))
    return out


def lse_row(qt, keys, sm_scale):
    """ln sum_u exp(s * q . k_u) for one query over a list of key rows, with plain floats."""
    logits = [sm_scale * sum(a * b for a, b in zip(qt, ku)) for ku in keys]
    mx = max(logits)
    return mx + math.log(sum(math.exp(x - mx) for x in logits))


def coarse_tail_row(qt, k, v, n_tokens, block, tail_blocks, sm_scale):
    """Block-mean estimate of one query's attention over the key blocks in `tail_blocks`:
    each block j counts n_j keys equal to its mean key, carrying its mean value. Returns
    (ln of the summed block masses, mass-weighted mean of the block values) with plain floats;
    (-inf, zeros) for an empty tail."""
    dim = len(v[0])
    if not tail_blocks:
        return -math.inf, [0.0] * dim
    kb = pool(k, n_tokens, block, dim)
    vb = pool(v, n_tokens, block, dim)
    logm = []
    for j in tail_blocks:
        nj = min(n_tokens, (j + 1) * block) - j * block
        dot = 0.0
        for a, b in zip(qt, kb[j]):
            dot += a * b
        logm.append(math.log(nj) + sm_scale * dot)
    mx = max(logm)
    w = [math.exp(x - mx) for x in logm]
    tot = sum(w)
    out = [0.0] * dim
    for wi, j in zip(w, tail_blocks):
        for d in range(dim):
            out[d] += wi / tot * vb[j][d]
    return mx + math.log(tot), out


def block_variance(k, n_tokens, block, dim):
    """[M][D] per-dimension key variance inside each block (population form), plain floats."""
    kb = pool(k, n_tokens, block, dim)
    out = []
    for j in range(len(kb)):
        lo, hi = j * block, min(n_tokens, (j + 1) * block)
        row = []
        for d in range(dim):
            acc = 0.0
            for t in range(lo, hi):
                acc += (k[t][d] - kb[j][d]) ** 2
            row.append(acc / (hi - lo))
        out.append(row)
    return out


def pooled_covariance(k, v, n_tokens, block, dim):
    """[D][D] pooled within-block value-key covariance, C[a][c] over value dim a, key dim c."""
    kb = pool(k, n_tokens, block, dim)
    vb = pool(v, n_tokens, block, dim)
    c = [[0.0] * dim for _ in range(dim)]
    for t in range(n_tokens):
        j = t // block
        for a in range(dim):
            for e in range(dim):
                c[a][e] += (v[t][a] - vb[j][a]) * (k[t][e] - kb[j][e])
    return [[x / n_tokens for x in row] for row in c]


def coarse_tail_moments_row(qt, k, v, n_tokens, block, tail_blocks, sm_scale):
    """The block-mean estimate with both moment refinements, with plain floats: block
    log-mass ln n_j + s q . K̄_j + (s^2/2) sum_d q_d^2 Var_j(k_d); output the mass-weighted
    block means plus s C q with the pooled covariance C."""
    dim = len(v[0])
    if not tail_blocks:
        return -math.inf, [0.0] * dim
    kb = pool(k, n_tokens, block, dim)
    vb = pool(v, n_tokens, block, dim)
    var = block_variance(k, n_tokens, block, dim)
    cov = pooled_covariance(k, v, n_tokens, block, dim)
    logm = []
    for j in tail_blocks:
        nj = min(n_tokens, (j + 1) * block) - j * block
        dot = 0.0
        quad = 0.0
        for d in range(dim):
            dot += qt[d] * kb[j][d]
            quad += qt[d] * qt[d] * var[j][d]
        logm.append(math.log(nj) + sm_scale * dot + 0.5 * sm_scale * sm_scale * quad)
    mx = max(logm)
    w = [math.exp(x - mx) for x in logm]
    tot = sum(w)
    out = [0.0] * dim
    for wi, j in zip(w, tail_blocks):
        for d in range(dim):
            out[d] += wi / tot * vb[j][d]
    for a in range(dim):
        for e in range(dim):
            out[a] += sm_scale * cov[a][e] * qt[e]
    return mx + math.log(tot), out


def e4m3_value(code: int) -> float:
    """Value of an 8-bit OCP E4M3 code from its bit fields (sign, exponent with bias 7, 3-bit
    mantissa; exponent field 0 is subnormal; S.1111.111 is NaN)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def e4m3_nearest(x: float) -> float:
    """Nearest finite E4M3 value by exhaustive search over all 256 codes; a tie goes to the
    code with an even mantissa (its lowest bit clear)."""
    best, best_code, best_d = None, None, None
    for c in range(256):
        v = e4m3_value(c)
        if math.isnan(v):
            continue
        d = abs(v - x)
        if best is None or d < best_d or (d == best_d and (c & 1) == 0 and (best_code & 1) == 1):
            best, best_code, best_d = v, c, d
    return best


def mx_quantize_group(vals, group_max_exp_offset: int = 7):
    """MX quantisation of one block (a list of floats): E = floor(log2(max |x|)) - 7, each element
    divided by 2^E, rounded with `e4m3_nearest`, multiplied back; an all-zero block stays zero."""
    amax = max(abs(v) for v in vals)
    if amax == 0.0:
        return [0.0 for _ in vals]
    e = max(-127, min(127, math.floor(math.log2(amax)) - group_max_exp_offset))
    return [e4m3_nearest(v / 2.0 ** e) * 2.0 ** e for v in vals]
