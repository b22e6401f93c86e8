"""Plain float64 CPU oracle for block-sparse top-p attention with a cached-residual epilogue.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the benchmark's CPU-baseline
leg may import this module; the HIP library never does, and this module imports nothing from
it. Every array is upcast to float64 before any arithmetic (bf16 -> fp64 is exact).

Sources (page title, then section / figure):
  [RECAP]   "RECAP: Reciprocal Sparse Attention and Hierarchical Caching for Efficient Video
            Diffusion", paperpeel.com/paper/2610.26244.
  [HEAD]    head-wise adaptive top-p abstract on thelatestinai.com/papers/2610.26244 (page titled
            RECAP), first abstract.
  [GSRS]    Growing Sparsity and Reduced Search abstract, same page, third abstract.
  [CALIB]   CalibAtt, thelatestinai.com/papers/2603.05503.
  [DFS]     "Ride the Wave: Precision-Allocated Sparse Attention for Smooth Video Generation",
            thelatestinai.com/papers/2604.12219 (DFSAttn abstract).

The method reaches plain masked softmax attention exactly (up to rounding) once the kept set
is known, so attention here is that definition written out. Mask prediction is a heuristic,
so it follows the steps in order: block partition, block means, block-pair softmax, top-p.
Readings where the pages are silent (all listed in the design notes):
  * the pooled logits use the attention scale s (default 1/sqrt(D)) and no log-block-size term;
  * the last block may be short; pooling averages its valid tokens only, padded keys carry
    no weight and padded query rows do not exist;
  * equal block probabilities are ordered by lower key-block index first;
  * the threshold is inclusive (the crossing block is kept, so kept mass >= p); p >= 1 keeps
    every block; p = 0 keeps exactly the top block;
  * the residual epilogue adds c_h * R to the sparse output, R = O_dense - O_sparse captured
    at a dense refresh on the same kept set;
  * the coarse tail (RECAP §3.2) uses each query token against the block means of the omitted
    key blocks, a block's mass being its token count times exp(s * q . K̄_j); with the moment
    refinements (moments=True) the block log-mass gains the second-order term
    (s^2 / 2) sum_d q_d^2 Var_j(k_d) (per-dimension key variance within the block, population
    form: the diagonal reading of "key variance"), and the output gains the first-order value
    compensation s * C q with C the pooled within-block value-key covariance of the head (one
    matrix shared by every block); the cached discrepancy is added unscaled.
"""
from __future__ import annotations

import numpy as np


def block_partition(n_tokens: int, block: int):
    """Block j holds tokens [j*b, min(N, (j+1)*b)); M = ceil(N / b); queries and keys alike.

    Blocks of b tokens over the flattened sequence: [CALIB] Table S6 (query x key block
    sizes) and Fig. S14; [DFS] abstract (block sparse attention over token blocks).
    Returns (starts, ends) as int arrays of length M.
    """
    if n_tokens < 1 or block < 1:
        raise ValueError("need n_tokens >= 1 and block >= 1")
    m = -(-n_tokens // block)
    starts = np.arange(m, dtype=np.int64) * block
    ends = np.minimum(starts + block, n_tokens)
    return starts, ends


def block_mean_pool(x: np.ndarray, block: int) -> np.ndarray:
    """Mean of each token block: X̄_j = (1/n_j) * sum_{t in block j} X_t.

    [RECAP] §3.2: block means give the initial estimates used to score omitted interactions.
    x: [B, H, N, D] -> [B, H, M, D] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    starts, ends = block_partition(x.shape[2], block)
    out = np.empty(x.shape[:2] + (len(starts), x.shape[3]), dtype=np.float64)
    for j, (s, e) in enumerate(zip(starts, ends)):
        out[:, :, j, :] = x[:, :, s:e, :].sum(axis=2) / float(e - s)
    return out


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """exp(L - max_j L) / sum_j exp(L - max_j L) along the last axis (two-pass, stable)."""
    shifted = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(shifted)
    return e / e.sum(axis=-1, keepdims=True)


def block_scores(q: np.ndarray, k: np.ndarray, block: int, sm_scale: float) -> np.ndarray:
    """Block-pair probabilities P̄[b,h,i,j] = softmax_j(s * Q̄_i . K̄_j).

    Mask prediction scores block pairs from mean-pooled queries and keys and normalises each
    query-block row with a softmax ([RECAP] §3.2 block means; [HEAD] online top-p mask
    prediction; [GSRS] top-p over block weights). q, k: [B, H, N, D] -> [B, H, M, M].
    """
    qb = block_mean_pool(q, block)
    kb = block_mean_pool(k, block)
    logits = float(sm_scale) * np.matmul(qb, np.swapaxes(kb, -1, -2))
    return softmax_rows(logits)


def topp_select(probs: np.ndarray, top_p) -> dict:
    """Per query-block row, keep the fewest key blocks whose probability mass reaches p_h.

    [HEAD] (per-head top-p thresholds, online top-p), [GSRS] (top-p selection for adaptive
    sparsity), [CALIB] Fig. 5 (threshold the top key blocks per query block):
      1. order key blocks by probability, descending; equal values by lower index first;
      2. C_k = running sum of the first k ordered probabilities (fp64, in that order);
      3. k* = M if p >= 1, else the smallest k with C_k >= p (M if none);
      4. keep the first k* ordered blocks; kept mass = C_{k*}.
    probs: [B, H, M_q, M]; top_p: scalar or per-head array of length H.
    Returns dict(mask bool [B,H,M,M], count int64 [B,H,M], mass float64 [B,H,M],
                 order int64 [B,H,M,M]).
    """
    probs = np.asarray(probs, dtype=np.float64)
    B, H, _, M = probs.shape  # rows are query blocks, columns key blocks
    p = np.broadcast_to(np.asarray(top_p, dtype=np.float64), (H,))
    idx = np.broadcast_to(np.arange(M, dtype=np.int64), probs.shape)
    # lexsort: last key is primary -> (-prob) ascending == prob descending, then index ascending
    order = np.lexsort((idx, -probs), axis=-1)
    sorted_p = np.take_along_axis(probs, order, axis=-1)
    csum = np.cumsum(sorted_p, axis=-1)  # sequential accumulation along each row
    p_b = p[None, :, None, None]
    reached = csum >= p_b
    first = np.where(reached.any(axis=-1), reached.argmax(axis=-1) + 1, M)
    count = np.where(p[None, :, None] >= 1.0, M, first).astype(np.int64)
    rank = np.empty_like(order)
    np.put_along_axis(rank, order, np.broadcast_to(np.arange(M), order.shape), axis=-1)
    mask = rank < count[..., None]
    mass = np.take_along_axis(csum, (count - 1)[..., None], axis=-1)[..., 0]
    return {"mask": mask, "count": count, "mass": mass, "order": order}


def kept_lists(mask: np.ndarray):
    """Ascending kept key-block indices per row: (count [B,H,M], idx [B,H,M,M] padded -1)."""
    B, H, M, _ = mask.shape
    count = mask.sum(axis=-1).astype(np.int64)
    idx = np.full((B, H, M, M), -1, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for i in range(M):
                js = np.nonzero(mask[b, h, i])[0]
                idx[b, h, i, : len(js)] = js
    return count, idx


def mask_from_lists(count: np.ndarray, idx: np.ndarray, m: int) -> np.ndarray:
    """Boolean block mask [B,H,M,M] from kept lists (entries past `count` are ignored)."""
    count = np.asarray(count)
    idx = np.asarray(idx)
    B, H, M = count.shape
    mask = np.zeros((B, H, M, m), dtype=bool)
    for b in range(B):
        for h in range(H):
            for i in range(M):
                c = int(count[b, h, i])
                mask[b, h, i, idx[b, h, i, :c]] = True
    return mask


def _attend(qt: np.ndarray, kt: np.ndarray, vt: np.ndarray, sm_scale: float) -> np.ndarray:
    """softmax(s * q k^T) v for one set of queries over one key set, two-pass in fp64."""
    s = float(sm_scale) * (qt @ kt.T)
    s -= s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    w /= w.sum(axis=-1, keepdims=True)
    return w @ vt


def masked_attention(q, k, v, block: int, sm_scale: float, mask: np.ndarray,
                     rows=None) -> np.ndarray:
    """Block-sparse attention: each query attends only to the valid tokens of its kept blocks.

    For a query t in block i with kept key blocks J_i, O_t = softmax_u(s * Q_t . K_u) V_u over
    u in the union of the blocks in J_i. This is the computation that block-sparse kernels
    perform on "selected interactions" ([RECAP] §4.1 implementation details; [DFS] abstract).
    q, k, v: [B, H, N, D]; mask: bool [B, H, M, M]; rows: optional iterable of (b, h, i)
    query blocks to compute (others are left NaN). Returns float64 [B, H, N, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    starts, ends = block_partition(N, block)
    M = len(starts)
    out = np.full((B, H, N, D), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(M)]
    for b, h, i in rows:
        js = np.nonzero(mask[b, h, i])[0]
        if len(js) == 0:
            raise ValueError("a query block must keep at least one key block")
        toks = np.concatenate([np.arange(starts[j], ends[j]) for j in js])
        qs = slice(starts[i], ends[i])
        out[b, h, qs] = _attend(q[b, h, qs], k[b, h, toks], v[b, h, toks], sm_scale)
    return out


def dense_attention(q, k, v, sm_scale: float, rows=None, block: int = 64) -> np.ndarray:
    """Full softmax attention over all N keys: the dense refresh ([RECAP] §4.1, §3.2)."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, D = q.shape
    M = -(-N // block)
    return masked_attention(q, k, v, block, sm_scale, np.ones((B, H, M, M), dtype=bool),
                            rows=rows)


def residual_epilogue(o_sparse: np.ndarray, residual: np.ndarray, res_scale) -> np.ndarray:
    """O' = O_sparse + c_h * R per head: the cached dense refinement added to the fresh sparse
    estimate ([RECAP] §3.2: with y_t = ȳ_t + d_t the reconstruction ŷ_t = ȳ_t + d_h has error
    d_h - d_t, zero at the refresh step; §1 and §5: fresh statistics set how strongly the aging
    refinement is applied, here the per-head scale c_h)."""
    o_sparse = np.asarray(o_sparse, dtype=np.float64)
    c = np.asarray(res_scale, dtype=np.float64).reshape(1, -1, 1, 1)
    return o_sparse + c * np.asarray(residual, dtype=np.float64)


def dense_with_capture(q, k, v, block: int, sm_scale: float, mask: np.ndarray, rows=None):
    """Dense refresh that also captures the dense-minus-sparse residual on the same inputs.

    R = O_dense - O_sparse(J) ([RECAP] §3.2 discrepancy d_h cached at the refresh step; §2:
    dense-minus-window attention residuals shared across steps). Returns (O_dense, R).
    """
    o_d = dense_attention(q, k, v, sm_scale, rows=rows, block=block)
    o_s = masked_attention(q, k, v, block, sm_scale, mask, rows=rows)
    return o_d, o_d - o_s


def _attended_tokens(mask, b, h, i, starts, ends):
    js = np.nonzero(mask[b, h, i])[0]
    if len(js) == 0:
        raise ValueError("a query block must keep at least one key block")
    return np.concatenate([np.arange(starts[j], ends[j]) for j in js])


def attention_lse(q, k, block: int, sm_scale: float, mask=None, rows=None) -> np.ndarray:
    """Log-sum-exp of the scaled scores over the keys each query attends:
    lse_t = ln sum_u exp(s * Q_t . K_u), u over the valid tokens of the query block's kept key
    blocks (every key when mask is None). It is the normaliser a flash-attention pass ends
    with, from which the exact attention weights follow as exp(s * Q_t . K_u - lse_t) (GSRS
    abstract [GSRS]). Max-shifted in fp64. Returns float64 [B, H, N] (NaN outside
    `rows`, an iterable of (b, h, i) query blocks)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, _ = q.shape
    starts, ends = block_partition(N, block)
    M = len(starts)
    out = np.full((B, H, N), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(M)]
    for b, h, i in rows:
        toks = np.arange(N) if mask is None else _attended_tokens(mask, b, h, i, starts, ends)
        qs = slice(starts[i], ends[i])
        sc = float(sm_scale) * (q[b, h, qs] @ k[b, h, toks].T)
        mx = sc.max(axis=-1)
        out[b, h, qs] = mx + np.log(np.exp(sc - mx[:, None]).sum(axis=-1))
    return out


def kept_attention_mass(q, k, block: int, sm_scale: float, mask, rows=None) -> np.ndarray:
    """Share of each query's dense attention mass that falls on its kept key blocks:
    sum over kept tokens u of softmax_u(s * Q_t . K_u) taken over all N keys. This is the
    attention recall of the block mask ([DFS] abstract) measured exactly at a dense pass.
    Returns float64 [B, H, N] in [0, 1] (NaN outside `rows`)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, _ = q.shape
    starts, ends = block_partition(N, block)
    M = len(starts)
    out = np.full((B, H, N), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(M)]
    for b, h, i in rows:
        qs = slice(starts[i], ends[i])
        sc = float(sm_scale) * (q[b, h, qs] @ k[b, h].T)
        w = np.exp(sc - sc.max(axis=-1, keepdims=True))
        w /= w.sum(axis=-1, keepdims=True)
        out[b, h, qs] = w[:, _attended_tokens(mask, b, h, i, starts, ends)].sum(axis=-1)
    return out


def candidate_scores(q, k, block: int, sm_scale: float, cand: np.ndarray) -> np.ndarray:
    """Block-pair softmax restricted to each query block's candidate key blocks ([GSRS]
    reduced search: a later search runs only over blocks found earlier):
    P_c[b,h,i,j] = exp(s * Q̄_i . K̄_j) / sum_{j' in C_i} exp(s * Q̄_i . K̄_j') for j in C_i,
    0 elsewhere. cand: bool [B,H,M,M]. Returns float64 [B,H,M,M] (block space)."""
    qb = block_mean_pool(q, block)
    kb = block_mean_pool(k, block)
    lg = float(sm_scale) * np.matmul(qb, np.swapaxes(kb, -1, -2))
    lg = np.where(cand, lg, -np.inf)
    mx = lg.max(axis=-1, keepdims=True)
    w = np.where(cand, np.exp(lg - np.where(np.isfinite(mx), mx, 0.0)), 0.0)
    tot = w.sum(axis=-1, keepdims=True)
    return np.divide(w, tot, out=np.zeros_like(w), where=tot > 0)


def topp_select_candidates(probs_c: np.ndarray, cand: np.ndarray, top_p) -> dict:
    """Top-p over each row's candidate distribution: the rule of `topp_select` applied to the
    row restricted to its candidates (in ascending block order, so ties go to the lower block),
    mapped back to block indices. A row without candidates keeps nothing."""
    probs_c = np.asarray(probs_c, dtype=np.float64)
    B, H, R, M = probs_c.shape
    p = np.broadcast_to(np.asarray(top_p, dtype=np.float64), (H,))
    mask = np.zeros((B, H, R, M), dtype=bool)
    count = np.zeros((B, H, R), dtype=np.int64)
    mass = np.zeros((B, H, R), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for i in range(R):
                js = np.nonzero(cand[b, h, i])[0]
                if len(js) == 0:
                    continue
                sub = topp_select(probs_c[b, h, i, js][None, None, None, :], [p[h]])
                keep = sub["mask"][0, 0, 0]
                mask[b, h, i, js[keep]] = True
                count[b, h, i] = int(sub["count"][0, 0, 0])
                mass[b, h, i] = float(sub["mass"][0, 0, 0])
    return {"mask": mask, "count": count, "mass": mass}


def mean_drift(qbar, kbar, qbar_ref, kbar_ref) -> np.ndarray:
    """Relative Frobenius change of the block means per (b, h) against a reference step:
    [..., 0] = ||Q̄ - Q̄_ref|| / ||Q̄_ref||, [..., 1] the same for K̄ (RECAP §2: reuse of
    early-step block indices across nearby steps; the reuse test). float64 [B, H, 2]."""
    out = []
    for x, r in ((qbar, qbar_ref), (kbar, kbar_ref)):
        x = np.asarray(x, dtype=np.float64)
        r = np.asarray(r, dtype=np.float64)
        num = np.sqrt(((x - r) ** 2).sum(axis=(-2, -1)))
        den = np.sqrt((r ** 2).sum(axis=(-2, -1)))
        out.append(np.divide(num, den, out=np.where(num > 0, np.inf, 0.0), where=den > 0))
    return np.stack(out, axis=-1)


def _row_blocks(mask, rows, B, H, M):
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(M)]
    return rows


def block_key_variance(k, block: int) -> np.ndarray:
    """Per-dimension variance of the keys inside each block, population form over the block's
    valid tokens: Var_j(k_d) = (1/n_j) sum_{u in j} (k_{u,d} - K̄_{j,d})^2 ([RECAP] §3.2: key
    variance for the second-order log-mass refinement). k: [B, H, N, D] -> [B, H, M, D]."""
    k = np.asarray(k, dtype=np.float64)
    starts, ends = block_partition(k.shape[2], block)
    kb = block_mean_pool(k, block)
    out = np.empty(k.shape[:2] + (len(starts), k.shape[3]))
    for j, (a, b) in enumerate(zip(starts, ends)):
        dev = k[:, :, a:b] - kb[:, :, j:j + 1]
        out[:, :, j] = (dev * dev).mean(axis=2)
    return out


def pooled_value_key_covariance(k, v, block: int) -> np.ndarray:
    """Pooled within-block value-key covariance of each head ([RECAP] §3.2 and §2: the pooled
    value-key covariance of PISA's shared first-order value compensation):
        C = (1/N) sum_j sum_{u in j} (v_u - V̄_j) (k_u - K̄_j)^T,
    rows indexed by the value dimension, columns by the key dimension; one matrix per (b, h),
    shared by every block. k, v: [B, H, N, D] -> [B, H, D, D]."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    starts, ends = block_partition(k.shape[2], block)
    kb, vb = block_mean_pool(k, block), block_mean_pool(v, block)
    acc = np.zeros(k.shape[:2] + (v.shape[3], k.shape[3]))
    for j, (a, b) in enumerate(zip(starts, ends)):
        dk = k[:, :, a:b] - kb[:, :, j:j + 1]
        dv = v[:, :, a:b] - vb[:, :, j:j + 1]
        acc += np.einsum("bhnv,bhnk->bhvk", dv, dk)
    return acc / float(k.shape[2])


def coarse_tail(q, k, v, block: int, sm_scale: float, mask, rows=None, moments: bool = False):
    """Zeroth-order estimate of the attention over each query's omitted key blocks, from block
    means ([RECAP] §3.2: block means give first estimates of the omitted tail's value and
    normalising mass; the coarse log-mass is the log of the summed block masses, the coarse
    output the block values weighted by their normalised masses; the estimate is recomputed at
    every sparse evaluation).

    For query t of block i and each key block j outside i's kept set, every key of block j is
    replaced by the block mean K̄_j, so the block's mass is n_j * exp(s * Q_t . K̄_j), n_j its
    token count (the last block may be short). Then
        lse_bar_t = ln sum_j n_j exp(s * Q_t . K̄_j)
        o_bar_t   = sum_j n_j exp(s * Q_t . K̄_j) V̄_j / sum_j n_j exp(s * Q_t . K̄_j).
    With moments=True, the two moment refinements the page names (key variance refines the
    log-mass at second order, COBS; pooled value-key covariance refines the value at first
    order, PISA), in the reading written out here: writing each key as K̄_j + e_u,
        ln sum_{u in j} exp(s Q_t . k_u) = ln n_j + s Q_t . K̄_j + ln mean_u exp(s Q_t . e_u)
    and the last term's second-order (cumulant) approximation with the per-dimension variances
    (the diagonal of the block's key covariance: "key variance") is
        (s^2 / 2) sum_d Q_{t,d}^2 Var_j(k_d)                          (`block_key_variance`);
    the block's attention output, to first order in e_u, is V̄_j + s C_j Q_t with C_j the
    block's value-key covariance; C_j is replaced by the pooled C of the head
    (`pooled_value_key_covariance`), shared by every block, so the weighted output gains
    s C Q_t whatever the weights:
        o_bar_t = sum_j w_tj V̄_j / sum_j w_tj + s C Q_t.
    A query block that keeps every key block has no tail: lse_bar = -inf, o_bar = 0.
    q, k, v: [B, H, N, D]; mask: bool [B, H, M, M]. Returns (lse_bar float64 [B, H, N],
    o_bar float64 [B, H, N, D]), NaN outside `rows` (an iterable of (b, h, i)).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, N, D = q.shape
    starts, ends = block_partition(N, block)
    M = len(starts)
    kb = block_mean_pool(k, block)
    vb = block_mean_pool(v, block)
    n = (ends - starts).astype(np.float64)
    s = float(sm_scale)
    if moments:
        var = block_key_variance(k, block)
        cov = pooled_value_key_covariance(k, v, block)
    lse = np.full((B, H, N), np.nan)
    out = np.full((B, H, N, D), np.nan)
    for b, h, i in _row_blocks(mask, rows, B, H, M):
        qs = slice(starts[i], ends[i])
        js = np.nonzero(~np.asarray(mask[b, h, i], dtype=bool))[0]
        if len(js) == 0:
            lse[b, h, qs] = -np.inf
            out[b, h, qs] = 0.0
            continue
        qt = q[b, h, qs]
        logw = s * (qt @ kb[b, h, js].T) + np.log(n[js])[None, :]
        if moments:
            logw = logw + 0.5 * s * s * ((qt * qt) @ var[b, h, js].T)
        mx = logw.max(axis=-1, keepdims=True)
        w = np.exp(logw - mx)
        tot = w.sum(axis=-1)
        lse[b, h, qs] = mx[:, 0] + np.log(tot)
        out[b, h, qs] = (w @ vb[b, h, js]) / tot[:, None]
        if moments:
            out[b, h, qs] += s * (qt @ cov[b, h].T)
    return lse, out


def exact_tail(q, k, v, block: int, sm_scale: float, mask, rows=None):
    """The omitted tail itself: log-sum-exp and softmax attention over the valid tokens of the
    key blocks outside each query block's kept set, i.e. `attention_lse` and
    `masked_attention` on the complementary mask ([RECAP] §3.2: the tail quantity whose coarse
    part the block means estimate; at a dense refresh it is available exactly). An empty tail
    gives -inf and 0. Returns (lse_T [B, H, N], o_T [B, H, N, D]) float64, NaN outside rows."""
    q = np.asarray(q, dtype=np.float64)
    B, H, N, D = q.shape
    M = -(-N // block)
    comp = ~np.asarray(mask, dtype=bool)
    rows = _row_blocks(mask, rows, B, H, M)
    full = [r for r in rows if comp[r].any()]
    empty = [r for r in rows if not comp[r].any()]
    lse = attention_lse(q, k, block, sm_scale, mask=comp, rows=full)
    out = masked_attention(q, k, v, block, sm_scale, comp, rows=full)
    starts, ends = block_partition(N, block)
    for b, h, i in empty:
        lse[b, h, starts[i]:ends[i]] = -np.inf
        out[b, h, starts[i]:ends[i]] = 0.0
    return lse, out


def tail_discrepancy(lse_t, o_t, lse_bar, o_bar):
    """What the coarse estimate leaves unresolved, taken at a dense refresh ([RECAP] §3.2: a
    tail quantity y_t = ȳ_t + d_t; d at the refresh step is cached):
    d_lse = lse_T - lse_bar (0 where both are -inf: no tail), d_o = o_T - o_bar."""
    lse_t = np.asarray(lse_t, dtype=np.float64)
    lse_bar = np.asarray(lse_bar, dtype=np.float64)
    both = np.isneginf(lse_t) & np.isneginf(lse_bar)
    with np.errstate(invalid="ignore"):
        d_lse = np.where(both, 0.0, lse_t - lse_bar)
    return d_lse, np.asarray(o_t, dtype=np.float64) - np.asarray(o_bar, dtype=np.float64)


def merge_attention(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key sets from each part's output and
    log-sum-exp: weights e^lse / (e^lse_a + e^lse_b), log-sum-exp logaddexp(lse_a, lse_b) (the
    log-mass merge of the sparse part with the tail, [RECAP] §3.2). A part with lse = -inf has
    no keys and weight 0. Returns (out, lse)."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    with np.errstate(invalid="ignore"):  # rows left NaN (outside a sample) stay NaN quietly
        lse = np.logaddexp(la, lb)
        wa = np.where(np.isneginf(la), 0.0, np.exp(la - lse))
        wb = np.where(np.isneginf(lb), 0.0, np.exp(lb - lse))
    out = wa[..., None] * o_a + wb[..., None] * o_b
    return out, lse


def tail_reconstruction(o_s, lse_s, lse_bar, o_bar, d_lse=None, d_o=None):
    """RECAP's attention-level reconstruction at a sparse step ([RECAP] §3.2): the fresh coarse
    tail plus the discrepancy cached at the last refresh, ŷ = ȳ + d_h for the log-mass and the
    output, merged with the sparse part by log-mass. Without d the coarse tail is merged as is.
    Returns float64 [B, H, N, D]."""
    lse_t = np.asarray(lse_bar, dtype=np.float64)
    o_t = np.asarray(o_bar, dtype=np.float64)
    if d_lse is not None:
        lse_t = lse_t + np.asarray(d_lse, dtype=np.float64)
        o_t = o_t + np.asarray(d_o, dtype=np.float64)
    return merge_attention(o_s, lse_s, o_t, lse_t)[0]


# ------------------------------------------------------------------ FP8 (MXFP8) products
E4M3_MAX = 448.0  # largest finite OCP E4M3 value (1.75 * 2^8)


def e4m3_round(y) -> np.ndarray:
    """Round to the nearest OCP FP8 E4M3 value, ties to even (sign, 4 exponent bits with bias 7,
    3 mantissa bits; normal values 2^-6..448 carry 4 significant bits, below 2^-6 the spacing
    is 2^-9). Inputs must lie within +-464 (half a step above 448); the MX scaling below keeps
    every magnitude under 256. Returns float64 values (the rounded numbers, not codes)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a >= 464.0) or np.any(~np.isfinite(a)):
        raise ValueError("value outside the E4M3 range")
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)            # subnormals share the spacing of the smallest binade
    step = np.exp2(e - 3.0)            # 3 mantissa bits
    q = np.round(a / step) * step      # numpy rounds halves to even
    return np.where(y < 0, -q, q)


def mx_scale_exponents(x, axis: int = -1, group: int = 32) -> np.ndarray:
    """Shared power-of-two exponent of each group of `group` consecutive elements along `axis`
    (OCP microscaling: one 8-bit exponent per block of 32 elements): E = floor(log2(amax)) - 7,
    so the largest magnitude of a block scales into [128, 256) and never reaches the E4M3 limit;
    clamped to [-127, 127] (the E8M0 range); an all-zero block gets -127. A ragged last group
    covers the remaining elements. Returns float64 exponents, one per group."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    g = -(-n // group)
    pad = np.zeros(x.shape[:-1] + (g * group - n,))
    a = np.abs(np.concatenate([x, pad], axis=-1)).reshape(x.shape[:-1] + (g, group)).max(-1)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7.0
    return np.where(a > 0, np.clip(e, -127.0, 127.0), -127.0)


def mx_quantize(x, axis: int = -1, group: int = 32) -> np.ndarray:
    """MXFP8 (E4M3) quantisation along `axis`: each element is divided by its block's scale
    2^E (`mx_scale_exponents`), rounded to E4M3 (`e4m3_round`) and multiplied back. Returns
    the dequantised float64 array (same shape): exactly the values FP8 products consume. Reading
    for the FP8 variant of the attention products (the pages name FP8 quantisation with fused
    kernels without a format): OCP MX blocks of 32 along each product's contraction dimension."""
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    e = mx_scale_exponents(xm, -1, group)
    sc = np.exp2(np.repeat(e, group, axis=-1)[..., :n])
    return np.moveaxis(e4m3_round(xm / sc) * sc, -1, axis)


def masked_attention_mx(q, k, v, block: int, sm_scale: float, mask: np.ndarray, rows=None):
    """The FP8 variant of block-sparse attention on its defining inputs: Q and K quantised to
    MXFP8 along the head dimension (blocks of 32 dims per token), V along the token axis
    (blocks of 32 tokens per channel, counted from token 0), then `masked_attention` in fp64 on
    the dequantised tensors. The attention weights are rounded to FP8 as well inside the fused
    kernel; that rounding depends on its running maximum and is left to the error bound."""
    return masked_attention(mx_quantize(q, -1), mx_quantize(k, -1), mx_quantize(v, 2), block,
                            sm_scale, mask, rows=rows)


def block_sparsity(count: np.ndarray, m: int) -> float:
    """Fraction of skipped block pairs: 1 - mean(k*) / M."""
    return 1.0 - float(np.mean(count)) / float(m)


def kept_flops(count_or_mask, n_tokens: int, block: int, head_dim: int) -> float:
    """Attention FLOPs on kept pairs: 4 * D * sum over kept (i, j) of n_i * n_j."""
    starts, ends = block_partition(n_tokens, block)
    n = (ends - starts).astype(np.float64)
    mask = np.asarray(count_or_mask)
    return float(4.0 * head_dim * np.einsum("bhij,i,j->", mask.astype(np.float64), n, n))
