"""HIP library vs the CPU oracle on the same seeded inputs, through the C ABI.

Small cases are compared in full (several tiles, ragged tails, degenerate sizes, both tensor
layouts, D in {64, 128}, block in {64, 128}, p = 0 and p = 1). The full-size workloads run in
the launch configuration the benchmark times and are compared on sampled heads and rows.
"""
import numpy as np
import pytest
import torch

import parity
import synth
from oracle import oracle as O

from gpu_common import DEV, bsa, f64, say, to_dev  # noqa: F401

pytestmark = pytest.mark.gpu


def run_small(bsa, cfg, seq=None, layout="bhnd", top_p=None, res_scale=None):
    q, k, v = synth.make_qkv(cfg, seq=seq)
    r = synth.make_residual(cfg, seq=seq)
    N = q.shape[2]
    M = -(-N // cfg.block)
    p_def, c_def = synth.head_params(cfg)
    p = p_def if top_p is None else np.broadcast_to(np.asarray(top_p, float), (cfg.heads,))
    c = np.full(cfg.heads, 0.5) if res_scale is None else np.asarray(res_scale, float)
    s = cfg.head_dim ** -0.5
    say(f"[case] B={cfg.batch} H={cfg.heads} D={cfg.head_dim} N={N} block={cfg.block} "
        f"layout={layout} p={np.round(p, 3).tolist()}")
    qd, kd, vd, rd = (to_dev(x, layout) for x in (q, k, v, r))
    desc = bsa.make_desc(qd, cfg.block)
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, mask, mass = bsa.recap_topp_mask(desc, probs, p.tolist(), want_mask=True,
                                                 want_mass=True)
    out = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, s)
    out_e = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, s, residual=rd,
                                        res_scale=c.tolist())
    od = bsa.recap_dense_attn(desc, qd, kd, vd, s)
    od2, rcap = bsa.recap_dense_attn(desc, qd, kd, vd, s, count, idx, capture=True)
    # row statistics: the same kernels with extra writes, so outputs must agree bit for bit
    out_st, lse_s = bsa.recap_block_sparse_attn_stats(desc, qd, kd, vd, count, idx, s)
    st_d = bsa.recap_dense_attn_stats(desc, qd, kd, vd, s)
    st_k = bsa.recap_dense_attn_stats(desc, qd, kd, vd, s, count, idx, want_kept_mass=True)
    st_c = bsa.recap_dense_attn_stats(desc, qd, kd, vd, s, count, idx, capture=True,
                                      want_kept_mass=True)
    torch.cuda.synchronize()
    assert torch.equal(out_st, out) and torch.equal(st_d["out"], od)
    assert torch.equal(st_k["out"], od2) and st_k["residual"] is None
    assert torch.equal(st_c["out"], od2) and torch.equal(st_c["residual"], rcap)
    assert torch.equal(st_k["kept_mass"], st_c["kept_mass"])
    assert torch.equal(st_k["lse"], st_c["lse"])

    q64, k64, v64, r64 = (synth.to_f64(x) for x in (q, k, v, r))
    ref_probs = O.block_scores(q64, k64, cfg.block, s)
    parity.check_probs(probs.cpu().numpy().astype(np.float64), ref_probs)
    sel = O.topp_select(ref_probs, p)
    gmask = mask.cpu().numpy().astype(bool)
    cnt, ix = count.cpu().numpy(), idx.cpu().numpy()
    parity.check_lists(cnt, ix, M, gmask)
    assert np.array_equal(O.mask_from_lists(cnt, ix, M), gmask)
    parity.check_mask(gmask, ref_probs, sel["mask"], p)
    gm = mass.cpu().numpy().astype(np.float64)
    assert np.abs(gm - (ref_probs * gmask).sum(-1)).max() <= 2e-5
    ref_s = O.masked_attention(q64, k64, v64, cfg.block, s, gmask)
    parity.check_out(f64(out), ref_s, "sparse")
    parity.check_out(f64(out_e), O.residual_epilogue(ref_s, r64, c), "sparse + epilogue")
    ref_d = O.dense_attention(q64, k64, v64, s, block=cfg.block)
    parity.check_out(f64(od), ref_d, "dense")
    parity.check_out(f64(od2), ref_d, "dense (capture pass)")
    parity.check_captured(ref_s, f64(rcap), ref_d)
    lse_d_ref = O.attention_lse(q64, k64, cfg.block, s)
    parity.check_row_stat(lse_s.cpu().numpy(), O.attention_lse(q64, k64, cfg.block, s, gmask),
                          "sparse lse")
    parity.check_row_stat(st_d["lse"].cpu().numpy(), lse_d_ref, "dense lse")
    parity.check_row_stat(st_c["lse"].cpu().numpy(), lse_d_ref, "dense lse (capture pass)")
    parity.check_row_stat(st_c["kept_mass"].cpu().numpy(),
                          O.kept_attention_mass(q64, k64, cfg.block, s, gmask), "kept mass")
    return dict(count=cnt, M=M, desc=desc, dev=(qd, kd, vd, rd), p=p, s=s)


SMALL = {
    "tiny": dict(name="tiny"),
    "ragged_d128_b64_bnhd": dict(name="tiny", batch=2, heads=3, head_dim=128, seq=1000,
                                 layout="bnhd", top_p=[0.5, 0.9, 0.99]),
    "ragged_d128_b128": dict(name="tiny", heads=2, head_dim=128, block=128, seq=1500),
    "b128_short_last_block": dict(name="tiny", heads=2, head_dim=128, block=128, seq=128 * 5 + 20),
    "d64_b128": dict(name="tiny", heads=2, head_dim=64, block=128, seq=2000),
    "single_partial_block": dict(name="tiny", heads=2, head_dim=128, seq=37),
    "one_token_last_block": dict(name="tiny", heads=1, head_dim=64, seq=129),
    "p_one_is_dense": dict(name="tiny", heads=2, head_dim=128, seq=700, top_p=1.0),
    "p_zero_one_block": dict(name="tiny", heads=2, head_dim=64, seq=900, top_p=0.0),
    # several 32-row score tiles with a ragged last one (46 and 33 query blocks)
    "score_tiles_ragged_46": dict(name="tiny", heads=2, head_dim=64, seq=64 * 45 + 10),
    "score_tiles_ragged_33": dict(name="tiny", heads=1, head_dim=128, seq=64 * 32 + 5),
    # the head limit of the C ABI (per-head p and c arrays of 128)
    "max_heads_128": dict(name="tiny", heads=128, head_dim=64, seq=300),
}


@pytest.mark.parametrize("case", list(SMALL))
def test_small_case(bsa, case):
    kw = dict(SMALL[case])
    name = kw.pop("name")
    seq = kw.pop("seq", None)
    layout = kw.pop("layout", "bhnd")
    top_p = kw.pop("top_p", None)
    grid = synth.WORKLOADS[name].grid
    if seq is not None:
        grid = (1, 1, seq)
    cfg = synth.workload(name, grid=grid, **kw)
    say(f"[test] {case}")
    res = run_small(bsa, cfg, layout=layout, top_p=top_p)
    if top_p == 1.0:
        assert np.all(res["count"] == res["M"])
    if top_p == 0.0:
        assert np.all(res["count"] == 1)


@pytest.mark.parametrize("m,d", [(1264, 128), (1265, 64), (2100, 128)])
def test_scores_and_topp_long_rows(bsa, m, d):
    """Block scores and top-p for rows around the single-pass (LDS-resident row) limit of the
    score kernel (M <= 1264) and past the register-resident top-p limit (M > 2048)."""
    cfg = synth.workload("tiny", heads=1, head_dim=d)
    N = m * cfg.block - 7  # ragged last block
    q, k, _ = synth.make_qkv(cfg, seq=N)
    s = d ** -0.5
    p = np.array([0.9])
    say(f"[case] scores+topp M={m} D={d} N={N}")
    qd, kd = to_dev(q), to_dev(k)
    desc = bsa.make_desc(qd, cfg.block)
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, mask, _ = bsa.recap_topp_mask(desc, probs, p.tolist(), want_mask=True)
    torch.cuda.synchronize()
    ref = O.block_scores(synth.to_f64(q), synth.to_f64(k), cfg.block, s)
    parity.check_probs(probs.cpu().numpy().astype(np.float64), ref)
    gmask = mask.cpu().numpy().astype(bool)
    parity.check_lists(count.cpu().numpy(), idx.cpu().numpy(), m, gmask)
    parity.check_mask(gmask, ref, O.topp_select(ref, p)["mask"], p)


def test_max_blocks_8192(bsa):
    """The block limit of the C ABI: M = 8192 key blocks (N = 524,285, ragged last block), so
    the two-pass score kernel and the LDS-sort top-p run at their largest sizes. Checked on
    sampled query blocks: probabilities, kept sets, and sparse attention rows."""
    cfg = synth.workload("tiny", heads=1, head_dim=64, grid=(1, 1, 8192 * 64 - 3))
    M, s, p = 8192, 64 ** -0.5, np.array([0.9])
    say(f"[case] max blocks M={M} N={cfg.seq}")
    q, k, v = synth.make_qkv(cfg)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    desc = bsa.make_desc(qd, cfg.block)
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, _, _ = bsa.recap_topp_mask(desc, probs, p.tolist())
    out = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, s)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 6, 8192)
    q64, k64, v64 = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    qb, kb = O.block_mean_pool(q64, cfg.block), O.block_mean_pool(k64, cfg.block)
    ref = O.softmax_rows(s * np.matmul(qb[:, :, rows], np.swapaxes(kb, -1, -2)))
    got = probs[:, :, rows].cpu().numpy().astype(np.float64)
    parity.check_probs(got, ref)
    cnt = count[:, :, rows].cpu().numpy()
    ix = idx[:, :, rows].cpu().numpy()
    gmask = np.zeros((1, 1, len(rows), M), bool)
    for r in range(len(rows)):
        gmask[0, 0, r, ix[0, 0, r, :cnt[0, 0, r]]] = True
    parity.check_lists(cnt, ix, M, gmask)
    parity.check_mask(gmask, ref, O.topp_select(ref, p)["mask"], p)
    full = np.zeros((1, 1, M, M), bool)
    full[0, 0, rows] = gmask[0, 0]
    att = O.masked_attention(q64, k64, v64, cfg.block, s, full,
                             rows=[(0, 0, i) for i in rows[:3]])
    o64 = f64(out)
    for i in rows[:3]:
        lo, hi = i * cfg.block, min(cfg.seq, (i + 1) * cfg.block)
        parity.check_out(o64[:, :, lo:hi], att[:, :, lo:hi], f"max-blocks block {i}")


def test_graph_capture_replays(bsa):
    """A refresh plus a corrected sparse step recorded in one HIP graph (the library allocates
    nothing and never synchronises), replayed several times with eager work and new inputs in
    between; every replay must equal the eager result bit for bit."""
    cfg = synth.workload("tiny", heads=2, head_dim=128, grid=(1, 1, 3000))
    s = cfg.head_dim ** -0.5
    q, k, v = synth.make_qkv(cfg)
    p, c = [0.9, 0.8], [1.0, 0.5]
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    q1d, k1d, v1d = (to_dev(synth.drifted(x, n, 1)) for x, n in ((q, "q"), (k, "k"), (v, "v")))
    desc = bsa.make_desc(qd, cfg.block)
    M = cfg.num_blocks
    probs = torch.empty((1, 2, M, M), dtype=torch.float32, device=DEV)
    cnt0, cnt1 = (torch.empty((1, 2, M), dtype=torch.int32, device=DEV) for _ in range(2))
    idx0, idx1 = (torch.empty((1, 2, M, M), dtype=torch.int32, device=DEV) for _ in range(2))
    od, rcap, out = (torch.empty_like(qd) for _ in range(3))
    ws = {op: torch.empty(max(1, bsa.recap_workspace_size(op, desc)), dtype=torch.uint8,
                          device=DEV) for op in (0, 2, 4)}

    def step():
        bsa.recap_block_scores(desc, qd, kd, s, probs=probs, workspace=ws[0])
        bsa.recap_topp_mask(desc, probs, p, kept_count=cnt0, kept_idx=idx0)
        bsa.recap_dense_attn(desc, qd, kd, vd, s, cnt0, idx0, out=od, residual_out=rcap,
                             workspace=ws[4])
        bsa.recap_block_scores(desc, q1d, k1d, s, probs=probs, workspace=ws[0])
        bsa.recap_topp_mask(desc, probs, p, kept_count=cnt1, kept_idx=idx1)
        bsa.recap_block_sparse_attn(desc, q1d, k1d, v1d, cnt1, idx1, s, residual=rcap,
                                    res_scale=c, out=out, workspace=ws[2])

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager on the side stream first (no first-use work inside the capture)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (od, rcap, out, cnt1)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in (od, rcap, out):
            t.fill_(float("nan"))  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((od, rcap, out, cnt1), eager):
            assert torch.equal(a, b), f"replay {rep}"
    # new inputs of the same shape flow through the recorded graph
    qd.copy_(to_dev(synth.drifted(q, "q", 2)))
    g.replay()
    torch.cuda.synchronize()
    replayed = out.clone()
    step()
    torch.cuda.synchronize()
    assert torch.equal(replayed, out)
    assert not torch.equal(replayed, eager[2])


def test_graph_capture_replays_tail_and_fp8(bsa):
    """RECAP's tail calls (coarse estimate, refresh with discrepancy, sparse call with tail
    merge) and the FP8 sparse call (with its packers, epilogue and lse) recorded in one HIP
    graph and replayed several times with eager work in between; every replay must equal the
    eager result bit for bit, and new inputs must flow through the recorded graph."""
    cfg = synth.workload("tiny", heads=2, head_dim=128, grid=(1, 1, 2100))
    s = cfg.head_dim ** -0.5
    q, k, v = synth.make_qkv(cfg)
    r = synth.make_residual(cfg)
    p, c = [0.9, 0.8], [1.0, 0.5]
    qd, kd, vd, rd = to_dev(q), to_dev(k), to_dev(v), to_dev(r)
    q1d, k1d, v1d = (to_dev(synth.drifted(x, n, 1)) for x, n in ((q, "q"), (k, "k"), (v, "v")))
    desc = bsa.make_desc(qd, cfg.block)
    say(f"[case] graph replay, tail + fp8: N={cfg.seq} M={cfg.num_blocks}")
    M = cfg.num_blocks
    probs = torch.empty((1, 2, M, M), dtype=torch.float32, device=DEV)
    cnt0, cnt1 = (torch.empty((1, 2, M), dtype=torch.int32, device=DEV) for _ in range(2))
    idx0, idx1 = (torch.empty((1, 2, M, M), dtype=torch.int32, device=DEV) for _ in range(2))
    od, ot, o8 = (torch.empty_like(qd) for _ in range(3))
    rows = lambda *tail: torch.empty((1, 2, cfg.seq) + tail, dtype=torch.float32, device=DEV)  # noqa: E731
    dlse, dout, tlse, tout, lse8 = rows(), rows(128), rows(), rows(128), rows()
    ws = {op: torch.empty(max(1, bsa.recap_workspace_size(op, desc)), dtype=torch.uint8,
                          device=DEV) for op in (0, 5, 6, 7, 8)}

    def step():
        bsa.recap_block_scores(desc, qd, kd, s, probs=probs, workspace=ws[0])
        bsa.recap_topp_mask(desc, probs, p, kept_count=cnt0, kept_idx=idx0)
        bsa.recap_dense_attn_tail(desc, qd, kd, vd, cnt0, idx0, s, out=od, tail_dlse=dlse,
                                  tail_dout=dout, workspace=ws[6])
        bsa.recap_block_scores(desc, q1d, k1d, s, probs=probs, workspace=ws[0])
        bsa.recap_topp_mask(desc, probs, p, kept_count=cnt1, kept_idx=idx1)
        bsa.recap_tail_estimate(desc, q1d, k1d, v1d, cnt1, idx1, s, tail_lse=tlse,
                                tail_out=tout, workspace=ws[5], moments=True)
        bsa.recap_block_sparse_attn_tail(desc, q1d, k1d, v1d, cnt1, idx1, s, tail_dlse=dlse,
                                         tail_dout=dout, out=ot, workspace=ws[7])
        bsa.recap_block_sparse_attn_fp8(desc, q1d, k1d, v1d, cnt1, idx1, s, residual=rd,
                                        res_scale=c, out=o8, workspace=ws[8], lse=lse8)

    results = (od, dlse, dout, tlse, tout, ot, o8, lse8)
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager on the side stream first (no first-use work inside the capture)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in results]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in results:
            t.fill_(float("nan"))  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(results, eager)):
            assert torch.equal(a, b), f"replay {rep}, result {i}"
    q1d.copy_(to_dev(synth.drifted(q, "q", 2)))
    g.replay()
    torch.cuda.synchronize()
    replayed = [t.clone() for t in (ot, o8)]
    step()
    torch.cuda.synchronize()
    assert torch.equal(replayed[0], ot) and torch.equal(replayed[1], o8)
    assert not torch.equal(replayed[0], eager[5]) and not torch.equal(replayed[1], eager[6])


def _to_blocks(vals, count, idx, m):
    """Candidate-position values -> block space (zeros outside each row's candidates)."""
    out = np.zeros(vals.shape[:-1] + (m,))
    for b, h, i in np.ndindex(*count.shape):
        n = count[b, h, i]
        out[b, h, i, idx[b, h, i, :n]] = vals[b, h, i, :n]
    return out


@pytest.mark.parametrize("m,d", [(300, 128), (2100, 64)])
def test_mask_reuse(bsa, m, d):
    """Mask-reuse building blocks against the oracle: block means; scores from means (equal
    bit for bit to recap_block_scores); scores and top-p restricted to candidate lists (the
    wavefront top-p for M <= 2048, the LDS sort beyond); a row with no candidates; drift of
    the means between two steps."""
    cfg = synth.workload("tiny", heads=2, head_dim=d, grid=(1, 1, m * 64 - 5))
    s, M = d ** -0.5, m
    say(f"[case] mask reuse M={M} D={d}")
    q, k, _ = synth.make_qkv(cfg)
    qd, kd = to_dev(q), to_dev(k)
    desc = bsa.make_desc(qd, cfg.block)
    qbar, kbar = bsa.recap_block_means(desc, qd, kd)
    full = bsa.recap_scores_from_means(desc, qbar, kbar, s)
    via_scores = bsa.recap_block_scores(desc, qd, kd, s)
    cc, ci, _, _ = bsa.recap_topp_mask(desc, full, [0.99, 0.97])
    pc = bsa.recap_scores_from_means(desc, qbar, kbar, s, cc, ci)
    p = np.array([0.9, 0.8])
    kc, ki, km, kmass = bsa.recap_topp_mask_cand(desc, pc, cc, ci, p.tolist(), want_mask=True,
                                                 want_mass=True)
    torch.cuda.synchronize()
    assert torch.equal(full, via_scores)
    q64, k64 = synth.to_f64(q), synth.to_f64(k)
    qb, kb = O.block_mean_pool(q64, cfg.block), O.block_mean_pool(k64, cfg.block)
    # fp32 sums of up to 64 bf16 values of magnitude <~ 8: error <= 64 * 2^-24 * 8 < 4e-5
    assert np.abs(qbar.cpu().numpy() - qb).max() < 4e-5
    assert np.abs(kbar.cpu().numpy() - kb).max() < 4e-5
    cnt, idx = cc.cpu().numpy(), ci.cpu().numpy()
    cand = O.mask_from_lists(cnt, idx, M)
    assert cand.sum() < cand.size  # a real restriction
    ref_c = O.candidate_scores(q64, k64, cfg.block, s, cand)
    parity.check_probs(_to_blocks(pc.cpu().numpy().astype(np.float64), cnt, idx, M), ref_c)
    ref_sel = O.topp_select_candidates(ref_c, cand, p)
    gmask = km.cpu().numpy().astype(bool)
    assert not (gmask & ~cand).any(), "kept blocks must be candidates"
    parity.check_lists(kc.cpu().numpy(), ki.cpu().numpy(), M, gmask)
    parity.check_mask(gmask, ref_c, ref_sel["mask"], p)
    assert np.abs(kmass.cpu().numpy() - (ref_c * gmask).sum(-1)).max() <= 2e-5
    # a row without candidates keeps nothing; the other rows are unchanged
    cc2 = cc.clone()
    cc2[0, 1, 3] = 0
    kc2, ki2, _, _ = bsa.recap_topp_mask_cand(desc, pc, cc2, ci, p.tolist())
    torch.cuda.synchronize()
    assert int(kc2[0, 1, 3]) == 0
    kc2[0, 1, 3] = kc[0, 1, 3]
    assert torch.equal(kc2, kc)
    # drift of the block means against a reference step
    q2, k2 = synth.drifted(q, "q", 1), synth.drifted(k, "k", 1)
    qbar2, kbar2 = bsa.recap_block_means(desc, to_dev(q2), to_dev(k2))
    dr = bsa.recap_mean_drift(desc, qbar2, kbar2, qbar, kbar)
    dr0 = bsa.recap_mean_drift(desc, qbar, kbar, qbar, kbar)
    torch.cuda.synchronize()
    assert torch.all(dr0 == 0)
    ref_dr = O.mean_drift(O.block_mean_pool(synth.to_f64(q2), cfg.block),
                          O.block_mean_pool(synth.to_f64(k2), cfg.block), qb, kb)
    got_dr = dr.cpu().numpy().astype(np.float64)
    assert np.all(ref_dr > 0) and np.abs(got_dr / ref_dr - 1).max() < 1e-3, (got_dr, ref_dr)


def test_all_kept_capture_is_exactly_zero(bsa):
    say("[test] all-kept capture")
    cfg = synth.workload("tiny", head_dim=128, grid=(1, 1, 1100))
    q, k, v = synth.make_qkv(cfg)
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    desc = bsa.make_desc(qd, cfg.block)
    M = cfg.num_blocks
    count = torch.full((1, cfg.heads, M), M, dtype=torch.int32, device=DEV)
    idx = torch.arange(M, dtype=torch.int32, device=DEV).expand(1, cfg.heads, M, M).contiguous()
    od, rcap = bsa.recap_dense_attn(desc, qd, kd, vd, None, count, idx, capture=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(rcap).item() == 0
    out = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx)
    torch.cuda.synchronize()
    # the same attention in a different key order; each is within the parity bound of the
    # oracle (checked in the small cases), so they are within twice that bound of each other
    assert (out.float() - od.float()).abs().max().item() <= 2 * parity.ATOL_OUT


def test_capture_when_kept_mass_underflows(bsa):
    """A kept list that leaves out a key block whose logits exceed everything else by far more
    than fp32 range: the dense pass's shared-maximum accumulator for the kept blocks underflows,
    so the residual must come from the per-block fallback pass."""
    say("[test] capture fallback (kept mass underflow)")
    B, H, N, D, blk = 1, 1, 64 * 6, 64, 64
    g = torch.Generator().manual_seed(5)
    q = torch.ones((B, H, N, D))
    k = 0.1 * torch.randn((B, H, N, D), generator=g)
    k[:, :, :64] = 20.0  # block 0: logits ~ 160 (about 230 binary orders above the rest)
    v = torch.randn((B, H, N, D), generator=g)
    q, k, v = (x.to(torch.bfloat16) for x in (q, k, v))
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    desc = bsa.make_desc(qd, blk)
    M = N // blk
    count = torch.full((B, H, M), 2, dtype=torch.int32, device=DEV)
    idx = torch.zeros((B, H, M, M), dtype=torch.int32, device=DEV)
    idx[..., 0], idx[..., 1] = 2, 4  # kept: blocks 2 and 4 (block 0 left out)
    od, rcap = bsa.recap_dense_attn(desc, qd, kd, vd, None, count, idx, capture=True)
    torch.cuda.synchronize()
    q64, k64, v64 = (synth.to_f64(x) for x in (q, k, v))
    mask = np.zeros((B, H, M, M), bool)
    mask[..., [2, 4]] = True
    s = D ** -0.5
    ref_d = O.dense_attention(q64, k64, v64, s, block=blk)
    ref_s = O.masked_attention(q64, k64, v64, blk, s, mask)
    parity.check_out(f64(od), ref_d, "dense")
    parity.check_out(f64(rcap), ref_d - ref_s, "residual")


@pytest.mark.parametrize("m", [16, 100, 700, 1182, 2000, 2100])
def test_topp_exact_ties(bsa, m):
    """Hand-made probability rows with exact ties (dyadic values, so every running mass is
    exact): the kept sets must equal the oracle's exactly, tie order included. Row lengths
    cover each register-resident variant and the sorting fallback for long rows."""
    say(f"[test] top-p exact ties, M={m}")
    H, rows = 2, []
    g = np.random.default_rng(m)
    for r in range(m):
        kind = r % 4
        row = np.zeros(m)
        if kind == 0:  # uniform
            row[:] = 1.0 / m
        elif kind == 1:  # a few equal large blocks at random places, the rest equal and small
            big = g.choice(m, size=min(4, m), replace=False)
            row[:] = 0.0
            row[big] = 0.125
            rest = np.setdiff1d(np.arange(m), big)
            row[rest] = 0.5 / len(rest)
        elif kind == 2:  # geometric with repeated pairs
            vals = 0.5 ** (1 + np.arange(m) // 2)
            row[g.permutation(m)] = vals
        else:  # one dominant block
            row[:] = 2.0 ** -20
            row[g.integers(m)] = 1.0 - (m - 1) * 2.0 ** -20
        rows.append(row.astype(np.float32))
    probs = np.stack(rows)[None, None].repeat(H, axis=1)  # [1, H, M, M]
    for p in ([0.0, 0.25], [0.5, 0.75], [0.9, 1.0], [0.3333, 0.999]):
        desc = bsa.RecapDesc(1, H, m * 64, 64, 64, 0, H * m * 64 * 64, m * 64 * 64, 64)
        pd = torch.from_numpy(probs).to(DEV)
        count, idx, mask, mass = bsa.recap_topp_mask(desc, pd, p, want_mask=True, want_mass=True)
        torch.cuda.synchronize()
        ref = O.topp_select(probs.astype(np.float64), np.array(p, dtype=np.float32).astype(np.float64))
        gm = mask.cpu().numpy().astype(bool)
        assert np.array_equal(gm, ref["mask"]), (p, np.argwhere((gm != ref["mask"]).any(-1))[:5])
        assert np.array_equal(count.cpu().numpy(), ref["count"])
        parity.check_lists(count.cpu().numpy(), idx.cpu().numpy(), m, gm)
        assert np.allclose(mass.cpu().numpy(), ref["mass"], rtol=1e-6, atol=1e-7)



@pytest.mark.parametrize("m", [100, 1182])
def test_topp_total_near_p(bsa, m):
    """Rows whose total lies within the fp32 sums' error bound of p, where the selection takes
    the total in fp64: 20 dyadic blocks 2^-1 .. 2^-20 at random places (total 1 - 2^-20, exact
    in fp32), the rest zero. p equal to the total keeps the 20 blocks; p 2^-21 above it keeps
    every block (no prefix reaches p); p 2^-20 below it keeps 19 (the running mass reaches p
    exactly one block early)."""
    say(f"[test] top-p with the row total near p, M={m}")
    H = 3
    g = np.random.default_rng(1000 + m)
    probs = np.zeros((1, H, m, m), dtype=np.float32)
    for h in range(H):
        for r in range(m):
            probs[0, h, r, g.choice(m, size=20, replace=False)] = 0.5 ** (1 + np.arange(20))
    p = [1.0 - 2.0 ** -20, 1.0 - 2.0 ** -21, 1.0 - 2.0 ** -19]
    desc = bsa.RecapDesc(1, H, m * 64, 64, 64, 0, H * m * 64 * 64, m * 64 * 64, 64)
    count, idx, mask, mass = bsa.recap_topp_mask(desc, torch.from_numpy(probs).to(DEV), p,
                                                 want_mask=True, want_mass=True)
    torch.cuda.synchronize()
    ref = O.topp_select(probs.astype(np.float64), np.array(p, dtype=np.float32).astype(np.float64))
    cnt = count.cpu().numpy()
    assert (cnt[0, 0] == 20).all() and (cnt[0, 1] == m).all() and (cnt[0, 2] == 19).all()
    gm = mask.cpu().numpy().astype(bool)
    assert np.array_equal(gm, ref["mask"])
    assert np.array_equal(cnt, ref["count"])
    parity.check_lists(cnt, idx.cpu().numpy(), m, gm)
    assert np.allclose(mass.cpu().numpy(), ref["mass"], rtol=1e-6, atol=1e-7)

def test_deterministic_poison_and_guards(bsa):
    say("[test] determinism, NaN poison, guard bands")
    cfg = synth.workload("tiny", heads=2, head_dim=128, grid=(1, 1, 1333))
    q, k, v = synth.make_qkv(cfg)
    r = synth.make_residual(cfg)
    qd, kd, vd, rd = (to_dev(x) for x in (q, k, v, r))
    desc = bsa.make_desc(qd, cfg.block)
    _, count, idx = bsa.sparse_step(desc, qd, kd, vd, [0.9, 0.8])
    guard = 1 << 14
    big = torch.full((qd.numel() + 2 * guard,), float("nan"), dtype=torch.bfloat16, device=DEV)
    big[:guard] = 7.0
    big[-guard:] = 7.0
    out = big[guard:guard + qd.numel()].view_as(qd)
    bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, None, rd, [0.5, 0.25], out=out)
    first = out.clone()
    bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, None, rd, [0.5, 0.25], out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    assert torch.equal(first, out)
    assert torch.all(big[:guard] == 7.0) and torch.all(big[-guard:] == 7.0)
    p1 = bsa.recap_block_scores(desc, qd, kd)
    p2 = bsa.recap_block_scores(desc, qd, kd)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2)


def test_sparse_grid_order_across_batches(bsa):
    """Paired sparse walks run the grid's last min(tiles, 1024) tiles in an order computed on the
    device from the kept counts. With B = 2 the grid has 2*4*151 = 1208 paired tiles, so the
    ordered group starts inside batch 0 and crosses into batch 1 (and ends on a pair with one
    query block, M = 301); each batch alone has 604 tiles, all ordered. The output of every
    query row depends only on its own lists, so both launches must agree bit for bit."""
    say("[test] sparse grid order: B=2 call against two B=1 calls")
    cfg = synth.workload("tiny", batch=2, heads=4, head_dim=64, grid=(1, 1, 19240))
    q, k, v = synth.make_qkv(cfg)
    r = synth.make_residual(cfg)
    qd, kd, vd, rd = (to_dev(x) for x in (q, k, v, r))
    desc = bsa.make_desc(qd, cfg.block)
    assert -(-cfg.seq // cfg.block) == 301
    p = [0.9, 0.8, 0.95, 0.7]
    c = [0.5, 1.0, 0.25, 0.0]
    _, count, idx = bsa.sparse_step(desc, qd, kd, vd, p)
    out = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, None, rd, c)
    lens = count.sum(dim=-1)
    assert int(lens.min()) < int(lens.max())  # unequal walks: the order matters
    for b in range(2):
        sl = slice(b, b + 1)
        d1 = bsa.make_desc(qd[sl], cfg.block)
        o1 = bsa.recap_block_sparse_attn(d1, qd[sl], kd[sl], vd[sl], count[sl].contiguous(),
                                         idx[sl].contiguous(), None, rd[sl], c)
        torch.cuda.synchronize()
        assert torch.equal(o1[0], out[b]), f"batch {b} differs"


# ------------------------------------------------------------------------- full-size workloads
def _sample_rows(m, n, seed):
    g = np.random.default_rng(seed)
    rows = {0, m - 1} | set(g.choice(m, size=min(n, m), replace=False).tolist())
    return sorted(rows)


def _check_head(probs_g, mask_g, cnt_g, idx_g, q64, k64, v64, cfg, p_h, s, rows, h,
                out_g=None, extra=None):
    """Oracle checks for one head: full probs and mask rows of the head, attention rows."""
    ref_probs = O.block_scores(q64, k64, cfg.block, s)
    parity.check_probs(probs_g, ref_probs)
    sel = O.topp_select(ref_probs, p_h)
    parity.check_lists(cnt_g, idx_g, cfg.num_blocks, mask_g)
    parity.check_mask(mask_g, ref_probs, sel["mask"], p_h)
    if out_g is not None:
        ref = O.masked_attention(q64, k64, v64, cfg.block, s, mask_g, rows=[(0, 0, i) for i in rows])
        if extra is not None:
            ref = extra(ref)
        for i in rows:
            lo, hi = i * cfg.block, min(cfg.seq, (i + 1) * cfg.block)
            parity.check_out(out_g[:, :, lo:hi], ref[:, :, lo:hi], f"head {h} block {i}")
        if len(rows) == cfg.num_blocks:
            parity.check_out(out_g, ref, f"head {h} whole")


def _head(x, h):
    return synth.to_f64(x[:, h:h + 1])


@pytest.mark.parametrize("name,heads", [("wan13b_480p", [0, 11]), ("wan14b_480p", [0, 17, 39]),
                                        ("hunyuan_720p", [0, 23])])
def test_full_size_sparse(bsa, name, heads):
    cfg = synth.WORKLOADS[name]
    say(f"[test] full-size {name}: generating inputs")
    q, k, v = synth.make_qkv(cfg)
    p, c = synth.head_params(cfg)
    s = cfg.head_dim ** -0.5
    r = synth.make_residual(cfg) if cfg.residual else None
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    rd = to_dev(r) if r is not None else None
    desc = bsa.make_desc(qd, cfg.block)
    say(f"[gpu] {name}: scores, top-p, sparse attention")
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, mask, _ = bsa.recap_topp_mask(desc, probs, p.tolist(), want_mask=True)
    out = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, idx, s, rd,
                                      c.tolist() if rd is not None else None)
    torch.cuda.synchronize()
    say(f"[check] {name}: oracle on every query block of heads {heads}")
    for h in heads:
        rows = list(range(cfg.num_blocks))
        extra = None
        if r is not None:
            r64 = _head(r, h)
            extra = lambda ref, r64=r64, ch=c[h]: O.residual_epilogue(ref, r64, [ch])
        _check_head(probs[:, h:h + 1].cpu().numpy().astype(np.float64),
                    mask[:, h:h + 1].cpu().numpy().astype(bool),
                    count[:, h:h + 1].cpu().numpy(), idx[:, h:h + 1].cpu().numpy(),
                    _head(q, h), _head(k, h), _head(v, h), cfg, p[h:h + 1], s, rows, h,
                    out_g=f64(out[:, h:h + 1]), extra=extra)


@pytest.mark.parametrize("name,heads", [("wan14b_720p", [0, 21]), ("hunyuan_720p", [0, 23])])
def test_full_size_mask_reuse(bsa, name, heads):
    """Mask reuse at the full workloads, as the benchmark's reuse leg runs it: block means at a
    reference step X_0 and the drifted step X_1 and their drift, candidate lists from X_0 at the
    looser threshold 1 - (1 - p) / 4, scores from X_1's means over the candidates and top-p at p
    over each row's candidate distribution; each against the oracle on whole heads."""
    cfg = synth.WORKLOADS[name]
    say(f"[test] full-size mask reuse {name}: generating inputs")
    q0, k0, _ = synth.make_qkv(cfg)
    q1, k1 = synth.drifted(q0, "q", 1), synth.drifted(k0, "k", 1)
    p, _ = synth.head_params(cfg)
    pc = np.minimum(1.0, 1.0 - (1.0 - p) / 4.0)
    s, M = cfg.head_dim ** -0.5, cfg.num_blocks
    q0d, k0d, q1d, k1d = (to_dev(x) for x in (q0, k0, q1, k1))
    desc = bsa.make_desc(q0d, cfg.block)
    say(f"[gpu] {name}: means, candidates at X_0, drift, restricted scores and top-p at X_1")
    qb0, kb0 = bsa.recap_block_means(desc, q0d, k0d)
    pr0 = bsa.recap_scores_from_means(desc, qb0, kb0, s)
    cc, ci, cmask, _ = bsa.recap_topp_mask(desc, pr0, pc.tolist(), want_mask=True)
    qb1, kb1 = bsa.recap_block_means(desc, q1d, k1d)
    dr = bsa.recap_mean_drift(desc, qb1, kb1, qb0, kb0)
    pr1 = bsa.recap_scores_from_means(desc, qb1, kb1, s, cc, ci)
    kc, ki, km, kmass = bsa.recap_topp_mask_cand(desc, pr1, cc, ci, p.tolist(), want_mask=True,
                                                 want_mass=True)
    torch.cuda.synchronize()
    say(f"[check] {name}: oracle on every query block of heads {heads}")
    for h in heads:
        q064, k064, q164, k164 = (_head(x, h) for x in (q0, k0, q1, k1))
        means0 = O.block_mean_pool(q064, cfg.block), O.block_mean_pool(k064, cfg.block)
        means1 = O.block_mean_pool(q164, cfg.block), O.block_mean_pool(k164, cfg.block)
        # fp32 sums of at most `block` bf16 values: each mean within block * 2^-24 * max|x|
        for got, ref, x in ((qb1, means1[0], q164), (kb1, means1[1], k164)):
            tol = cfg.block * 2.0 ** -24 * np.abs(x).max()
            assert np.abs(got[:, h:h + 1].cpu().numpy() - ref).max() <= tol, (name, h)
        ref_dr = O.mean_drift(*means1, *means0)
        got_dr = dr[:, h:h + 1].cpu().numpy().astype(np.float64)
        assert np.all(ref_dr > 0) and np.abs(got_dr / ref_dr - 1).max() < 1e-3, (got_dr, ref_dr)
        # candidate lists at X_0: the mask rule at the looser threshold
        ref0 = O.block_scores(q064, k064, cfg.block, s)
        parity.check_probs(pr0[:, h:h + 1].cpu().numpy().astype(np.float64), ref0)
        c_m = cmask[:, h:h + 1].cpu().numpy().astype(bool)
        cnt, idx = cc[:, h:h + 1].cpu().numpy(), ci[:, h:h + 1].cpu().numpy()
        parity.check_lists(cnt, idx, M, c_m)
        parity.check_mask(c_m, ref0, O.topp_select(ref0, pc[h:h + 1])["mask"], pc[h:h + 1])
        # X_1: scores over the GPU's candidate lists and top-p over them
        cand = O.mask_from_lists(cnt, idx, M)
        ref_c = O.candidate_scores(q164, k164, cfg.block, s, cand)
        parity.check_probs(_to_blocks(pr1[:, h:h + 1].cpu().numpy().astype(np.float64), cnt,
                                      idx, M), ref_c)
        gmask = km[:, h:h + 1].cpu().numpy().astype(bool)
        assert not (gmask & ~cand).any(), "kept blocks must be candidates"
        parity.check_lists(kc[:, h:h + 1].cpu().numpy(), ki[:, h:h + 1].cpu().numpy(), M, gmask)
        parity.check_mask(gmask, ref_c, O.topp_select_candidates(ref_c, cand, p[h:h + 1])["mask"],
                          p[h:h + 1])
        assert np.abs(kmass[:, h:h + 1].cpu().numpy() - (ref_c * gmask).sum(-1)).max() <= 2e-5


def test_full_size_refresh_then_sparse(bsa):
    """Wan2.1-14B 720p layer: dense refresh with residual capture, then a drifted sparse step
    that reuses the captured residual at scale 1."""
    cfg = synth.WORKLOADS["wan14b_720p"]
    heads = [0, 21]
    say("[test] full-size wan14b_720p: generating inputs")
    q, k, v = synth.make_qkv(cfg)
    p, c = synth.head_params(cfg)
    s = cfg.head_dim ** -0.5
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    desc = bsa.make_desc(qd, cfg.block)
    say("[gpu] wan14b_720p: refresh (scores, top-p, dense + capture)")
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, mask, _ = bsa.recap_topp_mask(desc, probs, p.tolist(), want_mask=True)
    st = bsa.recap_dense_attn_stats(desc, qd, kd, vd, s, count, idx, capture=True,
                                    want_kept_mass=True)
    od, rcap = st["out"], st["residual"]
    torch.cuda.synchronize()
    say("[check] refresh rows")
    for h in heads:
        rows = _sample_rows(cfg.num_blocks, 3, 100 + h)
        q64, k64, v64 = _head(q, h), _head(k, h), _head(v, h)
        m_h = mask[:, h:h + 1].cpu().numpy().astype(bool)
        _check_head(probs[:, h:h + 1].cpu().numpy().astype(np.float64), m_h,
                    count[:, h:h + 1].cpu().numpy(), idx[:, h:h + 1].cpu().numpy(),
                    q64, k64, v64, cfg, p[h:h + 1], s, rows, h)
        sel = [(0, 0, i) for i in rows]
        ref_d = O.dense_attention(q64, k64, v64, s, rows=sel, block=cfg.block)
        ref_s = O.masked_attention(q64, k64, v64, cfg.block, s, m_h, rows=sel)
        od_h, r_h = f64(od[:, h:h + 1]), f64(rcap[:, h:h + 1])
        parity.check_row_stat(st["lse"][:, h:h + 1].cpu().numpy(),
                              O.attention_lse(q64, k64, cfg.block, s, rows=sel),
                              f"dense lse h{h}")
        parity.check_row_stat(st["kept_mass"][:, h:h + 1].cpu().numpy(),
                              O.kept_attention_mass(q64, k64, cfg.block, s, m_h, rows=sel),
                              f"kept mass h{h}")
        for i in rows:
            lo, hi = i * cfg.block, min(cfg.seq, (i + 1) * cfg.block)
            parity.check_out(od_h[:, :, lo:hi], ref_d[:, :, lo:hi], f"dense h{h} b{i}")
            parity.check_out(ref_s[:, :, lo:hi] + r_h[:, :, lo:hi], ref_d[:, :, lo:hi],
                             f"capture identity h{h} b{i}")
    del od, st
    say("[gpu] wan14b_720p: drifted sparse step 1 with the captured residual")
    q1, k1, v1 = synth.drifted(q, "q", 1), synth.drifted(k, "k", 1), synth.drifted(v, "v", 1)
    q1d, k1d, v1d = (to_dev(x) for x in (q1, k1, v1))
    out, count1, idx1 = bsa.sparse_step(desc, q1d, k1d, v1d, p.tolist(), s, residual=rcap,
                                        res_scale=c.tolist())
    # the statistics entry point on the same lists: the same output bit for bit, plus the
    # log-sum-exp over each query's kept keys
    out_st, lse1 = bsa.recap_block_sparse_attn_stats(desc, q1d, k1d, v1d, count1, idx1, s,
                                                     rcap, c.tolist())
    torch.cuda.synchronize()
    assert torch.equal(out_st, out)
    del out_st
    say(f"[check] drifted step 1: oracle on every query block of heads {heads}")
    for h in heads:
        rows = list(range(cfg.num_blocks))
        m_h = O.mask_from_lists(count1[:, h:h + 1].cpu().numpy(), idx1[:, h:h + 1].cpu().numpy(),
                                cfg.num_blocks)
        q64, k64, v64 = _head(q1, h), _head(k1, h), _head(v1, h)
        ref = O.masked_attention(q64, k64, v64, cfg.block, s, m_h, rows=[(0, 0, i) for i in rows])
        ref = O.residual_epilogue(ref, f64(rcap[:, h:h + 1]), [c[h]])
        got = f64(out[:, h:h + 1])
        for i in rows:
            lo, hi = i * cfg.block, min(cfg.seq, (i + 1) * cfg.block)
            parity.check_out(got[:, :, lo:hi], ref[:, :, lo:hi], f"step1 h{h} b{i}")
        parity.check_out(got, ref, f"step1 h{h} whole head")
        sel = [(0, 0, i) for i in _sample_rows(cfg.num_blocks, 6, 200 + h)]
        parity.check_row_stat(lse1[:, h:h + 1].cpu().numpy(),
                              O.attention_lse(q64, k64, cfg.block, s, mask=m_h, rows=sel),
                              f"sparse lse step1 h{h}")
