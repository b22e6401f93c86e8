"""FP8 (MXFP8) variant of the block-sparse attention on the GPU against the CPU oracle.

* The encoder (recap_mx_quantize) is byte work: its codes and scales must equal the oracle's
  MXFP8 quantisation exactly, for blocks along the head dimension and along the tokens.
* The attention (recap_block_sparse_attn_fp8) is compared with the oracle's attention on the
  quantised Q, K, V (oracle.masked_attention_mx, the same quantisation the kernel applies); the
  remaining difference is the E4M3 rounding of the attention weights inside the kernel, bounded
  per element and in relative L2 by parity.fp8_weight_bounds / check_fp8_out. The log-sum-exp
  sums rounded weights: within ln(1 + 2^-4) plus the row-statistics bound.
"""
import math

import numpy as np
import pytest
import torch

import parity
import synth
from gpu_common import DEV, bsa, f64, say, to_dev  # noqa: F401
from oracle import brute
from oracle import oracle as O

pytestmark = pytest.mark.gpu

_E4M3 = np.array([brute.e4m3_value(c) for c in range(256)])


def _decode(codes, scales, along_tokens):
    """Values the GPU's codes and scales stand for (E4M3 value times 2^(scale - 127))."""
    val = _E4M3[codes.astype(np.int64)]
    e = scales.astype(np.float64) - 127.0
    if along_tokens:
        N = codes.shape[2]
        e = np.repeat(e, 32, axis=2)[:, :, :N, :]
    else:
        e = np.repeat(e, 32, axis=3)
    return val * np.exp2(e)


def _edge_tensor(B, H, N, D, seed):
    """bf16 values over many binades, with an all-zero 32-block, tiny and large blocks."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((B, H, N, D), generator=g) * torch.exp2(torch.randint(-6, 7, (B, H, N, 1), generator=g).float())
    x[0, 0, 0, :32] = 0.0
    x[0, 0, 1, :] *= 1e-30
    x[0, 0, 2, :] *= 1e30
    x[0, 0, 3, 5] = 1e-38
    return x.to(torch.bfloat16)


@pytest.mark.parametrize("N,D", [(1000, 128), (77, 64), (64, 128)])
def test_mx_quantize_bitexact(bsa, N, D):
    say(f"[test] mx_quantize N={N} D={D}")
    x = _edge_tensor(2, 3, N, D, 600 + N)
    for layout in ("bhnd", "bnhd"):
        xd = to_dev(x, layout)
        desc = bsa.make_desc(xd, 64)
        for along in (False, True):
            codes, scales = bsa.recap_mx_quantize(desc, xd, along_tokens=along)
            torch.cuda.synchronize()
            axis = 2 if along else 3
            x64 = synth.to_f64(x)
            want_e = O.mx_scale_exponents(x64, axis=axis)
            got_e = scales.cpu().numpy().astype(np.float64) - 127.0
            if along:
                want_e = np.moveaxis(want_e, -1, 2)
            assert np.array_equal(got_e, want_e), (layout, along)
            got = _decode(codes.cpu().numpy(), scales.cpu().numpy(), along)
            want = O.mx_quantize(x64, axis=axis)
            assert np.array_equal(got, want), (layout, along, np.abs(got - want).max())


def run_fp8(bsa, cfg, layout="bhnd", top_p=None, residual=False):
    q, k, v = synth.make_qkv(cfg)
    N = q.shape[2]
    M = -(-N // cfg.block)
    p_def, c_def = synth.head_params(cfg)
    p = p_def if top_p is None else np.broadcast_to(np.asarray(top_p, float), (cfg.heads,))
    s = cfg.head_dim ** -0.5
    say(f"[case] fp8 B={cfg.batch} H={cfg.heads} D={cfg.head_dim} N={N} block={cfg.block} "
        f"layout={layout} p={np.round(p, 3).tolist()} residual={residual}")
    qd, kd, vd = (to_dev(x, layout) for x in (q, k, v))
    desc = bsa.make_desc(qd, cfg.block)
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, _, _ = bsa.recap_topp_mask(desc, probs, p.tolist())
    out, lse = bsa.recap_block_sparse_attn_fp8(desc, qd, kd, vd, count, idx, s, want_lse=True)
    r = c = None
    if residual:
        r = synth.make_residual(cfg)
        c = np.full(cfg.heads, 0.75)
        out_e = bsa.recap_block_sparse_attn_fp8(desc, qd, kd, vd, count, idx, s, to_dev(r, layout),
                                                c.tolist())
    torch.cuda.synchronize()
    mask = O.mask_from_lists(count.cpu().numpy(), idx.cpu().numpy(), M)
    q64, k64, v64 = (synth.to_f64(x) for x in (q, k, v))
    qq, kk, vv = O.mx_quantize(q64, -1), O.mx_quantize(k64, -1), O.mx_quantize(v64, 2)
    ref = O.masked_attention_mx(q64, k64, v64, cfg.block, s, mask)
    bound, exp_sq = parity.fp8_weight_bounds(qq, kk, vv, mask, cfg.block, s, ref)
    err, rel, lim = parity.check_fp8_out(f64(out), ref, bound, exp_sq, "fp8 sparse")
    say(f"    max|err| {err:.3e} rel-L2 {rel:.3e} (limit {lim:.3e}); "
        f"bf16-path limit {parity.ATOL_OUT}/{parity.RTOL_L2}")
    lse_ref = O.attention_lse(qq, kk, cfg.block, s, mask)
    g = lse.cpu().numpy().astype(np.float64)
    parity.check_rows_within(g, lse_ref, parity.ATOL_STAT + math.log1p(parity.U_E4M3), "fp8 lse")
    if residual:
        parity.check_fp8_out(f64(out_e), O.residual_epilogue(ref, synth.to_f64(r), c), bound,
                             exp_sq, "fp8 sparse + epilogue")
    return dict(out=out, count=count, M=M)


FP8 = {
    "tiny": dict(),
    "ragged_d128_b64_bnhd": dict(batch=2, heads=3, head_dim=128, seq=1000, layout="bnhd",
                                 top_p=[0.5, 0.9, 0.99], residual=True),
    "odd_blocks_d64": dict(heads=2, head_dim=64, seq=64 * 9 + 17),
    "b128_short_last_block": dict(heads=2, head_dim=128, block=128, seq=128 * 5 + 20),
    "d64_b128": dict(heads=2, head_dim=64, block=128, seq=2000, residual=True),
    "single_partial_block": dict(heads=2, head_dim=128, seq=37),
    "one_token_last_block": dict(heads=1, head_dim=64, seq=129),
    "p_one_all_blocks": dict(heads=2, head_dim=128, seq=700, top_p=1.0),
    "max_heads_128": dict(heads=128, head_dim=64, seq=300),
}


@pytest.mark.parametrize("case", list(FP8))
def test_fp8_case(bsa, case):
    kw = dict(FP8[case])
    seq = kw.pop("seq", None)
    layout = kw.pop("layout", "bhnd")
    top_p = kw.pop("top_p", None)
    residual = kw.pop("residual", False)
    grid = synth.WORKLOADS["tiny"].grid if seq is None else (1, 1, seq)
    cfg = synth.workload("tiny", grid=grid, **kw)
    run_fp8(bsa, cfg, layout, top_p, residual)


def test_fp8_full_size(bsa):
    """Wan2.1-14B 720p layer (B=1, H=40, D=128, N=75,600, block 64, top-p 0.95): sampled heads
    and query blocks against the oracle on the quantised inputs."""
    cfg = synth.WORKLOADS["wan14b_720p"]
    say("[test] fp8 full-size wan14b_720p: generating inputs")
    q, k, v = synth.make_qkv(cfg)
    p, _ = synth.head_params(cfg)
    s = cfg.head_dim ** -0.5
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    desc = bsa.make_desc(qd, cfg.block)
    probs = bsa.recap_block_scores(desc, qd, kd, s)
    count, idx, _, _ = bsa.recap_topp_mask(desc, probs, p.tolist())
    del probs
    out = bsa.recap_block_sparse_attn_fp8(desc, qd, kd, vd, count, idx, s)
    torch.cuda.synchronize()
    M, blk = cfg.num_blocks, cfg.block
    for h in (0, 21):
        blocks = sorted({0, M - 1} | set(np.random.default_rng(700 + h).choice(M, 3, False).tolist()))
        say(f"[check] head {h} blocks {blocks}")
        m_h = O.mask_from_lists(count[:, h:h + 1].cpu().numpy(), idx[:, h:h + 1].cpu().numpy(), M)
        q64, k64, v64 = (synth.to_f64(x[:, h:h + 1]) for x in (q, k, v))
        qq, kk, vv = O.mx_quantize(q64, -1), O.mx_quantize(k64, -1), O.mx_quantize(v64, 2)
        sel = [(0, 0, i) for i in blocks]
        ref = O.masked_attention(qq, kk, vv, blk, s, m_h, rows=sel)
        got = f64(out[:, h:h + 1])
        for i in blocks:
            lo, hi = i * blk, min(cfg.seq, (i + 1) * blk)
            bound, exp_sq = parity.fp8_weight_bounds(qq, kk, vv, m_h, blk, s, np.nan_to_num(ref),
                                                     rows=[(0, 0, i)])
            parity.check_fp8_out(got[:, :, lo:hi], ref[:, :, lo:hi], bound[:, :, lo:hi], exp_sq,
                                 f"h{h} b{i}")


def _pv_key(h, e):
    return 32 * (e // 16) + 8 * ((e % 16) // 4) + 4 * h + e % 4


@pytest.mark.parametrize("D,N", [(64, 300), (128, 200)])
def test_packed_tiles_bitexact(bsa, D, N):
    """The K and V tiles the FP8 call packs into its workspace hold exactly the oracle's MXFP8
    values: K rows in key order with scales [half][row][s][m] (group 2 m + half of key 32 s +
    row), V rows per channel with byte 32 h + e = key pv_key(h, e) and scales [half][row][dt]
    (channel 32 dt + row, keys 32 half ..+31); keys past N are zero."""
    from block_sparse_attention_top_amd import _lib
    say(f"[test] packed tiles D={D} N={N}")
    g = torch.Generator().manual_seed(900 + D)
    q, k, v = (torch.randn((1, 2, N, D), generator=g).to(torch.bfloat16) for _ in range(3))
    qd, kd, vd = (to_dev(x) for x in (q, k, v))
    desc = bsa.make_desc(qd, 64)
    M = -(-N // 64)
    count = torch.full((1, 2, M), M, dtype=torch.int32, device=DEV)
    idx = torch.arange(M, dtype=torch.int32, device=DEV).expand(1, 2, M, M).contiguous()
    need = bsa.recap_workspace_size(_lib.OP_SPARSE_FP8, desc)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    bsa.recap_block_sparse_attn_fp8(desc, qd, kd, vd, count, idx, workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    al = lambda x: -(-x // 256) * 256
    T = M  # 64-key tiles per head
    TS = 66 * D
    k0 = al(2 * N * D) + al(2 * N * D // 32)
    kt = w[k0:k0 + 2 * T * TS].reshape(2, T, TS)
    v0 = k0 + al(2 * T * TS)
    vt = w[v0:v0 + 2 * T * TS].reshape(2, T, TS)
    kq = O.mx_quantize(synth.to_f64(k), -1)[0]
    vq = O.mx_quantize(synth.to_f64(v), 2)[0]
    for hd in range(2):
        for t in range(T):
            codes = _E4M3[kt[hd, t, :64 * D].astype(np.int64)].reshape(64, D)
            sc = kt[hd, t, 64 * D:].reshape(2, 32, 2, D // 64).astype(np.float64) - 127
            val = np.zeros((64, D))
            for h in range(2):
                for s_ in range(2):
                    for m in range(D // 64):
                        rows = slice(32 * s_, 32 * s_ + 32)
                        cols = slice(64 * m + 32 * h, 64 * m + 32 * h + 32)
                        val[rows, cols] = codes[rows, cols] * np.exp2(sc[h, :, s_, m])[:, None]
            keys = np.arange(64 * t, 64 * t + 64)
            want = np.where((keys < N)[:, None], kq[hd, np.minimum(keys, N - 1)], 0.0)
            assert np.array_equal(val, want), ("K", hd, t)
            vcodes = _E4M3[vt[hd, t, :64 * D].astype(np.int64)].reshape(D, 64)
            vsc = vt[hd, t, 64 * D:].reshape(2, 32, D // 32).astype(np.float64) - 127
            vval = np.zeros((D, 64))
            for h in range(2):
                for e in range(32):
                    key = _pv_key(h, e)
                    grp = key // 32
                    for dt in range(D // 32):
                        vval[32 * dt:32 * dt + 32, key] = vcodes[32 * dt:32 * dt + 32, 32 * h + e] * \
                            np.exp2(vsc[grp, :, dt])
            want_v = np.where((keys < N)[None, :], vq[hd, np.minimum(keys, N - 1)].T, 0.0)
            assert np.array_equal(vval, want_v), ("V", hd, t)
