"""GPU: sparse attention over hand-made kept lists (not produced by top-p), for the bf16 path,
its row statistics and the FP8 path.

The lists cover:
- rows keeping nothing;
- rows keeping one block, and rows keeping every block;
- a random third of the blocks;
- every other block;
- paired 64-row query blocks whose lists differ, so the kernels' union walks skip tiles for one
  half of the work-group.

A row keeping nothing follows the ABI's convention: zeros before the epilogue (so exactly
bf16(c_h R) with a residual) and lse = -inf. top-p never produces one, and the oracle leaves it
undefined. Every other row is checked against the oracle with the same bounds as the top-p
cases.
"""
import math

import numpy as np
import pytest
import torch

import parity
import synth
from gpu_common import DEV, bsa, f64, say, to_dev  # noqa: F401  (bsa is a fixture)
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _lists(B, H, M, seed):
    g = np.random.default_rng(seed)
    cnt = np.zeros((B, H, M), np.int32)
    idx = np.zeros((B, H, M, M), np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(M):
                kind = (i + h + b) % 5
                if kind == 0:
                    js = []
                elif kind == 1:
                    js = [int(g.integers(M))]
                elif kind == 2:
                    js = list(range(M))
                elif kind == 3:
                    js = sorted(g.choice(M, size=max(1, M // 3), replace=False).tolist())
                else:
                    js = [j for j in range(M) if j % 2 == i % 2]
                cnt[b, h, i] = len(js)
                idx[b, h, i, :len(js)] = js
    return cnt, idx


def _rows(cnt, block, N):
    """(b, h, i) of the query blocks that keep something / nothing, and their token ranges."""
    B, H, M = cnt.shape
    keep, empty = [], []
    for b in range(B):
        for h in range(H):
            for i in range(M):
                (keep if cnt[b, h, i] > 0 else empty).append((b, h, i))
    rng = lambda i: (i * block, min(N, (i + 1) * block))  # noqa: E731
    return keep, empty, rng


def _gather(x, rows, rng):
    return np.concatenate([x[b, h, slice(*rng(i))] for b, h, i in rows], axis=0)


CASES = {
    "d128_b64_pairs": dict(head_dim=128, block=64, seq=64 * 9 + 17, heads=2),
    "d64_b64_pairs": dict(head_dim=64, block=64, seq=300, heads=3),
    "d128_b128": dict(head_dim=128, block=128, seq=700, heads=2),
    "d64_b128": dict(head_dim=64, block=128, seq=128 * 4 + 50, heads=2),
}


@pytest.mark.parametrize("case", list(CASES))
def test_hand_made_lists(bsa, case):
    kw = dict(CASES[case])
    seq = kw.pop("seq")
    cfg = synth.workload("tiny", grid=(1, 1, seq), **kw)
    B, H, N, D, blk = cfg.batch, cfg.heads, seq, cfg.head_dim, cfg.block
    M = -(-N // blk)
    s = D ** -0.5
    say(f"[case] hand-made lists {case}: H={H} D={D} N={N} block={blk} M={M}")
    q, k, v = synth.make_qkv(cfg)
    r = synth.make_residual(cfg)
    c = [0.75] * H
    qd, kd, vd, rd = (to_dev(x) for x in (q, k, v, r))
    cnt, idx = _lists(B, H, M, 900 + D + blk)
    count = torch.from_numpy(cnt).to(DEV)
    kidx = torch.from_numpy(idx).to(DEV)
    desc = bsa.make_desc(qd, blk)

    out, lse = bsa.recap_block_sparse_attn_stats(desc, qd, kd, vd, count, kidx, s)
    out_e = bsa.recap_block_sparse_attn(desc, qd, kd, vd, count, kidx, s, rd, c)
    o8, lse8 = bsa.recap_block_sparse_attn_fp8(desc, qd, kd, vd, count, kidx, s, want_lse=True)
    o8_e = bsa.recap_block_sparse_attn_fp8(desc, qd, kd, vd, count, kidx, s, rd, c)
    torch.cuda.synchronize()

    keep, empty, rng = _rows(cnt, blk, N)
    assert keep and empty
    mask = O.mask_from_lists(cnt, idx, M)
    q64, k64, v64, r64 = (synth.to_f64(x) for x in (q, k, v, r))

    # rows keeping nothing: zeros, c_h R after the epilogue (bf16 rounding of an exact
    # product), lse -inf
    cr = (0.75 * r.float()).to(torch.bfloat16)
    for b, h, i in empty:
        sl = slice(*rng(i))
        for name, o_plain, o_epi, l_ in (("bf16", out, out_e, lse), ("fp8", o8, o8_e, lse8)):
            assert torch.count_nonzero(o_plain[b, h, sl].float()) == 0, (name, b, h, i)
            assert torch.equal(o_epi[b, h, sl].cpu(), cr[b, h, sl]), (name, b, h, i)
            assert torch.all(torch.isneginf(l_[b, h, sl])), (name, b, h, i)

    # every other row against the oracle
    ref = O.masked_attention(q64, k64, v64, blk, s, mask, rows=keep)
    parity.check_out(_gather(f64(out), keep, rng), _gather(ref, keep, rng), f"{case} bf16")
    ref_e = O.residual_epilogue(ref, r64, np.asarray(c))
    parity.check_out(_gather(f64(out_e), keep, rng), _gather(ref_e, keep, rng),
                     f"{case} bf16 + epilogue")
    lse_ref = O.attention_lse(q64, k64, blk, s, mask, rows=keep)
    parity.check_rows_within(_gather(lse.cpu().numpy().astype(np.float64), keep, rng),
                             _gather(lse_ref, keep, rng), parity.ATOL_STAT, f"{case} bf16 lse")

    qq, kk, vv = O.mx_quantize(q64, -1), O.mx_quantize(k64, -1), O.mx_quantize(v64, 2)
    ref8 = O.masked_attention_mx(q64, k64, v64, blk, s, mask, rows=keep)
    bound, exp_sq = parity.fp8_weight_bounds(qq, kk, vv, mask, blk, s, ref8, rows=keep)
    err, rel, lim = parity.check_fp8_out(_gather(f64(o8), keep, rng), _gather(ref8, keep, rng),
                                         _gather(bound, keep, rng), exp_sq, f"{case} fp8")
    say(f"    fp8 max|err| {err:.3e} rel-L2 {rel:.3e} (limit {lim:.3e})")
    ref8_e = O.residual_epilogue(ref8, r64, np.asarray(c))
    parity.check_fp8_out(_gather(f64(o8_e), keep, rng), _gather(ref8_e, keep, rng),
                         _gather(bound, keep, rng), exp_sq, f"{case} fp8 + epilogue")
    lse8_ref = O.attention_lse(qq, kk, blk, s, mask, rows=keep)
    parity.check_rows_within(_gather(lse8.cpu().numpy().astype(np.float64), keep, rng),
                             _gather(lse8_ref, keep, rng),
                             parity.ATOL_STAT + math.log1p(parity.U_E4M3), f"{case} fp8 lse")
