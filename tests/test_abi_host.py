"""Host side of the C ABI, without a GPU: the library loads, exports every symbol that
include/recap.h declares, sizes workspaces, and rejects bad arguments before any HIP call.

Validation tests pass fake device addresses; they run only where no GPU is visible, so a
validation bug could never turn into a launch with bogus pointers."""
import ctypes
import os
import re

import pytest
import torch

from block_sparse_attention_top_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "recap.h")
NO_GPU = torch.cuda.device_count() == 0
cpu_only = pytest.mark.skipif(not NO_GPU, reason="fake-pointer validation runs only without a GPU")

FAKE = 0x100000  # 16-byte aligned, never dereferenced


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(recap_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.recap_abi_version() == _lib.ABI_VERSION == 7
    for st in list(_lib.STATUS_NAMES) + [-99]:
        s = lib.recap_status_string(st)
        assert s and len(s.decode()) > 1


def desc(B=1, H=2, N=4096, D=64, block=64, layout="bhnd"):
    if layout == "bhnd":
        sb, sh, sn = H * N * D, N * D, D
    else:  # bnhd
        sb, sh, sn = N * H * D, D, H * D
    return _lib.RecapDesc(B, H, N, D, block, 0, sb, sh, sn)


def ws_size(op, d):
    n = ctypes.c_size_t(0)
    st = _lib.load().recap_workspace_size(op, ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_workspace_sizes():
    d = desc(B=1, H=40, N=75600, D=128, block=64)
    M = 1182
    st, n = ws_size(_lib.OP_BLOCK_SCORES, d)
    assert st == 0 and n == 2 * M * 40 * 128 * 4
    assert ws_size(_lib.OP_TOPP, d) == (0, 0)
    # sparse and plain dense attention read q, k, v as given; paired sparse walks (64-token
    # blocks) keep the order of the grid's last min(tiles, 1024) tiles (int32 each, 256-aligned)
    assert ws_size(_lib.OP_SPARSE, d) == (0, 1024 * 4)
    assert ws_size(_lib.OP_SPARSE, desc(H=2, N=4096)) == (0, 256)  # 2 x 32 pairs
    assert ws_size(_lib.OP_SPARSE, desc(H=24, N=118800, D=128, block=128)) == (0, 0)
    assert ws_size(_lib.OP_DENSE, d) == (0, 0)
    st, n2 = ws_size(_lib.OP_DENSE_CAPTURE, d)
    flags = -(-40 * M // 256) * 256  # one byte per query block, 256-byte aligned
    assert st == 0 and n2 == 40 * M * 64 * 128 * 4 + flags
    # coarse tail: K̄, V̄ fp32, then K̄ hi, K̄ lo, V̄ bf16 over M padded to 1216 pooled keys,
    # the kept bitmaps (ceil(M / 32) + 1 = 38 words per query block), and for the moment
    # refinements the key variances (fp32 and a bf16 copy), 37 slices of covariance partial
    # sums (fp32 D x D) and the covariance (a bf16 pair, D x D each), each 256-byte aligned
    pooled = 40 * M * 128 * 4
    p16 = 40 * 1216 * 128 * 2
    bits = -(-40 * M * 38 * 4 // 256) * 256
    mom = pooled + p16 + 40 * 37 * 128 * 128 * 4 + 2 * 40 * 128 * 128 * 2
    st, nt = ws_size(_lib.OP_TAIL, d)
    assert st == 0 and nt == 2 * pooled + 3 * p16 + bits + mom
    rows = 40 * 75600 * 4
    for op in (_lib.OP_DENSE_TAIL, _lib.OP_SPARSE_TAIL):
        assert ws_size(op, d) == (0, 2 * (rows + rows * 128) + nt)
    # FP8 call: Q codes + scales, packed K and V tiles of 66 * D bytes per 64 keys
    q8 = 40 * 75600 * 128
    qs = -(-40 * 75600 * 4 // 256) * 256
    tiles = 40 * (M * 64 // 64) * 66 * 128
    assert ws_size(_lib.OP_SPARSE_FP8, d) == (0, q8 + qs + 2 * tiles)
    assert ws_size(9, d)[0] == -5
    assert ws_size(99, d)[0] == -5
    assert _lib.load().recap_workspace_size(0, ctypes.byref(d), None) == -1


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, -2), ("heads", 0, -2), ("heads", 129, -2), ("seq", 0, -2),
    ("head_dim", 96, -2), ("block", 32, -2), ("reserved", 1, -2), ("seq", 8192 * 64 + 1, -2),
    ("stride_n", 60, -3), ("stride_n", 0, -3), ("stride_h", -8, -3), ("stride_n", 32, -3),
])
def test_descriptor_validation(field, value, status):
    d = desc()
    setattr(d, field, value)
    assert ws_size(_lib.OP_SPARSE, d)[0] == status


def test_token_stride_limit():
    """A token stride of 2^24 elements or more would overflow the 32-bit byte offsets of one
    key tile's rows (128 rows x stride_n x 2 bytes); such descriptors are rejected. The layout
    is [N, B, H, D]-like (tokens outermost) and otherwise valid."""
    D = 128
    ok = _lib.RecapDesc(1, 128, 100, D, 64, 0, 128 * D, D, (1 << 24) - 8)
    assert ws_size(_lib.OP_SPARSE, ok)[0] == 0
    bad = _lib.RecapDesc(1, 128, 100, D, 64, 0, 128 * D, D, 1 << 24)
    assert ws_size(_lib.OP_SPARSE, bad)[0] == -3


def test_strides_beyond_64_bit_offsets_rejected():
    """Strides whose tensor extent does not fit 64-bit element offsets are RECAP_E_STRIDE (the
    overlap check itself must not overflow: the sanitizer build runs this arithmetic too)."""
    d = _lib.RecapDesc(3, 5, 1000, 128, 128, 0, 1 << 62, 1 << 62, 128)
    assert ws_size(_lib.OP_SPARSE, d)[0] == -3
    d = _lib.RecapDesc(3, 5, 1000, 128, 128, 0, (1 << 63) - 8, 128 * 1000, 128)
    assert ws_size(_lib.OP_SPARSE, d)[0] == -3


def test_layouts_accepted():
    for layout in ("bhnd", "bnhd"):
        assert ws_size(_lib.OP_SPARSE, desc(B=2, H=3, N=1000, layout=layout))[0] == 0
    d = desc(B=2, H=3, N=1000)
    d.stride_h = d.stride_n * 999  # heads overlap the last token of the previous head
    assert ws_size(_lib.OP_SPARSE, d)[0] == -3


def _p(x=FAKE):
    return ctypes.c_void_p(x)


@cpu_only
def test_block_scores_noalloc_validation():
    """The allocation-free variant validates like recap_block_scores and rejects, before any
    HIP call, a call whose pooled means would not fit the fixed 64 MiB scratch."""
    lib = _lib.load()
    call = lambda d, q=_p(), k=_p(), s=0.125, pr=_p(): \
        lib.recap_block_scores_noalloc(ctypes.byref(d), q, k, s, pr, None)
    d = desc()
    assert call(d, q=None) == -1
    assert call(d, pr=_p(FAKE + 4)) == -4
    assert call(d, s=float("nan")) == -5
    assert call(d) == -7  # valid, fits, no device
    fits = desc(B=1, H=40, N=75600, D=128)  # 2 x 40 x 1182 x 128 x 4 = 48.4 MB
    assert ws_size(_lib.OP_BLOCK_SCORES, fits)[1] <= _lib.NOALLOC_SCRATCH_BYTES
    assert call(fits) == -7
    big = desc(B=1, H=64, N=75600, D=128)  # 77.5 MB of means
    assert ws_size(_lib.OP_BLOCK_SCORES, big)[1] > _lib.NOALLOC_SCRATCH_BYTES
    assert call(big) == -6


@cpu_only
def test_block_scores_validation():
    lib = _lib.load()
    d = desc()
    _, need = ws_size(_lib.OP_BLOCK_SCORES, d)
    call = lambda q=_p(), k=_p(), s=0.125, pr=_p(), ws=_p(), n=need: \
        lib.recap_block_scores(ctypes.byref(d), q, k, s, pr, ws, n, None)
    assert call(q=None) == -1
    assert call(pr=None) == -1
    assert call(q=_p(FAKE + 2)) == -4
    assert call(s=float("nan")) == -5
    assert call(s=0.0) == -5
    assert call(s=float("inf")) == -5
    assert call(ws=None) == -6
    assert call(n=need - 1) == -6
    assert call(ws=_p(FAKE + 16)) == -4
    assert call() == -7  # valid arguments, no device


@cpu_only
def test_topp_validation():
    lib = _lib.load()
    d = desc(H=2)
    good = (ctypes.c_float * 2)(0.9, 0.5)
    call = lambda tp=good, pr=_p(): lib.recap_topp_mask(ctypes.byref(d), pr, tp, _p(), _p(),
                                                       None, None, None)
    assert call(pr=None) == -1
    assert call(tp=None) == -1
    assert call(tp=(ctypes.c_float * 2)(0.9, 1.5)) == -5
    assert call(tp=(ctypes.c_float * 2)(-0.1, 0.5)) == -5
    assert call(tp=(ctypes.c_float * 2)(float("nan"), 0.5)) == -5
    assert call() == -7


@cpu_only
def test_sparse_and_dense_validation():
    lib = _lib.load()
    d = desc(H=2)
    _, need = ws_size(_lib.OP_SPARSE, d)
    sc = (ctypes.c_float * 2)(0.5, 1.0)

    def sparse(res=None, rs=None, out=_p(FAKE + 4096), ws=_p(), n=need, s=0.125):
        return lib.recap_block_sparse_attn(ctypes.byref(d), _p(), _p(FAKE + 1024),
                                           _p(FAKE + 2048), _p(), _p(), s, res, rs, out, ws, n,
                                           None)
    assert sparse(res=_p(FAKE + 8192)) == -1  # residual without scales
    assert sparse(out=None) == -1
    assert sparse(out=_p(FAKE)) == -5  # out aliases q
    assert sparse(res=_p(FAKE + 8192), rs=(ctypes.c_float * 2)(0.5, float("inf"))) == -5
    assert need == 256 and sparse(ws=None, n=0) == -6  # the end-order table is required
    assert sparse(n=need - 1) == -6
    assert sparse(s=-1.0) == -5
    assert sparse(res=_p(FAKE + 8192), rs=sc) == -7

    _, need_c = ws_size(_lib.OP_DENSE_CAPTURE, d)

    def dense(cnt=None, idx=None, rout=None, ws=_p(), n=need):
        return lib.recap_dense_attn(ctypes.byref(d), _p(), _p(FAKE + 1024), _p(FAKE + 2048),
                                    0.125, cnt, idx, _p(FAKE + 4096), rout, ws, n, None)
    assert dense(rout=_p(FAKE + 8192)) == -1  # capture needs kept lists
    assert dense(cnt=_p(), idx=_p(), rout=_p(FAKE + 8192)) == -6  # capture workspace larger
    assert dense(cnt=_p(), idx=_p(), rout=_p(FAKE + 4096), n=need_c) == -5  # R aliases out
    assert dense() == -7
    assert dense(cnt=_p(), idx=_p(), rout=_p(FAKE + 8192), n=need_c) == -7


@cpu_only
def test_stats_validation():
    lib = _lib.load()
    d = desc(H=2)
    _, need = ws_size(_lib.OP_SPARSE, d)
    _, need_c = ws_size(_lib.OP_DENSE_CAPTURE, d)

    def sparse(lse=_p(FAKE + 12288)):
        return lib.recap_block_sparse_attn_stats(ctypes.byref(d), _p(), _p(FAKE + 1024),
                                                 _p(FAKE + 2048), _p(), _p(), 0.125, None, None,
                                                 _p(FAKE + 4096), lse, _p(), need, None)
    assert sparse(lse=None) == -1  # the statistics output is the point of this entry point
    assert sparse(lse=_p(FAKE + 12290)) == -4
    assert sparse() == -7

    def dense(cnt=None, idx=None, rout=None, lse=_p(FAKE + 12288), km=None, n=need):
        return lib.recap_dense_attn_stats(ctypes.byref(d), _p(), _p(FAKE + 1024),
                                          _p(FAKE + 2048), 0.125, cnt, idx, _p(FAKE + 4096),
                                          rout, lse, km, _p(), n, None)
    assert dense(lse=None) == -1
    assert dense(km=_p(FAKE + 16384)) == -1  # kept mass needs the kept lists
    assert dense(cnt=_p(), idx=_p(), km=_p(FAKE + 16384)) == -6  # and the capture workspace
    assert dense(cnt=_p(), idx=_p(), km=_p(FAKE + 16388), n=need_c) == -4
    assert dense() == -7
    assert dense(cnt=_p(), idx=_p(), km=_p(FAKE + 16384), n=need_c) == -7


@cpu_only
def test_tail_validation():
    lib = _lib.load()
    d = desc(H=2)
    _, need_t = ws_size(_lib.OP_TAIL, d)
    _, need_m = ws_size(_lib.OP_SPARSE_TAIL, d)
    q, k, v = _p(), _p(FAKE + 1024), _p(FAKE + 2048)

    def est(cnt=_p(), lse=_p(FAKE + 8192), to=_p(FAKE + 16384), n=need_t, s=0.125, fl=0):
        return lib.recap_tail_estimate(ctypes.byref(d), q, k, v, cnt, _p(), s, fl, lse, to, _p(),
                                       n, None)
    assert est(fl=2) == -5 and est(fl=-1) == -5  # unknown flag bits
    assert est(fl=_lib.TAIL_MOMENTS) == -7
    assert est(cnt=None) == -1
    assert est(lse=None) == -1
    assert est(to=_p(FAKE + 16388)) == -4
    assert est(to=_p(FAKE + 8192)) == -5  # outputs alias
    assert est(s=float("nan")) == -5
    assert est(n=need_t - 1) == -6
    assert est() == -7

    def dense(out=_p(FAKE + 4096), dl=_p(FAKE + 8192), do=_p(FAKE + 16384), n=need_m, fl=0):
        return lib.recap_dense_attn_tail(ctypes.byref(d), q, k, v, 0.125, fl, _p(), _p(), out,
                                         dl, do, _p(), n, None)
    assert dense(fl=4) == -5 and dense(fl=1) == -7
    assert dense(dl=None) == -1
    assert dense(do=None) == -1
    assert dense(do=_p(FAKE + 4096)) == -5  # discrepancy aliases out
    assert dense(do=_p(FAKE + 8192)) == -5  # the two discrepancy outputs alias
    assert dense(out=_p(FAKE)) == -5        # out aliases q
    assert dense(n=need_m - 256) == -6
    assert dense() == -7

    def sparse(dl=None, do=None, out=_p(FAKE + 4096), n=need_m, fl=0):
        return lib.recap_block_sparse_attn_tail(ctypes.byref(d), q, k, v, _p(), _p(), 0.125, fl,
                                                dl, do, out, _p(), n, None)
    assert sparse(fl=3) == -5 and sparse(fl=1) == -7
    assert sparse(dl=_p(FAKE + 8192)) == -1  # both or neither
    assert sparse(do=_p(FAKE + 16384)) == -1
    assert sparse(out=None) == -1
    assert sparse(dl=_p(FAKE + 8194), do=_p(FAKE + 16384)) == -4
    assert sparse(n=need_t) == -6
    assert sparse() == -7
    assert sparse(dl=_p(FAKE + 8192), do=_p(FAKE + 16384)) == -7


@cpu_only
def test_fp8_validation():
    lib = _lib.load()
    d = desc(H=2)
    _, need = ws_size(_lib.OP_SPARSE_FP8, d)
    sc = (ctypes.c_float * 2)(0.5, 1.0)

    def fp8(res=None, rs=None, out=_p(FAKE + 4096), lse=None, n=need, s=0.125):
        return lib.recap_block_sparse_attn_fp8(ctypes.byref(d), _p(), _p(FAKE + 1024),
                                               _p(FAKE + 2048), _p(), _p(), s, res, rs, out, lse,
                                               _p(), n, None)
    assert fp8(out=None) == -1
    assert fp8(res=_p(FAKE + 8192)) == -1
    assert fp8(out=_p(FAKE + 1024)) == -5  # out aliases k
    assert fp8(lse=_p(FAKE + 12290)) == -4
    assert fp8(s=float("nan")) == -5
    assert fp8(n=need - 1) == -6
    assert fp8() == -7
    assert fp8(res=_p(FAKE + 8192), rs=sc, lse=_p(FAKE + 12288)) == -7

    def quant(x=_p(), mode=0, codes=_p(FAKE + 4096), scales=_p(FAKE + 8192)):
        return lib.recap_mx_quantize(ctypes.byref(d), x, mode, codes, scales, None)
    assert quant(codes=None) == -1
    assert quant(x=_p(FAKE + 2)) == -4
    assert quant(mode=2) == -5
    assert quant(scales=_p(FAKE + 4096)) == -5
    assert quant() == -7
    assert quant(mode=1) == -7
