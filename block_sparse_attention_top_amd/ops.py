"""torch-tensor marshalling for the librecap.so entry points (same names as the C functions).

Every step of the computation runs in the HIP library; this module checks dtypes, devices and
strides, allocates outputs and workspace with torch, and passes raw device pointers plus the
current HIP stream. There is no CPU or PyTorch fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import math
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import RecapDesc, check


def _on_stream(fn):
    """Run an entry point's body with its `stream` argument as torch's current stream, so that
    every buffer the body allocates (outputs, workspace, temporaries) comes from the caching
    allocator's pool of that stream. A block freed when the function returns can then be handed
    out again only to work queued behind the call's kernels on the same stream; allocated on
    another stream, it could be reused while those kernels still read or write it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        stream = sig.bind_partial(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)

    wrapper.on_stream = True
    return wrapper


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _host_floats(vals: Sequence[float], heads: int, what: str):
    vals = [float(x) for x in (vals if hasattr(vals, "__len__") else [vals] * heads)]
    if len(vals) != heads:
        raise ValueError(f"{what}: expected {heads} per-head values, got {len(vals)}")
    return (ctypes.c_float * heads)(*vals)


def make_desc(q: torch.Tensor, block: int) -> RecapDesc:
    """Descriptor for a [B, H, N, D] bf16 view (any element strides with D contiguous)."""
    if q.dim() != 4:
        raise ValueError("expected a 4-d [B, H, N, D] tensor view")
    B, H, N, D = q.shape
    sb, sh, sn, sd = q.stride()
    if sd != 1:
        raise ValueError("head dimension must be contiguous")
    return RecapDesc(B, H, N, D, int(block), 0, sb, sh, sn)


def _same_layout(desc: RecapDesc, *ts: Optional[torch.Tensor]) -> None:
    for t in ts:
        if t is None:
            continue
        if t.dtype != torch.bfloat16 or not t.is_cuda:
            raise TypeError("q, k, v, out and residual must be bf16 device tensors")
        if tuple(t.shape) != (desc.batch, desc.heads, desc.seq, desc.head_dim) or \
                tuple(t.stride()) != (desc.stride_b, desc.stride_h, desc.stride_n, 1):
            raise ValueError("q, k, v, out and residual must share shape and strides")


def num_blocks(desc: RecapDesc) -> int:
    return -(-desc.seq // desc.block)


def recap_workspace_size(op: int, desc: RecapDesc) -> int:
    n = ctypes.c_size_t(0)
    check(_lib.load().recap_workspace_size(op, ctypes.byref(desc), ctypes.byref(n)),
          "recap_workspace_size")
    return int(n.value)


def _workspace(op: int, desc: RecapDesc, device, given: Optional[torch.Tensor]):
    need = recap_workspace_size(op, desc)
    if need == 0:
        return None, 0
    if given is not None:
        if given.numel() * given.element_size() < need:
            raise ValueError("workspace too small")
        return given, given.numel() * given.element_size()
    return torch.empty(need, dtype=torch.uint8, device=device), need


def _like_out(t: torch.Tensor) -> torch.Tensor:
    return torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device)


@_on_stream
def recap_block_scores(desc: RecapDesc, q, k, sm_scale: Optional[float] = None, probs=None,
                       workspace=None, stream=None) -> torch.Tensor:
    """fp32 [B,H,M,M] block-pair softmax of mean-pooled Q and K (see include/recap.h)."""
    _same_layout(desc, q, k)
    M = num_blocks(desc)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    if probs is None:
        probs = torch.empty((desc.batch, desc.heads, M, M), dtype=torch.float32, device=q.device)
    ws, nbytes = _workspace(_lib.OP_BLOCK_SCORES, desc, q.device, workspace)
    check(_lib.load().recap_block_scores(ctypes.byref(desc), _ptr(q), _ptr(k), float(sm_scale),
                                         _ptr(probs), _ptr(ws), nbytes, _stream(stream)),
          "recap_block_scores")
    return probs


@_on_stream
def recap_block_scores_noalloc(desc: RecapDesc, q, k, sm_scale: Optional[float] = None,
                               probs=None, stream=None) -> torch.Tensor:
    """recap_block_scores with the library's fixed device scratch instead of a workspace
    (the C call allocates nothing; pass `probs` to allocate nothing here either)."""
    _same_layout(desc, q, k)
    M = num_blocks(desc)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    if probs is None:
        probs = torch.empty((desc.batch, desc.heads, M, M), dtype=torch.float32, device=q.device)
    elif probs.dtype != torch.float32 or tuple(probs.shape) != (desc.batch, desc.heads, M, M) \
            or not probs.is_contiguous():
        raise ValueError("probs must be contiguous fp32 [B, H, M, M]")
    check(_lib.load().recap_block_scores_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k),
                                                 float(sm_scale), _ptr(probs), _stream(stream)),
          "recap_block_scores_noalloc")
    return probs


@_on_stream
def recap_topp_mask(desc: RecapDesc, probs, top_p, kept_count=None, kept_idx=None,
                    want_mask: bool = False, want_mass: bool = False, stream=None):
    """Top-p selection per query block: (count [B,H,M], idx [B,H,M,M], mask|None, mass|None)."""
    M = num_blocks(desc)
    if probs.dtype != torch.float32 or tuple(probs.shape) != (desc.batch, desc.heads, M, M) \
            or not probs.is_contiguous():
        raise ValueError("probs must be contiguous fp32 [B, H, M, M]")
    dev = probs.device
    if kept_count is None:
        kept_count = torch.empty((desc.batch, desc.heads, M), dtype=torch.int32, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((desc.batch, desc.heads, M, M), dtype=torch.int32, device=dev)
    mask = torch.empty((desc.batch, desc.heads, M, M), dtype=torch.uint8, device=dev) \
        if want_mask else None
    mass = torch.empty((desc.batch, desc.heads, M), dtype=torch.float32, device=dev) \
        if want_mass else None
    tp = _host_floats(top_p, desc.heads, "top_p")
    check(_lib.load().recap_topp_mask(ctypes.byref(desc), _ptr(probs), tp, _ptr(kept_count),
                                      _ptr(kept_idx), _ptr(mask), _ptr(mass), _stream(stream)),
          "recap_topp_mask")
    return kept_count, kept_idx, mask, mass


def _row_stat(desc: RecapDesc, given: Optional[torch.Tensor], device) -> torch.Tensor:
    if given is None:
        return torch.empty((desc.batch, desc.heads, desc.seq), dtype=torch.float32, device=device)
    if given.dtype != torch.float32 or tuple(given.shape) != (desc.batch, desc.heads, desc.seq) \
            or not given.is_contiguous():
        raise ValueError("row statistics are contiguous fp32 [B, H, N]")
    return given


@_on_stream
def recap_block_sparse_attn(desc: RecapDesc, q, k, v, kept_count, kept_idx,
                            sm_scale: Optional[float] = None, residual=None, res_scale=None,
                            out=None, workspace=None, stream=None, lse=None,
                            want_lse: bool = False):
    """Attention over the kept blocks, optionally O += c_h * R (bf16, q's layout). With
    want_lse (or lse given) returns (out, lse) with lse the fp32 [B,H,N] log-sum-exp of the
    attended scores (recap_block_sparse_attn_stats)."""
    _same_layout(desc, q, k, v, out, residual)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    if out is None:
        out = _like_out(q)
    rs = None
    if residual is not None:
        if res_scale is None:
            raise ValueError("res_scale is required with a residual")
        rs = _host_floats(res_scale, desc.heads, "res_scale")
    ws, nbytes = _workspace(_lib.OP_SPARSE, desc, q.device, workspace)
    if want_lse or lse is not None:
        lse = _row_stat(desc, lse, q.device)
        check(_lib.load().recap_block_sparse_attn_stats(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_count), _ptr(kept_idx),
            float(sm_scale), _ptr(residual), rs, _ptr(out), _ptr(lse), _ptr(ws), nbytes,
            _stream(stream)), "recap_block_sparse_attn_stats")
        return out, lse
    check(_lib.load().recap_block_sparse_attn(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_count), _ptr(kept_idx),
        float(sm_scale), _ptr(residual), rs, _ptr(out), _ptr(ws), nbytes, _stream(stream)),
        "recap_block_sparse_attn")
    return out


@_on_stream
def recap_dense_attn(desc: RecapDesc, q, k, v, sm_scale: Optional[float] = None,
                     kept_count=None, kept_idx=None, out=None, residual_out=None,
                     capture: bool = False, workspace=None, stream=None,
                     want_lse: bool = False, want_kept_mass: bool = False):
    """Dense attention; with capture=True (or residual_out) also R = O_dense - O_sparse.
    Returns out, or (out, residual) when capturing. With want_lse / want_kept_mass the call
    goes through recap_dense_attn_stats and returns a dict with the keys out, residual (or
    None), lse and kept_mass (or None), each row statistic fp32 [B,H,N]."""
    _same_layout(desc, q, k, v, out, residual_out)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    if out is None:
        out = _like_out(q)
    capture = capture or residual_out is not None
    if capture and residual_out is None:
        residual_out = _like_out(q)
    stats = want_lse or want_kept_mass
    op = _lib.OP_DENSE_CAPTURE if (capture or want_kept_mass) else _lib.OP_DENSE
    ws, nbytes = _workspace(op, desc, q.device, workspace)
    if stats:
        lse = _row_stat(desc, None, q.device)
        kmass = _row_stat(desc, None, q.device) if want_kept_mass else None
        check(_lib.load().recap_dense_attn_stats(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), float(sm_scale), _ptr(kept_count),
            _ptr(kept_idx), _ptr(out), _ptr(residual_out), _ptr(lse), _ptr(kmass), _ptr(ws),
            nbytes, _stream(stream)), "recap_dense_attn_stats")
        return {"out": out, "residual": residual_out, "lse": lse, "kept_mass": kmass}
    check(_lib.load().recap_dense_attn(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), float(sm_scale), _ptr(kept_count),
        _ptr(kept_idx), _ptr(out), _ptr(residual_out), _ptr(ws), nbytes, _stream(stream)),
        "recap_dense_attn")
    return (out, residual_out) if capture else out


@_on_stream
def recap_block_sparse_attn_stats(desc: RecapDesc, q, k, v, kept_count, kept_idx,
                                  sm_scale: Optional[float] = None, residual=None,
                                  res_scale=None, out=None, lse=None, workspace=None,
                                  stream=None):
    """(out, lse): recap_block_sparse_attn plus the fp32 [B,H,N] log-sum-exp of the scores
    over each query's kept keys."""
    return recap_block_sparse_attn(desc, q, k, v, kept_count, kept_idx, sm_scale, residual,
                                   res_scale, out, workspace, stream, lse=lse, want_lse=True)


@_on_stream
def recap_dense_attn_stats(desc: RecapDesc, q, k, v, sm_scale: Optional[float] = None,
                           kept_count=None, kept_idx=None, out=None, residual_out=None,
                           capture: bool = False, want_kept_mass: bool = False,
                           workspace=None, stream=None):
    """recap_dense_attn plus the dense log-sum-exp and, with the kept lists and
    want_kept_mass, the kept share of each row's dense attention mass; returns the dict of
    recap_dense_attn(..., want_lse=True)."""
    return recap_dense_attn(desc, q, k, v, sm_scale, kept_count, kept_idx, out, residual_out,
                            capture, workspace, stream, want_lse=True,
                            want_kept_mass=want_kept_mass)


def _means_shape(desc: RecapDesc):
    return (desc.batch, desc.heads, num_blocks(desc), desc.head_dim)


def _check_means(desc: RecapDesc, *ts) -> None:
    for t in ts:
        if t.dtype != torch.float32 or tuple(t.shape) != _means_shape(desc) or \
                not t.is_contiguous():
            raise ValueError("block means are contiguous fp32 [B, H, M, D]")


@_on_stream
def recap_block_means(desc: RecapDesc, q, k, qbar=None, kbar=None, stream=None):
    """(Q̄, K̄): fp32 [B,H,M,D] block means (recap_block_means)."""
    _same_layout(desc, q, k)
    if qbar is None:
        qbar = torch.empty(_means_shape(desc), dtype=torch.float32, device=q.device)
    if kbar is None:
        kbar = torch.empty(_means_shape(desc), dtype=torch.float32, device=q.device)
    _check_means(desc, qbar, kbar)
    check(_lib.load().recap_block_means(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(qbar),
                                        _ptr(kbar), _stream(stream)), "recap_block_means")
    return qbar, kbar


@_on_stream
def recap_scores_from_means(desc: RecapDesc, qbar, kbar, sm_scale: Optional[float] = None,
                            cand_count=None, cand_idx=None, probs=None, stream=None):
    """fp32 [B,H,M,M] block-pair softmax from given means; with candidate lists, each row's
    softmax over its candidates at the candidate positions (recap_scores_from_means)."""
    _check_means(desc, qbar, kbar)
    M = num_blocks(desc)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    if probs is None:
        probs = torch.empty((desc.batch, desc.heads, M, M), dtype=torch.float32,
                            device=qbar.device)
    check(_lib.load().recap_scores_from_means(ctypes.byref(desc), _ptr(qbar), _ptr(kbar),
                                              float(sm_scale), _ptr(cand_count), _ptr(cand_idx),
                                              _ptr(probs), _stream(stream)),
          "recap_scores_from_means")
    return probs


@_on_stream
def recap_topp_mask_cand(desc: RecapDesc, probs, cand_count, cand_idx, top_p, kept_count=None,
                         kept_idx=None, want_mask: bool = False, want_mass: bool = False,
                         stream=None):
    """Top-p over each row's candidate distribution: (count, idx, mask|None, mass|None) with
    block indices (recap_topp_mask_cand)."""
    M = num_blocks(desc)
    dev = probs.device
    if kept_count is None:
        kept_count = torch.empty((desc.batch, desc.heads, M), dtype=torch.int32, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((desc.batch, desc.heads, M, M), dtype=torch.int32, device=dev)
    mask = torch.empty((desc.batch, desc.heads, M, M), dtype=torch.uint8, device=dev) \
        if want_mask else None
    mass = torch.empty((desc.batch, desc.heads, M), dtype=torch.float32, device=dev) \
        if want_mass else None
    tp = _host_floats(top_p, desc.heads, "top_p")
    check(_lib.load().recap_topp_mask_cand(ctypes.byref(desc), _ptr(probs), _ptr(cand_count),
                                           _ptr(cand_idx), tp, _ptr(kept_count),
                                           _ptr(kept_idx), _ptr(mask), _ptr(mass),
                                           _stream(stream)), "recap_topp_mask_cand")
    return kept_count, kept_idx, mask, mass


@_on_stream
def recap_mean_drift(desc: RecapDesc, qbar, kbar, qbar_ref, kbar_ref, drift=None, stream=None):
    """fp32 [B,H,2]: relative Frobenius change of Q̄ and of K̄ against a reference step."""
    _check_means(desc, qbar, kbar, qbar_ref, kbar_ref)
    if drift is None:
        drift = torch.empty((desc.batch, desc.heads, 2), dtype=torch.float32, device=qbar.device)
    check(_lib.load().recap_mean_drift(ctypes.byref(desc), _ptr(qbar), _ptr(kbar),
                                       _ptr(qbar_ref), _ptr(kbar_ref), _ptr(drift),
                                       _stream(stream)), "recap_mean_drift")
    return drift


@_on_stream
def recap_tail_estimate(desc: RecapDesc, q, k, v, kept_count, kept_idx,
                        sm_scale: Optional[float] = None, tail_lse=None, tail_out=None,
                        workspace=None, stream=None, moments: bool = False):
    """Coarse tail from block means over each query block's omitted key blocks: (tail_lse fp32
    [B,H,N], tail_out fp32 [B,H,N,D] contiguous). moments: the key-variance and value-key
    covariance refinements (RECAP_TAIL_MOMENTS)."""
    _same_layout(desc, q, k, v)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    tail_lse = _row_stat(desc, tail_lse, q.device)
    tail_out = _row_vec(desc, tail_out, q.device, "tail_out")
    ws, nbytes = _workspace(_lib.OP_TAIL, desc, q.device, workspace)
    check(_lib.load().recap_tail_estimate(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_count), _ptr(kept_idx),
        float(sm_scale), _lib.TAIL_MOMENTS if moments else 0, _ptr(tail_lse), _ptr(tail_out),
        _ptr(ws), nbytes, _stream(stream)),
        "recap_tail_estimate")
    return tail_lse, tail_out


def _row_vec(desc: RecapDesc, given: Optional[torch.Tensor], device, what: str):
    shp = (desc.batch, desc.heads, desc.seq, desc.head_dim)
    if given is None:
        return torch.empty(shp, dtype=torch.float32, device=device)
    if given.dtype != torch.float32 or tuple(given.shape) != shp or not given.is_contiguous():
        raise ValueError(f"{what} is contiguous fp32 [B, H, N, D]")
    return given


@_on_stream
def recap_dense_attn_tail(desc: RecapDesc, q, k, v, kept_count, kept_idx,
                          sm_scale: Optional[float] = None, out=None, tail_dlse=None,
                          tail_dout=None, workspace=None, stream=None, moments: bool = False):
    """Dense refresh that also writes the tail discrepancy on the kept set: (out bf16,
    tail_dlse fp32 [B,H,N], tail_dout fp32 [B,H,N,D]); moments as recap_tail_estimate."""
    _same_layout(desc, q, k, v, out)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    out = _like_out(q) if out is None else out
    tail_dout = _row_vec(desc, tail_dout, q.device, "tail_dout")
    tail_dlse = _row_stat(desc, tail_dlse, q.device)
    ws, nbytes = _workspace(_lib.OP_DENSE_TAIL, desc, q.device, workspace)
    check(_lib.load().recap_dense_attn_tail(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), float(sm_scale),
        _lib.TAIL_MOMENTS if moments else 0, _ptr(kept_count), _ptr(kept_idx), _ptr(out),
        _ptr(tail_dlse), _ptr(tail_dout), _ptr(ws), nbytes, _stream(stream)),
        "recap_dense_attn_tail")
    return out, tail_dlse, tail_dout


@_on_stream
def recap_block_sparse_attn_tail(desc: RecapDesc, q, k, v, kept_count, kept_idx,
                                 sm_scale: Optional[float] = None, tail_dlse=None,
                                 tail_dout=None, out=None, workspace=None, stream=None,
                                 moments: bool = False):
    """Block-sparse attention merged by log-mass with the fresh coarse tail plus the cached
    discrepancy (both or neither of tail_dlse, tail_dout); bf16 out in q's layout; moments as
    recap_tail_estimate (the refresh that cached the discrepancy must use the same)."""
    _same_layout(desc, q, k, v, out)
    if (tail_dlse is None) != (tail_dout is None):
        raise ValueError("tail_dlse and tail_dout go together")
    if tail_dlse is not None:
        _row_stat(desc, tail_dlse, q.device)
        _row_vec(desc, tail_dout, q.device, "tail_dout")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    out = _like_out(q) if out is None else out
    ws, nbytes = _workspace(_lib.OP_SPARSE_TAIL, desc, q.device, workspace)
    check(_lib.load().recap_block_sparse_attn_tail(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_count), _ptr(kept_idx),
        float(sm_scale), _lib.TAIL_MOMENTS if moments else 0, _ptr(tail_dlse), _ptr(tail_dout),
        _ptr(out), _ptr(ws), nbytes, _stream(stream)), "recap_block_sparse_attn_tail")
    return out


@_on_stream
def recap_block_sparse_attn_fp8(desc: RecapDesc, q, k, v, kept_count, kept_idx,
                                sm_scale: Optional[float] = None, residual=None, res_scale=None,
                                out=None, workspace=None, stream=None, lse=None,
                                want_lse: bool = False):
    """Block-sparse attention with MXFP8 products (bf16 in and out). Returns out, or
    (out, lse) with want_lse / lse given."""
    _same_layout(desc, q, k, v, out, residual)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(desc.head_dim)
    out = _like_out(q) if out is None else out
    rs = None
    if residual is not None:
        if res_scale is None:
            raise ValueError("res_scale is required with a residual")
        rs = _host_floats(res_scale, desc.heads, "res_scale")
    if want_lse or lse is not None:
        lse = _row_stat(desc, lse, q.device)
    ws, nbytes = _workspace(_lib.OP_SPARSE_FP8, desc, q.device, workspace)
    check(_lib.load().recap_block_sparse_attn_fp8(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(kept_count), _ptr(kept_idx),
        float(sm_scale), _ptr(residual), rs, _ptr(out), _ptr(lse), _ptr(ws), nbytes,
        _stream(stream)), "recap_block_sparse_attn_fp8")
    return (out, lse) if lse is not None else out


@_on_stream
def recap_mx_quantize(desc: RecapDesc, x, along_tokens: bool = False, stream=None):
    """MXFP8 encoding of a bf16 [B,H,N,D] view: (codes uint8 [B,H,N,D], scales uint8:
    [B,H,N,D/32] per token, or [B,H,ceil(N/32),D] per 32-token group with along_tokens)."""
    _same_layout(desc, x)
    B, H, N, D = desc.batch, desc.heads, desc.seq, desc.head_dim
    codes = torch.empty((B, H, N, D), dtype=torch.uint8, device=x.device)
    shp = (B, H, -(-N // 32), D) if along_tokens else (B, H, N, D // 32)
    scales = torch.empty(shp, dtype=torch.uint8, device=x.device)
    check(_lib.load().recap_mx_quantize(ctypes.byref(desc), _ptr(x), int(bool(along_tokens)),
                                        _ptr(codes), _ptr(scales), _stream(stream)),
          "recap_mx_quantize")
    return codes, scales


@_on_stream
def sparse_step(desc: RecapDesc, q, k, v, top_p, sm_scale: Optional[float] = None,
                residual=None, res_scale=None, out=None, stream=None):
    """One corrected sparse attention call: block scores -> top-p -> sparse attention
    (+ epilogue). Returns (out, kept_count, kept_idx)."""
    probs = recap_block_scores(desc, q, k, sm_scale, stream=stream)
    count, idx, _, _ = recap_topp_mask(desc, probs, top_p, stream=stream)
    o = recap_block_sparse_attn(desc, q, k, v, count, idx, sm_scale, residual, res_scale, out,
                                stream=stream)
    return o, count, idx
