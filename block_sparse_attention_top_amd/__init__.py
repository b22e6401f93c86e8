"""Block-sparse top-p attention with a cached-residual epilogue for MI355X (gfx950).

The compute path is the HIP library librecap.so (C ABI in include/recap.h); this package only
marshals torch device tensors into its entry points. Functions carry the C names:
recap_block_scores, recap_topp_mask, recap_block_sparse_attn, recap_dense_attn, and the
row-statistics variants recap_block_sparse_attn_stats and recap_dense_attn_stats, and the
mask-reuse building blocks recap_block_means, recap_scores_from_means, recap_topp_mask_cand and
recap_mean_drift, the tail reconstruction recap_tail_estimate, recap_dense_attn_tail and
recap_block_sparse_attn_tail, the FP8 variant recap_block_sparse_attn_fp8 with its encoder
recap_mx_quantize, and recap_block_scores_noalloc (block scores with a fixed library-held
scratch, for callers that cannot allocate).
"""
from ._lib import RecapDesc, RecapError, load  # noqa: F401
from .ops import (  # noqa: F401
    make_desc,
    recap_block_means,
    recap_block_scores,
    recap_block_scores_noalloc,
    recap_block_sparse_attn,
    recap_block_sparse_attn_fp8,
    recap_block_sparse_attn_stats,
    recap_block_sparse_attn_tail,
    recap_dense_attn,
    recap_dense_attn_stats,
    recap_dense_attn_tail,
    recap_mean_drift,
    recap_mx_quantize,
    recap_scores_from_means,
    recap_tail_estimate,
    recap_topp_mask,
    recap_topp_mask_cand,
    recap_workspace_size,
    sparse_step,
)
