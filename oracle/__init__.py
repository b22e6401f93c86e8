"""CPU oracle (TEST INFRASTRUCTURE ONLY).

A plain float64 definition of block-sparse top-p attention with a cached-residual epilogue,
written from the pages' description of the method. Only `tests/`, the package smoke check
(`__graft_entry__.smoke`) and the benchmark's `cpu_baseline` leg may import it. It shares no
code with the HIP library and never imports it.

Parity status per function (pins live in tests/test_oracle_pins.py):
  block_partition, block_mean_pool, block_scores, softmax_rows, topp_select, kept_lists,
  mask_from_lists, masked_attention, dense_attention, residual_epilogue, dense_with_capture,
  attention_lse, kept_attention_mass, candidate_scores, topp_select_candidates, mean_drift,
  coarse_tail (zeroth order and with moments), block_key_variance,
  pooled_value_key_covariance, exact_tail, tail_discrepancy, merge_attention, tail_reconstruction,
  e4m3_round, mx_scale_exponents, mx_quantize, masked_attention_mx, block_sparsity, kept_flops:
  pinned (closed forms, invariants, library special cases, brute force, planted mutants).
  The conventions the pages leave open (scale of the pooled logits, no log-block-size term,
  tie order, inclusive threshold) are readings; the pins fix the oracle to those readings.
"""
from .oracle import (  # noqa: F401
    attention_lse,
    block_key_variance,
    block_mean_pool,
    block_partition,
    block_scores,
    block_sparsity,
    candidate_scores,
    coarse_tail,
    dense_attention,
    dense_with_capture,
    e4m3_round,
    exact_tail,
    kept_attention_mass,
    kept_flops,
    kept_lists,
    mask_from_lists,
    masked_attention,
    masked_attention_mx,
    mean_drift,
    merge_attention,
    pooled_value_key_covariance,
    mx_quantize,
    mx_scale_exponents,
    residual_epilogue,
    softmax_rows,
    tail_discrepancy,
    tail_reconstruction,
    topp_select,
    topp_select_candidates,
)
