#!/usr/bin/env python3
"""Benchmark of one attention layer's hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input. For the default
workload (Wan2.1-14B-like 720p layer: B=1, H=40, D=128, N=75,600 tokens = 21 x 45 x 80, block
64, top-p 0.95) a step is:
  * a dense refresh on X_0: block scores -> top-p -> dense attention with residual capture;
  * three sparse calls on drifted inputs X_1..X_3: block scores -> top-p -> block-sparse
    attention with the fused epilogue O + 1.0 * R using the captured residual.
Other workloads (--workload) run one sparse call per step (+ epilogue where configured).

Reported (one JSON line): value = computed-block TFLOP/s of the block-sparse attention call
(kept-block FLOPs over the mean HIP-event time of recap_block_sparse_attn, the metric's subject),
ms per sparse call (mask prediction + attention + epilogue) and per step, the roofline of the
sparse attention kernel (roofline), of the dense refresh (roofline_refresh) and of the
mask-prediction kernels (roofline_mask), and the CPU oracle timed on a bounded sample of the
same sparse call (extrapolated to the whole call).
With --tail, RECAP's tail-reconstruction calls are also timed (a "tail" object, outside the
step and its figures); with --fp8, the MXFP8 variant of the sparse calls (an "fp8" object);
with --probe-peaks, the rates a plain bf16 GEMM (torch's library GEMM) and a device copy reach
on the same box (a "probe" object), as practical ceilings next to the spec peaks.
Inputs are resident in HBM before the timed region. Timing uses HIP events on the stream the
library launches on (torch's current stream).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn ms/call + computed-block TFLOP/s (% bf16 MFMA peak), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
CSRC = os.path.join(ROOT, "block_sparse_attention_top_amd", "csrc")
# the sources each kernel group is compiled from (the key of its counter figures)
KERNEL_SOURCES = {
    "attn": [os.path.join(CSRC, f) for f in ("attn_kernels.hip", "attn_device.h", "common.h")],
    "mask": [os.path.join(CSRC, f) for f in ("mask_kernels.hip", "common.h")],
    "fp8": [os.path.join(CSRC, f) for f in ("attn_fp8.hip", "attn_device.h", "common.h")],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def src_hash(paths):
    """Hash of kernel sources with comments and whitespace removed, so that counter figures
    recorded for them stay valid across documentation-only edits."""
    h = hashlib.sha256()
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on this
    workload and the kernel source is unchanged since; else None."""
    try:
        table = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = table.get(kernel_key)
    if not ent or ent.get("workload") != workload:
        return None
    srcs = KERNEL_SOURCES.get(ent.get("source"))
    if srcs is None or ent.get("source_sha") != src_hash(srcs):
        return None
    return ent.get("bytes_per_launch")


def kept_token_pairs(count, idx, N, block):
    """sum over kept (i, j) of n_i * n_j, from kept lists (torch tensors, on device)."""
    import torch

    B, H, M = count.shape
    n = torch.full((M,), block, dtype=torch.float64, device=count.device)
    n[-1] = N - (M - 1) * block
    cols = torch.arange(M, device=count.device).view(1, 1, 1, M)
    valid = cols < count.unsqueeze(-1)
    nj = torch.where(valid, n[idx.clamp(0, M - 1).long()], torch.zeros((), dtype=torch.float64,
                                                                       device=count.device))
    per_row = nj.sum(-1)  # [B, H, M]
    return float((per_row * n.view(1, 1, M)).sum().item())


def host_threads():
    """Host cores for the oracle: the CPUs this process may run on (sched_getaffinity), capped
    by OMP_NUM_THREADS when the environment sets it (the host share of one GPU on a shared
    box). Returns (threads used, affinity CPU count)."""
    aff = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS")
    n = min(aff, int(cap)) if cap and cap.isdigit() and int(cap) > 0 else aff
    return n, aff


def cpu_baseline(cfg, q, k, v, p, seconds, call_flops):
    """The oracle as it stands (fp64 numpy, never tuned for this), timed on the host on a
    bounded sample of one sparse call of the same workload, head 0:
      * mask prediction (block scores, top-p) of the head in full: t_mask;
      * sparse attention and the residual epilogue on query blocks spread over the sequence
        until the time budget is spent: kept FLOPs F_s in t_att.
    value = F_s / t_att, the oracle's computed-block rate (the unit of the GPU value). The
    whole call is extrapolated as H * t_mask + call_flops * t_att / F_s and labelled so."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import oracle as O

    threads, aff = host_threads()
    s = cfg.head_dim ** -0.5
    M, blk, N, H = cfg.num_blocks, cfg.block, cfg.seq, cfg.heads
    with threadpool_limits(limits=threads):
        q64, k64, v64 = (synth.to_f64(x[:, :1]) for x in (q, k, v))
        r64 = synth.to_f64(synth.random_bf16((1, 1, N, cfg.head_dim), 4, 0.05))
        t0 = time.perf_counter()
        probs = O.block_scores(q64, k64, blk, s)
        mask = O.topp_select(probs, p[:1])["mask"]
        t_mask = time.perf_counter() - t0
        order = np.argsort((np.arange(M) * 0.6180339887) % 1.0)  # spread over the sequence
        done = []
        t1 = time.perf_counter()
        for i in order:
            o = O.masked_attention(q64, k64, v64, blk, s, mask, rows=[(0, 0, int(i))])
            lo, hi = int(i) * blk, min(N, (int(i) + 1) * blk)
            O.residual_epilogue(o[:, :, lo:hi], r64[:, :, lo:hi], [1.0])
            done.append(int(i))
            if time.perf_counter() - t1 > seconds:
                break
        t_att = time.perf_counter() - t1
    sampled = np.zeros_like(mask)
    sampled[0, 0, done] = mask[0, 0, done]
    flops = O.kept_flops(sampled, N, blk, cfg.head_dim)
    rows_done = len(done)
    call_s = H * t_mask + call_flops * t_att / flops
    return {
        "value": flops / t_att / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"head 0 of {cfg.name}: mask prediction for all {M} query blocks "
                   f"({t_mask:.1f} s), then sparse attention + epilogue on {rows_done} of {M} "
                   f"query blocks ({t_att:.1f} s); value = computed-block FLOPs of those blocks "
                   f"/ their time; fp64 numpy on {threads} threads "
                   f"({aff} CPUs in the affinity mask) of {cpu_model()}"),
        "extrapolated": {"ms_per_sparse_call": call_s * 1e3,
                         "rule": "H x head-0 mask time + call FLOPs x attention s/FLOP"},
        "seconds": t_mask + t_att,
    }


def bench_tail(bsa, cfg, desc, dev_inputs, counts, idxs, s, avg, args, roof):
    """RECAP's tail reconstruction timed apart from the step, on the same inputs and kept
    lists, zeroth order and with the moment refinements: the refresh with the discrepancy
    (recap_dense_attn_tail on X_0), each drifted sparse call merged with the fresh coarse tail
    plus that discrepancy (recap_block_sparse_attn_tail on X_1..), and the coarse estimate alone
    (recap_tail_estimate on X_1). The roofline is the zeroth-order estimate's: 4 D FLOPs per
    (query token, omitted key block) pair over its call time. Accuracy at the drifted step X_1
    (the refresh's kept lists reused, as RECAP reuses them between refreshes): relative L2 and
    largest error against the dense output on X_1 of the plain sparse output, of the merge with
    the coarse tail alone and of the merge with coarse tail + discrepancy."""
    import numpy as np
    import torch

    B, H, N, D, blk, M = cfg.batch, cfg.heads, cfg.seq, cfg.head_dim, cfg.block, cfg.num_blocks
    dev = dev_inputs[0][0].device
    d_lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    d_o = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
    t_lse = torch.empty_like(d_lse)
    t_out = torch.empty_like(d_o)
    out = torch.empty_like(dev_inputs[0][0])
    ws_m = torch.empty(bsa.recap_workspace_size(7, desc), dtype=torch.uint8, device=dev)
    ws_e = torch.empty(bsa.recap_workspace_size(5, desc), dtype=torch.uint8, device=dev)

    def run(events, mom):
        def timed(name, fn):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            if events is not None:
                events.append((name, e0, e1))
        q0, k0, v0 = dev_inputs[0]
        timed("refresh", lambda: bsa.recap_dense_attn_tail(desc, q0, k0, v0, counts[0], idxs[0], s,
                                                           out, d_lse, d_o, ws_m, moments=mom))
        for ci in range(1, len(dev_inputs)):
            qq, kk, vv = dev_inputs[ci]
            timed("sparse", lambda: bsa.recap_block_sparse_attn_tail(
                desc, qq, kk, vv, counts[ci], idxs[ci], s, d_lse, d_o, out, ws_m, moments=mom))
        q1, k1, v1 = dev_inputs[1]
        timed("estimate", lambda: bsa.recap_tail_estimate(desc, q1, k1, v1, counts[1], idxs[1],
                                                          s, t_lse, t_out, ws_e, moments=mom))

    res = {}
    for mom in (False, True):
        tag = "moments" if mom else "zeroth"
        log(f"tail reconstruction ({tag}): warmup 1, timing")
        run(None, mom)
        torch.cuda.synchronize()
        events = []
        for _ in range(max(1, args.steps // 2)):
            run(events, mom)
        torch.cuda.synchronize()
        per = {}
        for name, e0, e1 in events:
            per.setdefault(name, []).append(e0.elapsed_time(e1))
        t = {k: float(np.median(v)) for k, v in per.items()}
        res[tag] = {"ms_refresh_call_with_discrepancy": t["refresh"],
                    "ms_sparse_call_with_tail": t["sparse"], "ms_tail_estimate": t["estimate"],
                    "refresh_overhead_ms": t["refresh"] - avg["refresh.attn"],
                    "sparse_overhead_ms": t["sparse"] - avg["sparse.attn"],
                    "n_timed": {k: len(v) for k, v in per.items()}}
        if not mom:
            # omitted (query token, key block) pairs of the estimate's kept lists
            starts = torch.arange(M, device=dev) * blk
            n_q = (torch.clamp(starts + blk, max=N) - starts).double()
            omitted = ((M - counts[1].double()) * n_q).sum().item()
            est_tflops = 4.0 * D * omitted / (t["estimate"] * 1e-3) / 1e12
            res["roofline_estimate"] = roof(
                "pool + tail_keys + kept_bits + tail_kernel (one zeroth-order recap_tail_estimate "
                "call; algorithmic FLOPs on omitted pairs only)", est_tflops, traffic_key="tail")

    # accuracy at the drifted step X_1 with the refresh's kept lists and discrepancy
    log("tail reconstruction: accuracy at the drifted step")
    q0, k0, v0 = dev_inputs[0]
    q1, k1, v1 = dev_inputs[1]
    c0, i0 = counts[0], idxs[0]
    ref = bsa.recap_dense_attn(desc, q1, k1, v1, s).float()
    nref = ref.norm().item()

    def err(x):
        e = x.float() - ref
        return {"rel_l2": e.norm().item() / nref, "max_abs": e.abs().max().item()}

    acc = {"reference": "dense attention on X_1 (recap_dense_attn)",
           "kept_lists": "the refresh's (X_0) lists reused at X_1",
           "sparse_only": err(bsa.recap_block_sparse_attn(desc, q1, k1, v1, c0, i0, s))}
    for mom in (False, True):
        tag = "moments" if mom else "zeroth"
        bsa.recap_dense_attn_tail(desc, q0, k0, v0, c0, i0, s, out, d_lse, d_o, ws_m, moments=mom)
        acc[f"coarse_tail_{tag}"] = err(bsa.recap_block_sparse_attn_tail(
            desc, q1, k1, v1, c0, i0, s, None, None, None, ws_m, moments=mom))
        acc[f"coarse_tail_plus_discrepancy_{tag}"] = err(bsa.recap_block_sparse_attn_tail(
            desc, q1, k1, v1, c0, i0, s, d_lse, d_o, None, ws_m, moments=mom))
    torch.cuda.synchronize()
    res["accuracy_at_drifted_step"] = acc
    return res


def bench_reuse(bsa, cfg, desc, x0, x1, p, s, args, tau):
    """Mask reuse across steps (NEXT-3), on a reference step X_0 and a drifted step X_1 of the
    same layer, timed apart from the step:
      * fresh: the full mask prediction at X_1 (recap_block_scores + recap_topp_mask);
      * gate: block means at X_1 and their relative drift against X_0's (recap_block_means +
        recap_mean_drift); when the largest drift is below tau the step reuses X_0's kept
        lists and skips scores and top-p (Temporal Mask Reuse in the head-wise adaptive
        abstract: skip mask prediction on low query-key drift);
      * candidates: block means at X_1, scores over candidate lists taken at X_0 with a looser
        threshold p_c = 1 - (1 - p) / 4 (recap_scores_from_means with the lists), then top-p
        at p over each row's candidate distribution (recap_topp_mask_cand) (GSRS abstract:
        search restricted to an early candidate set).
    Agreement with the fresh mask at X_1: share of equal block pairs, and the fresh block
    probability mass the reused / restricted kept sets carry (against p)."""
    import numpy as np
    import torch

    B, H, M = cfg.batch, cfg.heads, cfg.num_blocks
    dev = x0[0].device
    (q0, k0), (q1, k1) = x0, x1
    plist = p.tolist()
    pc = [min(1.0, 1.0 - (1.0 - float(v)) / 4.0) for v in plist]
    means = lambda q, k: bsa.recap_block_means(desc, q, k)  # noqa: E731
    qb0, kb0 = means(q0, k0)
    pr0 = bsa.recap_scores_from_means(desc, qb0, kb0, s)
    c0, i0, _, _ = bsa.recap_topp_mask(desc, pr0, plist)
    cc, ci, _, _ = bsa.recap_topp_mask(desc, pr0, pc)
    del pr0
    probs = torch.empty((B, H, M, M), dtype=torch.float32, device=dev)
    ws = torch.empty(bsa.recap_workspace_size(0, desc), dtype=torch.uint8, device=dev)
    qb1 = torch.empty_like(qb0)
    kb1 = torch.empty_like(kb0)
    drift = torch.empty((B, H, 2), dtype=torch.float32, device=dev)
    c1, i1 = torch.empty_like(c0), torch.empty_like(i0)
    ccand, icand = torch.empty_like(c0), torch.empty_like(i0)

    legs = {
        "fresh": lambda: (bsa.recap_block_scores(desc, q1, k1, s, probs, ws),
                          bsa.recap_topp_mask(desc, probs, plist, c1, i1)),
        "gate": lambda: (bsa.recap_block_means(desc, q1, k1, qb1, kb1),
                         bsa.recap_mean_drift(desc, qb1, kb1, qb0, kb0, drift)),
        "candidates": lambda: (bsa.recap_block_means(desc, q1, k1, qb1, kb1),
                               bsa.recap_scores_from_means(desc, qb1, kb1, s, cc, ci, probs),
                               bsa.recap_topp_mask_cand(desc, probs, cc, ci, plist, ccand,
                                                        icand)),
    }
    ms = {}
    for name, fn in legs.items():
        fn()
        torch.cuda.synchronize()
        ev = []
        for _ in range(max(3, args.steps)):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms[name] = float(np.median([a.elapsed_time(b) for a, b in ev]))
    # the gate's decision needs the drift on the host: one synchronisation per gated step
    # (wall time of the gate's launches, its kernels and the read of the largest drift, after a
    # warm-up of the reduction)
    legs["gate"]()
    float(drift.max().item())
    t0 = time.perf_counter()
    legs["gate"]()
    dmax = float(drift.max().item())
    ms["gate_with_host_decision"] = (time.perf_counter() - t0) * 1e3
    # masks: fresh (c1, i1 from the last fresh run), reused (c0, i0), restricted (ccand, icand)
    legs["fresh"]()
    legs["candidates"]()
    bsa.recap_block_scores(desc, q1, k1, s, probs, ws)
    torch.cuda.synchronize()

    def mask_of(cnt, idx):
        cols = torch.arange(M, device=dev).view(1, 1, 1, M)
        valid = cols < cnt.unsqueeze(-1).long()
        m = torch.zeros((B, H, M, M), dtype=torch.bool, device=dev)
        m.scatter_(-1, torch.where(valid, idx.long(), torch.zeros_like(idx.long())), valid)
        return m

    fresh = mask_of(c1, i1)
    ptens = torch.tensor(plist, device=dev, dtype=torch.float64).view(1, H, 1)

    def agreement(m):
        mass = (probs.double() * m).sum(-1)
        return {"equal_block_pairs": float((m == fresh).double().mean().item()),
                "mean_fresh_mass_kept": float(mass.mean().item()),
                "rows_below_p": float((mass < ptens - 1e-4).double().mean().item()),
                "kept_blocks_per_row": float(m.sum(-1).double().mean().item())}

    res = {"threshold_tau": tau, "max_relative_drift": dmax, "reuse_chosen": dmax < tau,
           "candidate_threshold": pc[0] if len(set(pc)) == 1 else "1 - (1 - p_h) / 4",
           "ms": ms,
           "ms_saved_by_reuse": ms["fresh"] - ms["gate"],
           "ms_saved_by_candidates": ms["fresh"] - ms["candidates"],
           "fresh": {"kept_blocks_per_row": float(fresh.sum(-1).double().mean().item())},
           "reused_mask": agreement(mask_of(c0, i0)),
           "candidate_mask": agreement(mask_of(ccand, icand))}
    return res


def bench_fp8(bsa, cfg, desc, dev_inputs, counts, idxs, s, res, res_scale, avg, sparse_flops,
              args, roof):
    """The MXFP8 variant of the step's sparse calls, timed apart from the step on the same
    inputs, kept lists and epilogue: recap_block_sparse_attn_fp8, which quantises Q and packs
    the K / V tiles (E4M3 codes with per-32 power-of-two scales) before the attention kernel.
    The roofline is the whole call's algorithmic FLOPs against the fp8 MFMA peak."""
    import numpy as np
    import torch

    dev = dev_inputs[0][0].device
    out = torch.empty_like(dev_inputs[0][0])
    ws = torch.empty(bsa.recap_workspace_size(8, desc), dtype=torch.uint8, device=dev)
    first = 1 if cfg.refresh_then_sparse else 0

    def run(events):
        for ci in range(first, len(dev_inputs)):
            qq, kk, vv = dev_inputs[ci]
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            bsa.recap_block_sparse_attn_fp8(desc, qq, kk, vv, counts[ci], idxs[ci], s, res,
                                            res_scale if res is not None else None, out,
                                            workspace=ws)
            e1.record()
            if events is not None:
                events.append((e0, e1))

    log("fp8 sparse calls: warmup 1, timing")
    run(None)
    torch.cuda.synchronize()
    events = []
    for _ in range(max(1, args.steps // 2)):
        run(events)
    torch.cuda.synchronize()
    ms = [e0.elapsed_time(e1) for e0, e1 in events]
    t = float(np.median(ms))
    tflops = float(np.mean(sparse_flops)) / (t * 1e-3) / 1e12
    return {
        "ms_sparse_attn_fp8": t,
        "ms_sparse_attn_fp8_min": float(np.min(ms)),
        "speedup_vs_bf16_attn": avg["sparse.attn"] / t,
        "sparse_attn_fp8_tflops": tflops,
        "n_timed": len(ms),
        "roofline_fp8": roof("mx_rows + mx_k_tiles + mx_v_tiles + attn_mx_kernel<D=128> (one "
                             "recap_block_sparse_attn_fp8 call; traffic: attn_mx_kernel)", tflops,
                             peak=PEAK_FP8_TFLOPS, traffic_key="fp8"),
    }


def probe_peaks(dev, bsa):
    """Practical ceilings on this machine: a plain bf16 GEMM (8192^3, contiguous 2-D operands,
    torch's library GEMM), a 2 GiB device-to-device copy, and dense attention at 8 heads of the
    720p shape (B=1, N=75,600, D=128, bf16) through this library's recap_dense_attn and through
    torch's scaled_dot_product_attention restricted to its flash and memory-efficient backends
    (no math fallback), each timed with HIP events over several repetitions after a warm-up."""
    import numpy as np
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            out.append(e0.elapsed_time(e1))
        return float(np.median(out))

    n = 8192
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), device=dev).to(torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    ms_gemm = timed(lambda: torch.matmul(a, b, out=c), 20)
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms_copy = timed(lambda: dst.copy_(src), 20)
    gemm = 2.0 * n ** 3 / (ms_gemm * 1e-3) / 1e12
    copy = 2.0 * nbytes / (ms_copy * 1e-3) / 1e9  # read + write
    del a, b, c, src, dst

    # dense attention, this library against torch's fused attention backends
    ah, an, ad = 8, 75600, 128
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    q, k, v = (torch.randn((1, ah, an, ad), generator=g, device=dev).to(torch.bfloat16)
               for _ in range(3))
    aflops = 4.0 * ah * an * an * ad
    out = torch.empty_like(q)
    desc = bsa.make_desc(q, 64)
    attn = {"shape": {"batch": 1, "heads": ah, "seq": an, "head_dim": ad}}
    ms = timed(lambda: bsa.recap_dense_attn(desc, q, k, v, None, None, None, out), 3)
    attn["recap_dense_attn_tflops"] = aflops / (ms * 1e-3) / 1e12
    from torch.nn.attention import SDPBackend, sdpa_kernel
    for name, backend in (("flash", SDPBackend.FLASH_ATTENTION),
                          ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([backend]):
                ms = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v), 3)
            attn[f"torch_sdpa_{name}_tflops"] = aflops / (ms * 1e-3) / 1e12
        except RuntimeError as e:  # backend not built for this device: no fallback is timed
            attn[f"torch_sdpa_{name}_tflops"] = None
            log(f"torch SDPA {name} backend unavailable: {str(e)[:120]}")
    return {"gemm_bf16_tflops": gemm, "gemm_frac_bf16_peak": gemm / PEAK_BF16_TFLOPS,
            "gemm_shape": [n, n, n], "copy_gbs": copy, "copy_frac_hbm_peak": copy / PEAK_HBM_GBS,
            "copy_bytes": nbytes, "dense_attention": attn}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="time budget of the CPU-oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--probe-peaks", action="store_true",
                    help="also time a plain bf16 GEMM and a device copy (practical ceilings)")
    ap.add_argument("--fp8", action="store_true",
                    help="also time the MXFP8 variant of the sparse calls (reported apart)")
    ap.add_argument("--reuse", action="store_true",
                    help="also time mask reuse across steps: the drift gate and the candidate-"
                         "restricted search, against fresh mask prediction (reported apart)")
    ap.add_argument("--reuse-tau", type=float, default=0.05,
                    help="drift threshold of the mask-reuse gate (relative Frobenius change)")
    ap.add_argument("--tail", action="store_true",
                    help="also time the tail-reconstruction calls (reported apart from the step; "
                         "they launch the step's attention kernels with extra outputs, so they "
                         "are left out of the default run and its per-kernel profile)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path is per-head independent and would shard heads across GPUs without "
              "communication, which this benchmark does not run.", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_attention_top_amd as bsa
    import synth

    bsa.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = synth.WORKLOADS[args.workload]
    B, H, N, D, blk, M = cfg.batch, cfg.heads, cfg.seq, cfg.head_dim, cfg.block, cfg.num_blocks
    s = D ** -0.5
    log(f"generating {cfg.name}: B={B} H={H} N={N} D={D} block={blk} M={M}")
    t_gen = time.time()
    q, k, v = synth.make_qkv(cfg)
    p, c = synth.head_params(cfg)
    inputs = [(q, k, v)]
    if cfg.refresh_then_sparse:
        dq = synth.drift_series(q, "q", cfg.refresh_then_sparse)
        dk = synth.drift_series(k, "k", cfg.refresh_then_sparse)
        dv = synth.drift_series(v, "v", cfg.refresh_then_sparse)
        inputs += list(zip(dq, dk, dv))
    r_host = synth.make_residual(cfg) if (cfg.residual and not cfg.refresh_then_sparse) else None
    log(f"inputs generated in {time.time() - t_gen:.1f}s; copying to HBM")
    dev_inputs = [tuple(x.to(dev) for x in trip) for trip in inputs]
    r_dev = r_host.to(dev) if r_host is not None else None
    desc = bsa.make_desc(dev_inputs[0][0], blk)

    # outputs and workspaces, allocated once outside the timed region
    ncalls = len(dev_inputs)
    probs = torch.empty((B, H, M, M), dtype=torch.float32, device=dev)
    counts = [torch.empty((B, H, M), dtype=torch.int32, device=dev) for _ in range(ncalls)]
    idxs = [torch.empty((B, H, M, M), dtype=torch.int32, device=dev) for _ in range(ncalls)]
    out = torch.empty_like(dev_inputs[0][0])
    rcap = torch.empty_like(dev_inputs[0][0]) if cfg.refresh_then_sparse else None
    ws_sc = torch.empty(bsa.recap_workspace_size(0, desc), dtype=torch.uint8, device=dev)
    ws_sp = torch.empty(bsa.recap_workspace_size(2, desc), dtype=torch.uint8, device=dev)
    ws_dc = torch.empty(bsa.recap_workspace_size(4, desc), dtype=torch.uint8, device=dev) \
        if cfg.refresh_then_sparse else None
    plist, clist = p.tolist(), c.tolist()
    res_scale = clist if cfg.res_scale is not None else None

    def step(events):
        def timed(name, fn):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            if events is not None:
                events.append((name, e0, e1))

        for ci, (qq, kk, vv) in enumerate(dev_inputs):
            refresh = cfg.refresh_then_sparse and ci == 0
            tag = "refresh" if refresh else "sparse"
            timed(f"{tag}.scores", lambda: bsa.recap_block_scores(desc, qq, kk, s, probs, ws_sc))
            timed(f"{tag}.topp", lambda: bsa.recap_topp_mask(desc, probs, plist, counts[ci],
                                                             idxs[ci]))
            if refresh:
                timed("refresh.attn", lambda: bsa.recap_dense_attn(
                    desc, qq, kk, vv, s, counts[ci], idxs[ci], out, rcap, workspace=ws_dc))
            else:
                res = rcap if cfg.refresh_then_sparse else r_dev
                timed("sparse.attn", lambda: bsa.recap_block_sparse_attn(
                    desc, qq, kk, vv, counts[ci], idxs[ci], s, res,
                    res_scale if res is not None else None, out, ws_sp))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    events = []
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(events)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    per = {}
    calls = {"refresh": [], "sparse": []}  # whole-call times (scores + top-p + attention)
    for i, (name, e0, e1) in enumerate(events):
        ms = e0.elapsed_time(e1)
        per.setdefault(name, []).append(ms)
        tag, op = name.split(".")
        if op == "scores":
            calls[tag].append(0.0)
        calls[tag][-1] += ms
    avg = {k: float(np.mean(v)) for k, v in per.items()}

    def dist(v):
        v = np.asarray(v, dtype=np.float64)
        return {"median": float(np.median(v)), "min": float(v.min()),
                "p90": float(np.percentile(v, 90)), "n": int(v.size)}

    # computed-block work of one step
    dense_flops = 4.0 * D * B * H * float(N) * float(N)
    sparse_flops = []
    sparsity = []
    for ci in range(ncalls):
        if cfg.refresh_then_sparse and ci == 0:
            continue
        sparse_flops.append(4.0 * D * kept_token_pairs(counts[ci], idxs[ci], N, blk))
        sparsity.append(1.0 - counts[ci].double().mean().item() / M)
    step_flops = sum(sparse_flops) + (dense_flops if cfg.refresh_then_sparse else 0.0)
    step_tflops = step_flops / (ms_step * 1e-3) / 1e12
    sp_attn_ms = avg["sparse.attn"]
    sp_call_ms = avg["sparse.scores"] + avg["sparse.topp"] + sp_attn_ms
    sp_tflops = float(np.mean(sparse_flops)) / (sp_attn_ms * 1e-3) / 1e12
    value = sp_tflops  # the metric: computed-block TFLOP/s of the block-sparse attention call

    # mask-prediction algorithmic bytes per call (pool, scores, top-p)
    mean_kept = float(np.mean([counts[ci].double().mean().item() for ci in range(ncalls)]))
    mask_bytes = (2 * B * H * N * D * 2 + 2 * B * H * M * D * 4  # pool: read Q, K; write means
                  + 2 * B * H * M * D * 4 + B * H * M * M * 4  # scores: read means; write P
                  + B * H * M * M * 4 + B * H * M * (mean_kept + 1) * 4)  # top-p
    mask_ms = avg["sparse.scores"] + avg["sparse.topp"]

    def roof(kernel, achieved, bound="mfma", traffic_key=None, peak=None):
        if peak is None:
            peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
        return {"bound": bound, "achieved": achieved, "peak": peak,
                "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": achieved / peak,
                "traffic": measured_traffic(traffic_key, cfg.name) if traffic_key else None,
                "kernel": kernel}

    # achieved: algorithmic FLOPs over the HIP-event time of the library call (the sparse call
    # is one launch; the refresh also runs the residual fallback pass, 0.13 ms when no block is
    # flagged); traffic: the attention kernel's own counters
    sparse_roof = roof("attn_kernel<D=128, 4 wavefronts, sparse> (block-sparse attention with "
                       "the fused epilogue; timed as one recap_block_sparse_attn call)",
                       sp_tflops, traffic_key="attn_sparse")
    if cfg.refresh_then_sparse:
        dense_ms = avg["refresh.attn"]
        dense_tflops = dense_flops / (dense_ms * 1e-3) / 1e12
        refresh_roof = roof("attn_kernel<D=128, 4 wavefronts, dense + residual capture> "
                            "(timed as one recap_dense_attn call)", dense_tflops,
                            traffic_key="attn_capture")
    else:
        dense_ms = None
        refresh_roof = None
    mask_roof = roof("pool + score + topp kernels (one call's mask prediction)",
                     mask_bytes / (mask_ms * 1e-3) / 1e9, bound="hbm", traffic_key="mask")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: one attention layer, B={B} H={H} D={D} N={N} "
                         f"({'x'.join(map(str, cfg.grid))} tokens) block={blk} "
                         + (f"top-p {cfg.top_p}" if not isinstance(cfg.top_p, tuple)
                            else f"top-p U{cfg.top_p[1:]}")
                         + ("; step = dense refresh with residual capture + "
                            f"{cfg.refresh_then_sparse} drifted sparse calls with epilogue "
                            "(scale 1)" if cfg.refresh_then_sparse else "; step = one sparse call"
                            + (" with epilogue" if r_dev is not None else ""))),
            "batch": B, "heads": H, "head_dim": D, "seq_len": N, "block": blk,
            "parallelism": "single GPU",
        },
        "ms_per_sparse_call": sp_call_ms,
        "ms_sparse_attn": sp_attn_ms,
        "step_tflops": step_tflops,
        "ms_mask_prediction": mask_ms,
        "ms_refresh_call": (avg["refresh.scores"] + avg["refresh.topp"] + dense_ms)
        if dense_ms is not None else None,
        "sparse_attn_tflops": sp_tflops,
        "sparse_attn_frac_bf16_peak": sp_tflops / PEAK_BF16_TFLOPS,
        "block_sparsity": float(np.mean(sparsity)),
        "sparse_call_tflops": float(np.mean(sparse_flops)) / (sp_call_ms * 1e-3) / 1e12,
        "per_op_ms": avg,
        "per_op_ms_dist": {k: dist(v) for k, v in per.items()},
        "per_call_ms_dist": {k: dist(v) for k, v in calls.items() if v},
        "roofline": sparse_roof,
        "roofline_refresh": refresh_roof,
        "roofline_mask": mask_roof,
    }
    if args.probe_peaks:
        log("probe: bf16 GEMM, device copy, dense attention against torch SDPA")
        result["probe"] = probe_peaks(dev, bsa)
    if args.fp8:
        res = rcap if cfg.refresh_then_sparse else r_dev
        result["fp8"] = bench_fp8(bsa, cfg, desc, dev_inputs, counts, idxs, s, res, res_scale,
                                  avg, sparse_flops, args, roof)
    if args.reuse:
        log("mask reuse: gate and candidate search against fresh mask prediction")
        if cfg.refresh_then_sparse:
            x1 = dev_inputs[1]
        else:
            x1 = tuple(synth.drifted(t, n, 1).to(dev) for t, n in ((q, "q"), (k, "k")))
        result["reuse"] = bench_reuse(bsa, cfg, desc, dev_inputs[0][:2], x1[:2], p, s, args,
                                      args.reuse_tau)
    if cfg.refresh_then_sparse and args.tail:
        result["tail"] = bench_tail(bsa, cfg, desc, dev_inputs, counts, idxs, s, avg, args, roof)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        qs, ks, vs = inputs[1] if cfg.refresh_then_sparse else inputs[0]
        cb = cpu_baseline(cfg, qs, ks, vs, p, args.cpu_seconds, float(np.mean(sparse_flops)))
        result["cpu_baseline"] = {kk: vv for kk, vv in cb.items() if kk != "seconds"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
