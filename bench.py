#!/usr/bin/env python3
"""Benchmark of the dynamic top-k sparse attention forward on one MI355X.

One step = one call of sparse_attn_fwd (projection -> 16-bit MFMA scorer and
filter -> exact re-rank -> gather attention) over the whole 128K headline
workload: B=1, H=32, N=131072, D=128, d_proj=64, k=512, bf16, non-causal,
seeded synthetic inputs resident in HBM before timing starts.  --workload
picks one of the other workloads instead; for the band workload a step is
sparse_attn_band_indices followed by sparse_attn_gather.

Prints one JSON line.  value = queries/s (a query is one (b, h, i) row);
eff_tflops counts algorithmic flops only:
  F_proj = 4·B·H·N·D·d_proj, F_score = 2·d_proj·(pairs), F_gather = 4·D·Σk_i.
Per-kernel times come from HIP events the library records around each of its
launches on the launch stream (sparse_attn_profile_enable).

roofline: the kernel with the largest time per step, its algorithmic amount
per launch over its average launch time:
  filter   2·d_proj·pairs flops (16-bit MFMA, dense peak 2516.6 TFLOP/s)
  gather   K and V rows of the kept keys + the idx row + the q row, bytes
           (HBM peak 8 TB/s; the partial kernel of the key-range split)
  rerank   candidate entries (8 B) + idx row + exact-rescored k_low rows
traffic (HBM bytes per launch of that kernel) is taken from the rocprofv3
FETCH_SIZE / WRITE_SIZE readings recorded in TRAFFIC below, scaled by what the
same counters read for a plain 1 GiB copy, and only while the kernel's source
file is unchanged since (else null).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "queries/s + eff. TFLOP/s, top-k sparse attn fwd, N=128K H=32 D=128 k=512"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector


# rocprofv3 --pmc readings of the headline command (see profiles/), per launch
# of the kernel, already scaled by the plain-copy factors (FETCH_SIZE reads half
# a known copy's bytes, WRITE_SIZE all of them).  "src" is the sha256 of the
# kernel's sources (KERNEL_SOURCE) when the counters were taken.  They hold
# for that command only: the headline workload, fp16 filter operands, all 32
# heads in one selection launch (COUNTER_RUN); other runs report null.
COUNTER_RUN = {"workload": "headline_128k", "filter_dtype": "f16", "heads_per_launch": 32}
TRAFFIC = {
    # profiles/headline_128k_hbm_traffic.md (bytes) and headline_128k_l2_hits.md (the
    # gather's L2 hit rate); the filter's is its main launch (32 heads), the re-rank's its
    # main launch (32 heads), the gather's its partial kernel (one head)
    "filter": {"fetch_bytes": 120.884e9, "write_bytes": 93.501e9,
               "src": "3021e687f2adad69fa230cd6b911cb844de524181d9058865db90509957ce0af"},
    "gather": {"fetch_bytes": 11.027e9, "write_bytes": 0.570e9,
               "l2_hit_rate": 0.694,
               "src": "570b28bdbabc1d4a470a2af02397d298cdb957dd0aa715ca70142bc0e863e3af"},
    "rerank": {"fetch_bytes": 68.142e9, "write_bytes": 8.751e9,
               "src": "cb7b7494a83992f3f2b47126003a62b17bc6ddd65d51404de0ae35149cce1dbf"},
}
# the sources each kernel's code comes from (their sha256, concatenated in
# this order, is recorded with the counters)
KERNEL_SOURCE = {"filter": ["scorer.hip"], "gather": ["gather.hip", "rows.h"],
                 "rerank": ["finalize.hip"]}

# rocprofv3 --pmc readings of the filter's MFMA activity on the headline
# command (profiles/filter_128k_mfma_counters.md), with the sha256 of
# scorer.hip when taken.  mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES over
# (1024 SIMDs x GRBM_GUI_ACTIVE per XCD); shader_clock_ghz = the cycles per
# XCD over the dispatch's duration.
MFMA_COUNTERS: dict = {
    "filter": {"SQ_INSTS_MFMA": 2147483648, "SQ_VALU_MFMA_BUSY_CYCLES": 68719476736,
               "GRBM_GUI_ACTIVE_all_xcds": 1313034725, "dispatch_ms": 92.09,
               "mfma_busy_frac": 0.4089, "shader_clock_ghz": 1.782,
               "src": "3021e687f2adad69fa230cd6b911cb844de524181d9058865db90509957ce0af"},
}


def source_sha(kernel: str):
    import hashlib
    names = KERNEL_SOURCE.get(kernel)
    if names is None:
        return None
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "dynamic_top_sparse_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic(w) -> dict:
    """Algorithmic work of one forward over workload w."""
    B, H, N, D, dp, k = w.B, w.H, w.N, w.D, w.d_proj, w.k
    BH = B * H
    if w.mode == "band":
        pairs = 0
        sum_k = sum(min(N - 1, i + w.window) - max(0, i - w.window) + 1 for i in range(N))
    elif w.causal:
        pairs = N * (N + 1) // 2
        sum_k = sum(min(k, i + 1) for i in range(N))
    else:
        pairs = N * N
        sum_k = N * min(k, N)
    e = 2 if w.dtype == "bf16" else 4
    return {
        "F_proj": 4.0 * BH * N * D * dp,
        "F_score": 2.0 * dp * pairs * BH,
        "F_gather": 4.0 * D * sum_k * BH,
        # per head: K and V rows of every kept key, the idx row, q in, O out
        "gather_bytes_per_head": float(sum_k * 2 * D * e + N * k * 4 + N * 2 * D * e),
        # the same without O (written by the merge of the key-range split)
        "gather_part_bytes_per_head": float(sum_k * 2 * D * e + N * k * 4 + N * D * e),
        "pairs_per_head": float(pairs),
    }


def counters_apply(workload: str, filter_dtype: str, heads_per_launch) -> bool:
    """Whether this run is the command the committed counters were taken on."""
    return (workload == COUNTER_RUN["workload"] and filter_dtype == COUNTER_RUN["filter_dtype"]
            and heads_per_launch == COUNTER_RUN["heads_per_launch"])


def gather_counter_frac(kern: dict, band: bool, applies: bool):
    """Counter bytes per launch of the gather's main kernel over its measured
    average launch time, as a fraction of the HBM peak (headline command's
    counters only; null when they do not apply)."""
    tr = TRAFFIC.get("gather")
    d = kern.get("gather")
    if band or not applies or not tr or not d or tr.get("src") != source_sha("gather") or \
            "gather_merge" not in kern:
        return None
    avg_s = d["ms_total"] / d["launches"] / 1e3
    return (tr["fetch_bytes"] + tr["write_bytes"]) / avg_s / 1e9 / PEAK_HBM_GBS


def l2_hit_rate(kernel: str):
    """L2 hit rate of a kernel of the headline forward from the committed
    rocprofv3 TCC_HIT / TCC_MISS run (null once its source has changed)."""
    tr = TRAFFIC.get(kernel)
    if not tr or "l2_hit_rate" not in tr or tr.get("src") != source_sha(kernel):
        return None
    return tr["l2_hit_rate"]


def filter_mfma_counters():
    """MFMA activity of the filter from the committed rocprofv3 counter run
    (null once the filter source has changed since it was taken)."""
    c = MFMA_COUNTERS.get("filter")
    if not c or c.get("src") != source_sha("filter"):
        return None
    return {k: v for k, v in c.items() if k != "src"}


def pick_heads_per_chunk(w) -> int:
    """Largest of (all heads, 16, 8) whose workspace takes at most a quarter of
    the device's memory.  Larger chunks mean fewer, fuller launches: each
    filter launch is a whole number of workgroup rounds only for some sizes
    (at the headline size 32 heads run 22 rounds of the chip's resident
    workgroups where four chunks of 8 run 24)."""
    import torch
    import dynamic_top_sparse_amd as sa
    budget = torch.cuda.get_device_properties(0).total_memory // 4
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    for hc in (w.B * w.H, 16, 8):
        n = sa.sparse_attn_workspace_size(w.B, w.H, w.N, w.D, w.d_proj, w.k, w.causal, dt,
                                          True, hc)
        if 0 < n <= budget:
            return hc
    return 8


def cpu_baseline(x, w, target_s: float = 20.0) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same
    workload: query rows of head (0, 0), including that head's projections
    (for the band workload: the band rows and their attention).  BLAS runs on
    every core this process may use; the rate is extrapolated linearly from
    the sample to the whole workload."""
    import numpy as np
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:
        limiter = None
    Q1, K1, V1 = (x[n][:1, :1] for n in ("Q", "K", "V"))
    sscale, ascale = (w.d_proj ** -0.5 if w.d_proj else 0.0), w.D ** -0.5
    rng = np.random.default_rng(0)

    def run(rows):
        t = time.perf_counter()
        if w.mode == "band":
            idx = O.band_indices(w.N, w.window, w.window, w.k)[rows][None, None]
            O.gather_attention(Q1, K1, V1, idx, ascale, rows)
        else:
            O.sparse_attn_fwd(Q1, K1, V1, x["Pq"], x["Pk"], w.k, w.causal, sscale, ascale, rows)
        return time.perf_counter() - t

    try:
        pilot = sorted(rng.choice(w.N, 16, replace=False).tolist())
        tp = run(pilot)
        n_rows = int(min(4096, w.N, max(32, 16 * target_s / max(tp, 1e-3))))
        rows = sorted(rng.choice(w.N, n_rows, replace=False).tolist())
        t = run(rows)
    finally:
        if limiter is not None:
            limiter.unregister()
    mode = "full" if n_rows == w.N and w.B * w.H == 1 else "extrapolated"
    return {"value": n_rows / t, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "mode": mode, "oracle_seconds": t,
            "extrapolated_workload_seconds": t * w.queries / n_rows,
            "sample": (f"{n_rows} random query rows of head (0,0) of the {w.name} workload "
                       + ("through the fp64 oracle's band indices and softmax gather"
                          if w.mode == "band" else
                          "through the fp64 oracle forward (scores, top-k, softmax gather), "
                          "including that head's key projection")
                       + f"; {t:.1f} s with BLAS on {cores} cores")}


def time_steps(step, prof, steps: int, warmup: int):
    """W untimed steps, then K steps each bracketed by HIP events on the
    current stream with a 512 MiB cache-flushing write between them (outside
    the events).  Returns (sorted per-step ms, wall ms per step, kernel
    records of the timed steps)."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        flush.fill_(1)
        e0.record(stream)
        step(prof)
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    del flush
    return sorted(e0.elapsed_time(e1) for e0, e1 in ev), (t1 - t0) * 1e3 / steps, prof.read()


def kernel_table(recs, steps):
    kern = {}
    for name, ms in recs:
        d = kern.setdefault(name, {"launches": 0, "ms_total": 0.0})
        d["launches"] += 1
        d["ms_total"] += ms
    return kern, {n: d["ms_total"] / steps for n, d in kern.items()}


def oracle_rate(fn, n_total: int, target_s: float = 20.0):
    """Times fn(rows) of the oracle on a sample sized to about target_s from a
    64-row pilot (after an 8-row warm-up); BLAS on every core this process
    may use."""
    import numpy as np
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:
        limiter = None
    rng = np.random.default_rng(0)
    try:
        fn(sorted(rng.choice(n_total, min(8, n_total), replace=False).tolist()))   # warm-up
        m = min(64, n_total)
        t = time.perf_counter()
        fn(sorted(rng.choice(n_total, m, replace=False).tolist()))
        tp = time.perf_counter() - t
        n = int(min(n_total, max(16, m * target_s / max(tp, 1e-4))))
        rows = sorted(rng.choice(n_total, n, replace=False).tolist())
        t = time.perf_counter()
        fn(rows)
        t = time.perf_counter() - t
    finally:
        if limiter is not None:
            limiter.unregister()
    return n, t, cores


def run_op(args, w) -> int:
    """The rows of the method beyond the forward, measured like the forward:
    per-step HIP events, cache flush between steps, roofline of the kernel
    with the largest time, and the fp64 oracle on a bounded sample."""
    import numpy as np
    import torch
    import dynamic_top_sparse_amd as sa
    import oracle as O
    from dynamic_top_sparse_amd import workloads as W

    prof = sa.Profile()
    x = W.make_inputs(w, W.default_seed())
    g = {k: v.cuda() for k, v in x.items()}
    B, H, N, D, dp, k = w.B, w.H, w.N, w.D, w.d_proj, w.k
    e = 2 if w.dtype == "bf16" else 4
    BH = B * H
    op = args.op
    extra = {}
    if op == "bwd":
        gen = torch.Generator().manual_seed(1)
        dO = torch.randn(B, H, N, D, generator=gen).to(w.torch_dtype).cuda()
        _, idx = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], k, w.causal,
                                    return_idx=True)
        n_ws = sa.load_library().sparse_attn_bwd_workspace_size(
            sa.sa_dims(B, H, N, D), dp, k, 1, sa._options(bwd_parts=args.bwd_parts))
        bws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
        sum_k = float((idx >= 0).sum().item())

        def step(p):
            sa.sparse_attn_bwd(g["Q"], g["K"], g["V"], dO, idx, g["Pq"], g["Pk"], workspace=bws,
                               profile=p, parts=args.bwd_parts)
        units = BH * N
        metric = f"queries/s, top-k sparse attn backward (dQ, dK, dV, dPq, dPk), {w.name}"
        extra = {"bwd_parts": args.bwd_parts}
        # algorithmic bytes of the two wave passes (per launch: all heads)
        amount = {
            "bwd_rows": sum_k * (2 * D * e) + BH * N * (2 * D * e + 4 * k + 8 * k + 4 * D),
            "bwd_keys": sum_k * (12 + 2 * D * e) + BH * N * (8 * D + 8),
            # the largest heads take the key pass in two launches, dV then H
            "bwd_keys_dv": sum_k * (12 + D * e) + BH * N * (4 * D + 4),
            "bwd_keys_h": sum_k * (12 + D * e) + BH * N * (4 * D + 4),
            "bwd_fill": float(BH * N * k * (4 + 8) + sum_k * 12),
        }
        desc = {"bwd_rows": "K, V rows of kept keys + q, dO, idx rows + (p, dl) + dQ",
                "bwd_keys": "records + Q, dO rows of the rows that kept each key + dK, dV",
                "bwd_keys_dv": "records + dO rows of the rows that kept each key + dV",
                "bwd_keys_h": "records + Q rows of the rows that kept each key + dK",
                "bwd_fill": "idx + (p, dl) read, 12-byte records written"}
        idx_np = idx.cpu().numpy()
        # the head's rows as the oracle takes them, converted once outside the timing
        Qh, Kh, Vh = (O.f64(t[0, 0]) for t in (x["Q"], x["K"], x["V"]))
        dOh = O.f64(dO[0, 0].cpu())

        def oracle_fn(rows):
            for i in rows:
                O.attend_row_backward(Qh[i], Kh, Vh, idx_np[0, 0, i].astype(np.int64), D ** -0.5,
                                      dOh[i])
        sample_desc = "rows of head (0,0) through the oracle's per-row backward"
    elif op == "decode":
        cache = sa.DecodeCache(B, H, N, D, g["Pq"], g["Pk"], k, dtype=w.torch_dtype)
        cache.append(g["K"], g["V"])
        q = g["Q"][:, :, N - 1:N].contiguous()
        o = torch.empty_like(q)

        def step(p):
            cache.step(q, O=o, profile=p)
        units = BH
        metric = f"decode queries/s (one query per head over a full KV cache), {w.name}"
        nsl = (N + 2047) // 2048      # slices of the score and collect steps
        amount = {"decode_scores": float(BH * N * (4 * dp + 4)),
                  "decode_collect": float(BH * N * 4 + BH * nsl * 2048 * 4),
                  "decode_gather": float(BH * k * 2 * D * e + BH * (k * 4 + 2 * D * e))}
        desc = {"decode_scores": "k_low cache rows (fp32) + scores",
                "decode_collect": "each head's scores + its bin counts, read once per slice",
                "decode_gather": "K, V cache rows of the kept keys + idx + q (partials apart)"}

        def oracle_fn(rows):
            for _ in rows:
                O.decode_step(x["Q"][0, 0, N - 1], x["K"][0, 0], x["V"][0, 0], x["Pq"], x["Pk"],
                              k, N, dp ** -0.5, D ** -0.5)
        sample_desc = "decode steps of head (0,0) through the oracle (one per sampled row)"
    elif op == "block":
        block, kb = 64, max(1, k // 64)
        idx = torch.empty(B, H, N, kb * block, dtype=torch.int32, device="cuda")
        n_ws = sa.load_library().sparse_attn_block_workspace_size(sa.sa_dims(B, H, N, D), dp,
                                                                  block, kb)
        bws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
        out = torch.empty_like(g["Q"])

        def step(p):
            sa.sparse_attn_block_topk(g["Q"], g["K"], g["Pq"], g["Pk"], block, kb, w.causal,
                                      idx=idx, workspace=bws, profile=p)
            sa.sparse_attn_gather(g["Q"], g["K"], g["V"], idx, O=out, profile=p)
        units = BH * N
        NB = (N + block - 1) // block
        metric = f"queries/s, block-granular top-{kb} of {block}-key blocks + gather, {w.name}"
        extra = {"block": block, "kb": kb}
        amount = {"block_select": float(BH * N * NB * 2 * dp),
                  "gather": float(BH * N * (kb * block * 2 * D * e + kb * block * 4 + 2 * D * e))}
        desc = {"block_select": "2*d_proj flop per (query, block) score, fp32 FMA",
                "gather": "K, V rows of the kept keys + idx + q, O"}

        def oracle_fn(rows):
            idx_r = O.block_topk_indices(x["Q"][:1, :1], x["K"][:1, :1], x["Pq"], x["Pk"], block,
                                         kb, w.causal, dp ** -0.5, rows)
            O.gather_attention(x["Q"][:1, :1], x["K"][:1, :1], x["V"][:1, :1], idx_r, D ** -0.5,
                               rows)
        sample_desc = "rows of head (0,0) through the oracle's block selection and gather"
    elif op == "smooth":
        gap = 0.02
        idx = torch.empty(B, H, N, k + 1, dtype=torch.int32, device="cuda")
        sws = sa.allocate_workspace(g["Q"], dp, k + 1, w.causal)
        out = torch.empty_like(g["Q"])

        def step(p):
            sa.sparse_attn_scores_topk_smoothed(g["Q"], g["K"], g["Pq"], g["Pk"], k, gap,
                                                w.causal, idx=idx, workspace=sws, profile=p)
            sa.sparse_attn_gather(g["Q"], g["K"], g["V"], idx, O=out, profile=p)
        units = BH * N
        metric = f"queries/s, top-{k} with boundary smoothing (gap {gap}) + gather, {w.name}"
        extra = {"gap": gap}
        amount = {"filter": float(2 * dp * (N * N if not w.causal else N * (N + 1) // 2) * BH),
                  "gather": float(BH * N * ((k + 1) * 2 * D * e + (k + 1) * 4 + 2 * D * e))}
        desc = {"filter": "2*d_proj flop per (query, key) pair", "gather": "K, V rows + idx + q, O"}

        def oracle_fn(rows):
            S = O.scores(x["Q"][:1, :1], x["K"][:1, :1], x["Pq"], x["Pk"], dp ** -0.5, 0, 0, rows)
            idx_r = O.smoothed_topk_rows(S, rows, k, w.causal, gap)[None, None]
            O.gather_attention(x["Q"][:1, :1], x["K"][:1, :1], x["V"][:1, :1], idx_r, D ** -0.5,
                               rows)
        sample_desc = "rows of head (0,0) through the oracle's smoothed top-k and gather"
    else:   # dilated
        window, dilation = 129, 4
        idx = torch.empty(B, H, N, window, dtype=torch.int32, device="cuda")
        out = torch.empty_like(g["Q"])

        def step(p):
            sa.sparse_attn_dilated_indices(B, H, N, window, dilation, window, idx=idx, profile=p)
            sa.sparse_attn_gather(g["Q"], g["K"], g["V"], idx, O=out, profile=p)
        units = BH * N
        metric = f"queries/s, dilated window ({window} keys, dilation {dilation}) + gather, {w.name}"
        extra = {"window": window, "dilation": dilation}
        amount = {"gather": float(BH * N * (window * 2 * D * e + window * 4 + 2 * D * e))}
        desc = {"gather": "K, V rows of the window + idx + q, O"}
        didx = O.dilated_indices(N, window, dilation, window)

        def oracle_fn(rows):
            O.gather_attention(x["Q"][:1, :1], x["K"][:1, :1], x["V"][:1, :1],
                               didx[rows][None, None], D ** -0.5, rows)
        sample_desc = "rows of head (0,0) through the oracle's attention over the dilated window"

    step_ms, wall_ms, recs = time_steps(step, prof, args.steps, args.warmup)
    prof.close()
    kern, per_step = kernel_table(recs, args.steps)
    ms = float(np.median(step_ms))
    dom = max((n for n in per_step if n in amount), key=per_step.get)
    avg_s = kern[dom]["ms_total"] / kern[dom]["launches"] / 1e3
    per_launch = amount[dom] / (kern[dom]["launches"] / args.steps)
    if dom == "filter":
        roof = {"kernel": dom, "bound": "mfma", "achieved": per_launch / avg_s / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    elif dom == "block_select":
        roof = {"kernel": dom, "bound": "alu", "achieved": per_launch / avg_s / 1e12,
                "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": per_launch / avg_s / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["algorithmic_per_launch"] = f"{per_launch:.4g} ({desc[dom]})"
    roof["avg_launch_ms"] = avg_s * 1e3
    result = {
        "metric": metric, "value": units / (ms / 1e3), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_min": step_ms[0], "ms_per_step_mean": float(np.mean(step_ms)),
        "wall_ms_per_step_incl_flush": wall_ms,
        "timing": ("median of per-step HIP events on the launch stream; a 512 MiB write "
                   "between steps (outside the events) flushes L2 and the memory-side cache"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "op": op, "B": B, "H": H, "N": N, "D": D, "d_proj": dp,
                   "k": k, "causal": w.causal, "dist": w.dist, "seed": W.default_seed(), **extra},
        "kernel_ms_per_step": {n: round(v, 3) for n, v in sorted(per_step.items(),
                                                                  key=lambda kv: -kv[1])},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        n, t, cores = oracle_rate(oracle_fn, N)
        result["cpu_baseline"] = {
            "value": n / t, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "mode": "extrapolated", "oracle_seconds": t,
            "sample": f"{n} {sample_desc} of the {w.name} workload; {t:.1f} s"}
    print(json.dumps(result))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="headline_128k")
    ap.add_argument("--heads-per-chunk", type=int, default=0,
                    help="workspace sized for this many heads per chunk (0 = the largest of all "
                         "heads, 16, 8 whose workspace fits in a quarter of device memory)")
    ap.add_argument("--filter-dtype", choices=("f16", "bf16"), default="f16",
                    help="16-bit operand type of the MFMA filter (indices do not depend on it)")
    ap.add_argument("--op", default="fwd",
                    choices=("fwd", "bwd", "decode", "block", "smooth", "dilated"),
                    help="fwd: the forward (default); bwd: the backward over the forward's index "
                         "sets; decode: one decode step over a full KV cache; block: block-granular "
                         "selection + gather; smooth: top-k with boundary smoothing + gather; "
                         "dilated: dilated wrap-around window + gather")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bwd-parts", choices=("auto", "whole", "split"), default="auto",
                    help="--op bwd: the row and key passes whole, in key-range parts, or as the "
                         "library picks (parts from 2^22 row elements per head)")
    ap.add_argument("--other-filter-steps", type=int, default=5,
                    help="forward steps timed with the filter's other 16-bit operand type after "
                         "the main ones (0: none, e.g. for a kernel trace of the main forward)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB: the known-size "
                         "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    import dynamic_top_sparse_amd as sa
    from dynamic_top_sparse_amd import workloads as W

    fdt = torch.float16 if args.filter_dtype == "f16" else torch.bfloat16
    prof = sa.Profile()
    try:
        w = W.get(args.workload)
    except KeyError:
        print(f"unknown workload {args.workload!r}; one of {sorted(W.WORKLOADS)}", file=sys.stderr)
        return 2
    if args.op != "fwd":
        return run_op(args, w)
    band = w.mode == "band"
    x = W.make_inputs(w, W.default_seed())
    g = {k: v.cuda() for k, v in x.items()}
    out = torch.empty_like(g["Q"])
    if band:
        ws = None
        idx = torch.empty((w.B, w.H, w.N, w.k), dtype=torch.int32, device="cuda")

        def step(p=None):
            sa.sparse_attn_band_indices(w.B, w.H, w.N, w.window, w.window, w.k, idx=idx,
                                        profile=p)
            sa.sparse_attn_gather(g["Q"], g["K"], g["V"], idx, O=out, profile=p)
    else:
        hc = args.heads_per_chunk or pick_heads_per_chunk(w)
        ws = sa.allocate_workspace(g["Q"], w.d_proj, w.k, w.causal, with_idx=True,
                                   heads_per_chunk=hc)

        def step(p=None, fd=fdt):
            sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, w.causal,
                               O=out, workspace=ws, filter_dtype=fd, profile=p)
    # 512 MiB written between timed steps (outside their event brackets), so
    # no step starts with the previous one's data in L2 or the memory-side
    # cache
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        flush.fill_(1)
        e0.record(stream)
        step(prof)          # every library launch bracketed by its own events, same stream
        e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    recs = prof.read()
    prof.close()
    stats = sa.sparse_attn_workspace_stats(ws) if ws is not None else None
    # the same forward with the filter's other 16-bit operand type (the
    # indices do not depend on it), timed the same way over a few steps
    alt_filter = None
    if not band and args.steps > 0 and args.other_filter_steps > 0:
        adt_name = "bf16" if args.filter_dtype == "f16" else "f16"
        adt = torch.bfloat16 if adt_name == "bf16" else torch.float16
        n_alt = args.other_filter_steps
        step(fd=adt)
        torch.cuda.synchronize()
        aprof = sa.Profile()
        aev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n_alt)]
        for e0, e1 in aev:
            flush.fill_(1)
            e0.record(stream)
            step(aprof, fd=adt)
            e1.record(stream)
        torch.cuda.synchronize()
        a_ms = sorted(e0.elapsed_time(e1) for e0, e1 in aev)
        a_filter = [ms for name, ms in aprof.read() if name == "filter"]
        aprof.close()
        alt_filter = {"filter_dtype": adt_name, "steps": n_alt,
                      "ms_per_step": float(np.median(a_ms)),
                      "filter_ms_per_launch": float(np.mean(a_filter)) if a_filter else None}
    del flush
    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_step = float(np.median(step_ms))
    a = algorithmic(w)
    queries = w.queries
    flops = a["F_proj"] + a["F_score"] + a["F_gather"]
    # per-kernel totals per step and per-launch averages
    kern = {}
    for name, ms in recs:
        d = kern.setdefault(name, {"launches": 0, "ms_total": 0.0})
        d["launches"] += 1
        d["ms_total"] += ms
    per_step = {n: d["ms_total"] / args.steps for n, d in kern.items()}
    scorer_names = ("init", "project", "pack", "sample", "threshold", "filter", "rerank",
                    "filter_retry", "rerank_retry", "fallback")
    gather_names = ("gather", "gather_merge")
    t_scorer = sum(per_step.get(n, 0.0) for n in scorer_names) / 1e3
    t_gather = sum(per_step.get(n, 0.0) for n in gather_names) / 1e3

    n_filter = kern.get("filter", {}).get("launches", 0)
    heads_per_chunk = (w.B * w.H * args.steps) / n_filter if n_filter else None
    # roofline of the kernel with the largest time per step
    dom = max(per_step, key=per_step.get) if not band else "gather"
    avg_launch_s = kern[dom]["ms_total"] / kern[dom]["launches"] / 1e3
    heads = w.B * w.H * args.steps / kern[dom]["launches"]
    if dom == "filter":
        amount = 2.0 * w.d_proj * a["pairs_per_head"] * heads
        roof = {"kernel": dom, "bound": "mfma", "achieved": amount / avg_launch_s / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
        roof["algorithmic_per_launch"] = f"{amount:.4g} flop (2*d_proj*pairs, {heads:g} heads)"
    elif dom == "rerank":
        nq = w.N * heads
        cand = stats["candidates"] / max(stats["queries"], 1)
        resc = stats["rescored"] / max(stats["queries"], 1)
        amount = nq * (8.0 * cand + 4.0 * w.k + 4.0 * w.d_proj * resc)
        roof = {"kernel": dom, "bound": "hbm", "achieved": amount / avg_launch_s / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        roof["algorithmic_per_launch"] = (f"{amount:.4g} B (candidates, idx rows, rescored "
                                          f"k_low rows; {heads:g} heads)")
    else:
        per_head = a["gather_part_bytes_per_head"] if "gather_merge" in per_step \
            else a["gather_bytes_per_head"]
        amount = per_head * heads
        roof = {"kernel": dom, "bound": "hbm", "achieved": amount / avg_launch_s / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
        roof["algorithmic_per_launch"] = (f"{amount:.4g} B (K,V rows of kept keys + idx + q, "
                                          f"{heads:g} heads)")
    roof["frac"] = roof["achieved"] / roof["peak"]
    applies = counters_apply(w.name, args.filter_dtype, heads_per_chunk)
    tr = TRAFFIC.get(dom)
    roof["traffic"] = (tr["fetch_bytes"] + tr["write_bytes"]) if applies and tr and \
        tr.get("src") == source_sha(dom) else None
    roof["avg_launch_ms"] = avg_launch_s * 1e3

    result = {
        "metric": METRIC if w.name == "headline_128k" else
        f"queries/s + eff. TFLOP/s, {'band' if band else 'top-k'} sparse attn fwd, {w.name}",
        "value": queries / (ms_step / 1e3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_min": step_ms[0],
        "ms_per_step_mean": float(np.mean(step_ms)),
        "wall_ms_per_step_incl_flush": (t1 - t0) * 1e3 / args.steps,
        "timing": ("median of per-step HIP events on the launch stream; a 512 MiB write "
                   "between steps (outside the events) flushes L2 and the memory-side cache"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "D": w.D,
                   "d_proj": w.d_proj, "k": w.k, "causal": w.causal, "dist": w.dist,
                   "seed": W.default_seed(), "heads_per_chunk": heads_per_chunk,
                   **({"window": w.window} if band else {})},
        "eff_tflops": flops / (ms_step / 1e3) / 1e12,
        "scorer_frac_of_bf16_peak": ((a["F_proj"] + a["F_score"]) / t_scorer / 1e12
                                     / PEAK_BF16_TFLOPS) if t_scorer else None,
        # logical bytes (every kept K/V row counted as if read from HBM), over
        # the gather stage's time: above 1 when L2 and the memory-side cache
        # serve repeated rows
        "gather_logical_bytes_per_s_over_hbm_peak": (
            (a["gather_bytes_per_head"] * w.B * w.H) / t_gather / 1e9 / PEAK_HBM_GBS)
        if t_gather else None,
        # counter-measured bytes between L2 and the fabric (FETCH_SIZE +
        # WRITE_SIZE, memory-side-cache hits included) per gather launch, over
        # that launch's time; null once the gather source has changed since
        # the counters were taken
        "gather_frac_of_hbm_peak": gather_counter_frac(kern, band, applies),
        # TCC_HIT / (TCC_HIT + TCC_MISS) of the gather's partial kernel
        "gather_l2_hit_rate": l2_hit_rate("gather") if applies and not band else None,
        "gather_stage_ms": t_gather * 1e3,
        "kernel_ms_per_step": {n: round(v, 3) for n, v in sorted(per_step.items(),
                                                                  key=lambda kv: -kv[1])},
        "roofline": roof,
    }
    if stats is not None:
        result["selection"] = {
            "candidates_per_query": stats["candidates"] / max(stats["queries"], 1),
            "rescored_per_query": stats["rescored"] / max(stats["queries"], 1),
            "fallback_queries": stats["fallback_queries"],
            "overflow_queries": stats["overflow_queries"],
            "retried_queries": stats["retried"],
            "margin_violations": stats["margin_violations"],
            "rerank_queries_from_memory": stats.get("wide_queries"),
            "filter_dtype": args.filter_dtype}
        result["filter_mfma_counters"] = filter_mfma_counters() if applies else None
    if alt_filter is not None:
        fl = alt_filter["filter_ms_per_launch"]
        if fl and n_filter:
            heads_f = w.B * w.H * args.steps / n_filter
            alt_filter["filter_frac_of_bf16_peak"] = (
                2.0 * w.d_proj * a["pairs_per_head"] * heads_f / (fl / 1e3) / 1e12
                / PEAK_BF16_TFLOPS)
        result["other_filter_operands"] = alt_filter
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
