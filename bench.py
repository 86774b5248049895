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

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "queries/s + eff. TFLOP/s, top-k sparse attn fwd, N=128K H=32 D=128 k=512"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


# rocprofv3 --pmc readings of the headline command (see profiles/), per launch
# of the kernel, already scaled by the plain-copy factors (FETCH_SIZE reads half
# a known copy's bytes, WRITE_SIZE all of them).  "src" is the sha256 of the
# kernel's source file when the counters were taken.
TRAFFIC = {
    # profiles/headline_128k_hbm_traffic.md; the filter's is its main launch (32 heads),
    # the re-rank's its main launch (32 heads), the gather's its partial kernel (one head)
    "filter": {"fetch_bytes": 120.957e9, "write_bytes": 93.378e9,
               "src": "c2fd4f618ca754cb8861533b8c8a12713eb99adaa6da0ee9097139d27472aa58"},
    "gather": {"fetch_bytes": 11.025e9, "write_bytes": 0.570e9,
               "src": "5877c0c9b38d66bf2db13d14434eb11b76d2099e41d909161337876ede489689"},
    "rerank": {"fetch_bytes": 69.471e9, "write_bytes": 10.888e9,
               "src": "f4407d799910cd43fb4a75b18a8fca50eec3133ed9f1aa1a0616b23d5c45d73e"},
}
KERNEL_SOURCE = {"filter": "scorer.hip", "gather": "gather.hip", "rerank": "finalize.hip"}


def source_sha(kernel: str):
    import hashlib
    name = KERNEL_SOURCE.get(kernel)
    if name is None:
        return None
    path = os.path.join(ROOT, "dynamic_top_sparse_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


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
    (for the band workload: the band rows and their attention)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
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

    pilot = sorted(rng.choice(w.N, 16, replace=False).tolist())
    tp = run(pilot)
    n_rows = int(min(4096, w.N, max(32, 16 * target_s / max(tp, 1e-3))))
    rows = sorted(rng.choice(w.N, n_rows, replace=False).tolist())
    t = run(rows)
    return {"value": n_rows / t, "unit": "queries/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"{n_rows} random query rows of head (0,0) of the {w.name} workload "
                       + ("through the fp64 oracle's band indices and softmax gather"
                          if w.mode == "band" else
                          "through the fp64 oracle forward (scores, top-k, softmax gather), "
                          "including that head's key projection") + f"; {t:.1f} s")}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="headline_128k")
    ap.add_argument("--heads-per-chunk", type=int, default=0,
                    help="workspace sized for this many heads per chunk (0 = the largest of all "
                         "heads, 16, 8 whose workspace fits in a quarter of device memory)")
    ap.add_argument("--filter-dtype", choices=("f16", "bf16"), default="f16",
                    help="16-bit operand type of the MFMA filter (indices do not depend on it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    sa.sparse_attn_set_filter_dtype(torch.float16 if args.filter_dtype == "f16" else torch.bfloat16)
    try:
        w = W.get(args.workload)
    except KeyError:
        print(f"unknown workload {args.workload!r}; one of {sorted(W.WORKLOADS)}", file=sys.stderr)
        return 2
    band = w.mode == "band"
    x = W.make_inputs(w, W.default_seed())
    g = {k: v.cuda() for k, v in x.items()}
    out = torch.empty_like(g["Q"])
    if band:
        ws = None
        idx = torch.empty((w.B, w.H, w.N, w.k), dtype=torch.int32, device="cuda")

        def step():
            sa.sparse_attn_band_indices(w.B, w.H, w.N, w.window, w.window, w.k, idx=idx)
            sa.sparse_attn_gather(g["Q"], g["K"], g["V"], idx, O=out)
    else:
        hc = args.heads_per_chunk or pick_heads_per_chunk(w)
        ws = sa.allocate_workspace(g["Q"], w.d_proj, w.k, w.causal, with_idx=True,
                                   heads_per_chunk=hc)

        def step():
            sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, w.causal,
                               O=out, workspace=ws)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sa.sparse_attn_profile_enable(True)
    sa.sparse_attn_profile_read()          # drop anything recorded before
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    recs = sa.sparse_attn_profile_read()
    sa.sparse_attn_profile_enable(False)
    stats = sa.sparse_attn_workspace_stats(ws) if ws is not None else None
    if args.copy_probe_mib > 0:
        src = torch.ones(args.copy_probe_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_step = (t1 - t0) * 1e3 / args.steps
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
    tr = TRAFFIC.get(dom)
    roof["traffic"] = (tr["fetch_bytes"] + tr["write_bytes"]) if tr and \
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
        "gather_frac_of_hbm_peak": ((a["gather_bytes_per_head"] * w.B * w.H) / t_gather / 1e9
                                    / PEAK_HBM_GBS) if t_gather else None,
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
            "filter_dtype": str(sa.sparse_attn_get_filter_dtype()).replace("torch.", "")}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
