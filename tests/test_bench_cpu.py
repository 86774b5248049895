"""Host-side checks of bench.py: the algorithmic work it divides by is counted
by brute force from the oracle's own definitions of the valid keys and of the
band rows, and the one-GPU contract is kept."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle as O
from dynamic_top_sparse_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("causal", [False, True])
def test_topk_work_counts(causal):
    w = W.get("tiny_fp32", N=300, H=3, B=2, k=40, causal=causal)
    a = bench.algorithmic(w)
    pairs = sum(int(O.valid_keys(w.N, i, causal).sum()) for i in range(w.N))
    sum_k = sum(min(w.k, int(O.valid_keys(w.N, i, causal).sum())) for i in range(w.N))
    BH = w.B * w.H
    assert a["pairs_per_head"] == pairs
    assert a["F_score"] == 2 * w.d_proj * pairs * BH
    assert a["F_proj"] == 4 * BH * w.N * w.D * w.d_proj
    assert a["F_gather"] == 4 * w.D * sum_k * BH
    e = 4   # fp32 rows
    assert a["gather_bytes_per_head"] == sum_k * 2 * w.D * e + w.N * w.k * 4 + w.N * 2 * w.D * e


def test_band_work_counts():
    w = W.get("band_fp32", N=500, window=7, k=15)
    a = bench.algorithmic(w)
    idx = O.band_indices(w.N, w.window, w.window, w.k)
    sum_k = int((idx >= 0).sum())
    assert a["pairs_per_head"] == 0 and a["F_score"] == 0 and a["F_proj"] == 0
    assert a["F_gather"] == 4 * w.D * sum_k * w.B * w.H


def test_bench_runs_on_one_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counters_apply_to_their_command_only():
    """The committed rocprofv3 readings describe the headline command (fp16
    filter operands, 32 heads per selection launch); any other run must report
    them as null rather than borrow them."""
    assert bench.counters_apply("headline_128k", "f16", 32)
    assert bench.counters_apply("headline_128k", "f16", 32.0)
    assert not bench.counters_apply("bf16_32k", "f16", 32)
    assert not bench.counters_apply("causal_mixture", "f16", 32)
    assert not bench.counters_apply("headline_128k", "bf16", 32)
    assert not bench.counters_apply("headline_128k", "f16", 16)
    assert not bench.counters_apply("headline_128k", "f16", None)
    assert bench.gather_counter_frac({"gather": {"ms_total": 1.0, "launches": 1},
                                      "gather_merge": {"ms_total": 1.0, "launches": 1}},
                                     False, False) is None
