"""Comparison rules between a GPU result and the fp64 oracle.

TEST INFRASTRUCTURE ONLY (see sparse_attn_oracle.py).

Set overlap with near-tie excuse.  For one query row let A be the oracle's
kept set and G the GPU's.  The keys of A∖G (missed) are sorted by oracle
score ascending, those of G∖A (taken instead) descending, and paired in that
order.  A pair (a, b) is excused when S_a - S_b < eps: the GPU swapped two
keys whose exact scores differ by less than eps.  The overlap is
1 - (unexcused pairs) / (kept keys), summed over rows.  The hard invariants
are checked separately: a GPU row has exactly min(k, #valid) distinct valid
keys in ascending order, then -1 padding.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np


def row_invariants(idx_row: np.ndarray, k: int, n_valid_keys: int, max_key: int) -> None:
    """Raise AssertionError unless idx_row is a well-formed selection:
    min(k, n_valid_keys) distinct keys in [0, max_key], strictly ascending,
    followed by -1 entries only."""
    kept = min(k, n_valid_keys)
    row = np.asarray(idx_row, dtype=np.int64)
    assert row.shape == (k,), f"row has shape {row.shape}, want ({k},)"
    head, tail = row[:kept], row[kept:]
    assert np.all(tail == -1), f"padding is not -1: {tail[:8]}"
    assert np.all(head >= 0) and np.all(head <= max_key), "key out of range"
    assert np.all(np.diff(head) > 0), "keys not strictly ascending"


def set_overlap(S: np.ndarray, oracle_idx: np.ndarray, gpu_idx: np.ndarray,
                eps: float = 1e-3) -> Dict[str, float]:
    """S [R, N] fp64 oracle scores; oracle_idx, gpu_idx [R, k] (-1 padded).
    Returns overlap, raw (unexcused-free) overlap, the worst row's overlap and
    counts."""
    total = 0
    missed_total = 0
    unexcused_total = 0
    worst = 1.0
    for r in range(S.shape[0]):
        A = set(int(x) for x in oracle_idx[r] if x >= 0)
        G = set(int(x) for x in gpu_idx[r] if x >= 0)
        assert len(A) == len(G), "kept-set sizes differ"
        missed = sorted(A - G, key=lambda j: S[r, j])
        extra = sorted(G - A, key=lambda j: -S[r, j])
        unexcused = sum(1 for a, b in zip(missed, extra) if S[r, a] - S[r, b] >= eps)
        total += len(A)
        missed_total += len(missed)
        unexcused_total += unexcused
        if A:
            worst = min(worst, 1.0 - unexcused / len(A))
    return {
        "overlap": 1.0 - unexcused_total / max(total, 1),
        "raw_overlap": 1.0 - missed_total / max(total, 1),
        "worst_row": worst,
        "kept": float(total),
        "unexcused": float(unexcused_total),
    }
