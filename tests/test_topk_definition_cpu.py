"""The torch form of the top-k rule used by the all-rows GPU checks
(tests/topk_definition.py) against the oracle's topk_rows, on the CPU:
random tie-heavy integer scores, causal and not, k above and below the
valid count; and a planted mistake (a kept key swapped for a dropped one,
or a row out of order) is caught."""
import numpy as np
import pytest
import torch

import oracle as O
from topk_definition import actual_mask, check_row_form, expected_mask


def test_torch_rule_equals_oracle_topk_rows():
    rng = np.random.default_rng(0)
    for _ in range(300):
        N = int(rng.integers(5, 60))
        k = int(rng.integers(1, 20))
        causal = bool(rng.integers(0, 2))
        R = int(rng.integers(1, 10))
        S = rng.integers(-3, 4, size=(R, N)).astype(np.float32)     # many exact ties
        rows = rng.integers(0, N, size=R)
        want = np.asarray(O.topk_rows(S.astype(np.float64), list(rows), k, causal))
        m, kk = expected_mask(torch.from_numpy(S), torch.from_numpy(rows), k, causal)
        idx = torch.from_numpy(want).int()
        assert torch.equal(actual_mask(idx, N), m)
        check_row_form(idx, kk)


def test_planted_mistakes_are_caught():
    rng = np.random.default_rng(1)
    N, k = 40, 8
    S = rng.integers(-3, 4, size=(6, N)).astype(np.float32)
    rows = np.full(6, N - 1)
    want = np.asarray(O.topk_rows(S.astype(np.float64), list(rows), k, False))
    m, kk = expected_mask(torch.from_numpy(S), torch.from_numpy(rows), k, False)
    bad = torch.from_numpy(want).int().clone()
    dropped = int((~m[0]).nonzero()[0, 0])
    bad[0, 0] = dropped                      # a dropped key in place of a kept one
    assert not torch.equal(actual_mask(bad, N), m)
    swapped = torch.from_numpy(want).int().clone()
    swapped[1, [0, 1]] = swapped[1, [1, 0]]  # same set, out of order
    with pytest.raises(AssertionError):
        check_row_form(swapped, kk)
