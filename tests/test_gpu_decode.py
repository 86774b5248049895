"""Decode path (through the C ABI) against the prefill and the fp64 oracle:
one new query per (b, h) over a KV cache whose k_low rows were written by
sparse_attn_decode_append_keys.  With the cache holding keys 0..n-1 the
step's index row must equal, bit for bit, the causal prefill's row n-1 (same
projection and score arithmetic) and the oracle's top-k of the dumped fp32
scores of that row; O must match the oracle's attention over those keys."""
import numpy as np
import pytest
import torch

import dynamic_top_sparse_amd as sa
import oracle as O
from dynamic_top_sparse_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("dtype,D,dp,k,N,lengths,chunks", [
    ("bf16", 128, 64, 64, 3000, (3000, 1777, 40, 1), (1000, 1500, 500)),
    ("f32", 64, 16, 32, 1500, (1500, 33, 31), (1500,)),
    ("bf16", 64, 32, 200, 4100, (4100, 2049), (4100,)),
    ("f32", 128, 128, 50, 4500, (4500, 2048, 2047), (2000, 2500)),
])
def test_decode_equals_prefill_last_row_and_oracle(dtype, D, dp, k, N, lengths, chunks):
    w = W.Workload("dec", 2, 3, N, D, dtype, d_proj=dp, k=k, causal=True)
    x = W.make_inputs(w, 11)
    g = {n: t.cuda() for n, t in x.items()}
    cache = sa.DecodeCache(w.B, w.H, N + 64, D, g["Pq"], g["Pk"], k, dtype=w.torch_dtype)
    pos = 0
    for c in chunks:                       # the keys arrive in pieces
        cache.append(g["K"][:, :, pos:pos + c].contiguous(), g["V"][:, :, pos:pos + c].contiguous())
        pos += c
    assert cache.len == N
    _, pre_idx = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], k, True,
                                    return_idx=True)
    pre_idx = _np(pre_idx)
    sscale, ascale = sa.default_score_scale(dp), sa.default_softmax_scale(D)
    for n in lengths:
        cache.len = n                      # attend over the first n cached keys
        q = g["Q"][:, :, n - 1:n].contiguous()
        idx = torch.empty(w.B, w.H, k, dtype=torch.int32, device="cuda")
        out, idx = cache.step(q, idx=idx)
        idx = _np(idx)
        np.testing.assert_array_equal(idx, pre_idx[:, :, n - 1])
        S = _np(sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], n - 1, 1, True))
        for b in range(w.B):
            for h in range(w.H):
                want = O.topk_rows(S[b, h].astype(np.float64), [n - 1], k, True)[0]
                np.testing.assert_array_equal(idx[b, h], want)
                o_ref = O.attend_row(O.f64(x["Q"][b, h, n - 1]), O.f64(x["K"][b, h, :n]),
                                     O.f64(x["V"][b, h, :n]), idx[b, h].astype(np.int64), ascale)
                err = np.abs(_np(out[b, h, 0].float()) - o_ref).max()
                assert err <= TOL[w.torch_dtype], (n, b, h, err)
        # the oracle's own decode step on fp64 scores agrees up to near ties
        i0, _ = O.decode_step(x["Q"][0, 0, n - 1], x["K"][0, 0], x["V"][0, 0], x["Pq"], x["Pk"],
                              k, n, sscale, ascale)
        S64 = O.scores(x["Q"], x["K"], x["Pq"], x["Pk"], sscale, 0, 0, [n - 1])
        S64[:, n:] = -np.inf
        ov = O.set_overlap(S64, i0[None], idx[0, 0][None])
        assert ov["overlap"] >= 0.999, ov


def test_decode_selection_counts():
    """Selection frequency: every step adds one to each key it keeps."""
    w = W.Workload("dec", 1, 2, 2000, 128, "bf16", d_proj=64, k=50, causal=True)
    x = W.make_inputs(w, 12)
    g = {n: t.cuda() for n, t in x.items()}
    cache = sa.DecodeCache(1, 2, 2000, 128, g["Pq"], g["Pk"], 50)
    cache.append(g["K"][:, :, :1900].contiguous(), g["V"][:, :, :1900].contiguous())
    want = np.zeros((1, 2, 2000), np.int64)
    for t in range(1900, 2000):
        cache.append(g["K"][:, :, t:t + 1].contiguous(), g["V"][:, :, t:t + 1].contiguous())
        idx = torch.empty(1, 2, 50, dtype=torch.int32, device="cuda")
        _, idx = cache.step(g["Q"][:, :, t:t + 1].contiguous(), idx=idx, count=True)
        for h in range(2):
            for j in _np(idx)[0, h]:
                want[0, h, j] += 1
    np.testing.assert_array_equal(_np(cache.counts).astype(np.int64), want)


@pytest.mark.parametrize("same_keys", [False, True])
def test_decode_select_long_cache(same_keys):
    """A 20000-key cache: the select keeps the keys at or above the k-th
    key's leading 11-bit bin in LDS (a small share of random scores); when
    every key scores the same, that bin holds all 20000 keys and the select
    runs over the scores in memory instead.  Both against the oracle's top-k
    of the dumped fp32 scores (all equal: keys 0 .. k-1), with the counts."""
    N, k = 20000, 100
    w = W.Workload("dec", 1, 2, N, 64, "f32", d_proj=16, k=k, causal=True)
    x = W.make_inputs(w, 21)
    if same_keys:
        x["K"][:] = x["K"][:, :, :1].clone()
    g = {n: t.cuda() for n, t in x.items()}
    cache = sa.DecodeCache(1, 2, N, 64, g["Pq"], g["Pk"], k, dtype=torch.float32)
    cache.append(g["K"], g["V"])
    q = g["Q"][:, :, N - 1:N].contiguous()
    idx = torch.empty(1, 2, k, dtype=torch.int32, device="cuda")
    out, idx = cache.step(q, idx=idx, count=True)
    idx = _np(idx)
    S = _np(sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], N - 1, 1, True))
    for h in range(2):
        want = O.topk_rows(S[0, h].astype(np.float64), [N - 1], k, True)[0]
        np.testing.assert_array_equal(idx[0, h], want)
        if same_keys:
            np.testing.assert_array_equal(idx[0, h], np.arange(k))
        counts = np.zeros(N, np.int64)
        counts[idx[0, h]] += 1
        np.testing.assert_array_equal(_np(cache.counts[0, h]).astype(np.int64), counts)
        o_ref = O.attend_row(O.f64(x["Q"][0, h, N - 1]), O.f64(x["K"][0, h]), O.f64(x["V"][0, h]),
                             idx[0, h].astype(np.int64), sa.default_softmax_scale(64))
        assert np.abs(_np(out[0, h, 0]) - o_ref).max() <= 1e-5


@pytest.mark.parametrize("case", ["spread_ties", "slice_overflow"])
def test_decode_select_collect_paths(case):
    """The select finishes over the keys each 2048-key slice of the cache
    collected near the k-th score.  spread_ties: every 100th key shares one
    top score (200 keys over ten slices), k = 100: the 100 lowest-index ones,
    which only the slices taken in order give.  slice_overflow: keys 0..2047
    (slice 0) share the top score, k = 1024: more than a slice's 512 slots,
    so the select runs over the scores in memory; keys 0..1023.  Both against
    the oracle's top-k of the dumped scores, with the counts."""
    N = 20000
    k = 100 if case == "spread_ties" else 1024
    w = W.Workload("dec", 1, 2, N, 64, "f32", d_proj=16, k=k, causal=True)
    x = W.make_inputs(w, 23)
    top = np.arange(0, N, 100) if case == "spread_ties" else np.arange(2048)
    # rows whose projection is about 4 q_low (Pk's columns are nearly
    # orthonormal): a score far above every random key's
    q_low = x["Q"][:, :, N - 1:N].double() @ x["Pq"].double()
    x["K"][:, :, torch.from_numpy(top)] = (4.0 * q_low @ x["Pk"].double().T).float()
    g = {n: t.cuda() for n, t in x.items()}
    cache = sa.DecodeCache(1, 2, N, 64, g["Pq"], g["Pk"], k, dtype=torch.float32)
    cache.append(g["K"], g["V"])
    q = g["Q"][:, :, N - 1:N].contiguous()
    idx = torch.empty(1, 2, k, dtype=torch.int32, device="cuda")
    out, idx = cache.step(q, idx=idx, count=True)
    idx = _np(idx)
    S = _np(sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], N - 1, 1, True))
    for h in range(2):
        want = O.topk_rows(S[0, h].astype(np.float64), [N - 1], k, True)[0]
        np.testing.assert_array_equal(want, top[:k])     # the construction holds
        np.testing.assert_array_equal(idx[0, h], want)
        counts = np.zeros(N, np.int64)
        counts[idx[0, h]] += 1
        np.testing.assert_array_equal(_np(cache.counts[0, h]).astype(np.int64), counts)
        o_ref = O.attend_row(O.f64(x["Q"][0, h, N - 1]), O.f64(x["K"][0, h]), O.f64(x["V"][0, h]),
                             idx[0, h].astype(np.int64), sa.default_softmax_scale(64))
        assert np.abs(_np(out[0, h, 0]) - o_ref).max() <= 1e-5
