"""Pins of the oracle's index variants against other formulations:

  * boundary smoothing (page "mhpq.cn/news/1098205", §4.2: keep both the
    k-th and the (k+1)-th key when their score gap is below a threshold):
    pure-Python subset enumeration on tiny rows, and the two closed cases
    (threshold 0 gives the plain top-k, an infinite one the top-(k+1));
  * dilated window with wrap-around (page "Attention机制优化：原理、挑战与
    工程实践", §3.3): each key counted as often as (j - i) mod N hits a
    multiple t*dilation with t < window, and attention over those indices
    equals dense attention under that mask;
  * one band radius per batch sample (page "nxmr.cn/news/163144", §6): dense
    attention under each sample's own band mask.
"""
import itertools

import numpy as np
import pytest

import oracle as O


def _brute_smoothed(s, valid, k, gap):
    """Top-k by enumeration, then the next key by enumeration of the top-(k+1)."""
    keys = [j for j, ok in enumerate(valid) if ok]
    top = O.brute_force_topk(list(s), list(valid), k)
    if len(keys) <= k:
        return top
    top1 = O.brute_force_topk(list(s), list(valid), k + 1)
    nxt = [j for j in top1 if j not in top][0]

    def beats(a, b):
        return s[a] > s[b] or (s[a] == s[b] and a < b)

    # the k-th key: the member of the top-k that every other member beats
    kth = [a for a in top if all(beats(b, a) for b in top if b != a)][0]
    return sorted(top + [nxt]) if s[kth] - s[nxt] < gap else top


@pytest.mark.parametrize("seed", range(6))
def test_smoothing_matches_enumeration(seed):
    rng = np.random.default_rng(seed)
    N = 9
    s = np.round(rng.standard_normal(N), 1)          # coarse values: ties and small gaps
    for causal_row in (None, 5):
        valid = np.ones(N, bool) if causal_row is None else O.valid_keys(N, causal_row, True)
        for k in (1, 3, 5):
            for gap in (0.0, 0.05, 0.15, 0.5, np.inf):
                got = O.smoothed_topk_row(s, valid, k, gap)
                want = _brute_smoothed(s, valid, k, gap)
                assert [int(x) for x in got if x >= 0] == want, (s, k, gap)
                assert np.all(got[len(want):] == -1)


def test_smoothing_closed_cases():
    rng = np.random.default_rng(7)
    S = rng.standard_normal((20, 50))
    rows = list(range(20))
    for k in (1, 7, 49):
        plain = O.topk_rows(S, rows, k, False)
        plus = O.topk_rows(S, rows, k + 1, False)
        np.testing.assert_array_equal(O.smoothed_topk_rows(S, rows, k, False, 0.0)[:, :k], plain)
        assert np.all(O.smoothed_topk_rows(S, rows, k, False, 0.0)[:, k] == -1)
        np.testing.assert_array_equal(O.smoothed_topk_rows(S, rows, k, False, np.inf), plus)
    # an exact tie at the boundary is kept whole for any positive threshold
    s = np.array([3.0, 1.0, 2.0, 2.0, 0.5])
    np.testing.assert_array_equal(O.smoothed_topk_row(s, np.ones(5, bool), 2, 1e-9),
                                  [0, 2, 3])


@pytest.mark.parametrize("N,window,dilation", [(16, 4, 3), (10, 7, 3), (12, 12, 1), (5, 9, 2)])
def test_dilated_indices_count_each_key_by_offset(N, window, dilation):
    idx = O.dilated_indices(N, window, dilation, window + 2)
    for i in range(N):
        row = [int(j) for j in idx[i] if j >= 0]
        assert len(row) == window
        for j in range(N):
            mult = sum(1 for t in range(window) if (j - i) % N == (t * dilation) % N)
            assert row.count(j) == mult
    assert np.all(idx[:, window:] == -1)


def test_dilated_attention_equals_dense_masked_attention():
    rng = np.random.default_rng(3)
    B, H, N, D = 1, 2, 24, 5
    Q, K, V = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    window, dilation = 5, 4                         # window * dilation <= N: no repeats
    idx = O.dilated_indices(N, window, dilation, window)
    got = O.gather_attention(Q, K, V, np.broadcast_to(idx, (B, H, N, window)), 0.4)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    off = (j - i) % N
    mask = (off % dilation == 0) & (off // dilation < window)
    want = O.dense_attention(Q, K, V, 0.4, mask=mask)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    # dilation 1 over the whole sequence: every key once, i.e. dense attention
    full = O.dilated_indices(N, N, 1, N)
    np.testing.assert_allclose(O.gather_attention(Q, K, V, np.broadcast_to(full, (B, H, N, N)),
                                                  0.4),
                               O.dense_attention(Q, K, V, 0.4), rtol=1e-12, atol=1e-12)


def test_per_sample_band_equals_dense_attention_per_sample():
    rng = np.random.default_rng(4)
    B, H, N, D = 3, 2, 30, 4
    Q, K, V = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    radii = [0, 3, 11]
    width = 2 * max(radii) + 1
    idx = O.band_indices_per_batch(B, H, N, radii, width)
    got = O.gather_attention(Q, K, V, idx, 0.3)
    for b, w in enumerate(radii):
        want = O.dense_attention(Q[b:b + 1], K[b:b + 1], V[b:b + 1], 0.3,
                                 mask=O.local_mask(N, w))
        np.testing.assert_allclose(got[b:b + 1], want, rtol=1e-12, atol=1e-12)
        for i in range(N):
            row = [int(x) for x in idx[b, 0, i] if x >= 0]
            assert row == list(range(max(0, i - w), min(N - 1, i + w) + 1))


@pytest.mark.parametrize("length,k", [(40, 8), (5, 8), (1, 3), (40, 40)])
def test_decode_step_is_last_causal_row(length, k):
    """A decode step over cached keys 0..n-1 is row n-1 of the causal
    forward (page "mhpq.cn/news/1098205", §3.4 inference with a KV cache)."""
    rng = np.random.default_rng(length + k)
    B, H, N, D, dp = 1, 1, 40, 6, 4
    Q, K, V = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    Pq, Pk = (rng.standard_normal((D, dp)) for _ in range(2))
    idx_f, out_f = O.sparse_attn_fwd(Q[:, :, :length], K[:, :, :length], V[:, :, :length],
                                     Pq, Pk, k, True, 0.5, 0.3)
    idx_d, o_d = O.decode_step(Q[0, 0, length - 1], K[0, 0], V[0, 0], Pq, Pk, k, length, 0.5,
                               0.3)
    np.testing.assert_array_equal(idx_d, idx_f[0, 0, length - 1])
    np.testing.assert_allclose(o_d, out_f[0, 0, length - 1], rtol=1e-13, atol=1e-13)
    # by enumeration on the same scores (short caches only)
    for n in (min(length, 10),):
        S = O.scores(Q, K, Pq, Pk, 0.5, 0, 0, [n - 1])[0, :n]
        idx_n, _ = O.decode_step(Q[0, 0, n - 1], K[0, 0], V[0, 0], Pq, Pk, min(k, 4), n, 0.5, 0.3)
        want = O.brute_force_topk(list(S), [True] * n, min(k, 4))
        assert [int(x) for x in idx_n if x >= 0] == want


# ------------------------------------------------ block-granular selection ---

def _blk_inputs(N, D, dp, seed):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((1, 2, N, D)) for _ in range(3))
    Pq, Pk = (rng.standard_normal((D, dp)) for _ in range(2))
    return Q, K, V, Pq, Pk


def test_block_score_is_mean_of_fine_scores():
    """Scoring a block by its mean key gives the mean of its keys' scores
    (the score is linear in the key), ragged last block included."""
    Q, K, V, Pq, Pk = _blk_inputs(37, 6, 4, 0)
    S = O.scores(Q, K, Pq, Pk, 0.5, 0, 1)
    kbar = O.block_means(O.project(O.f64(K[0, 1]), O.f64(Pk)), 8)
    SB = O.score_rows(O.project(O.f64(Q[0, 1]), O.f64(Pq)), kbar, 0.5)
    for J in range(5):
        np.testing.assert_allclose(SB[:, J], S[:, J * 8:min(37, J * 8 + 8)].mean(axis=1),
                                   rtol=1e-12, atol=1e-12)


def test_block_size_one_is_plain_top_k():
    Q, K, V, Pq, Pk = _blk_inputs(30, 5, 3, 1)
    np.testing.assert_array_equal(O.block_topk_indices(Q, K, Pq, Pk, 1, 7, False, 0.5),
                                  O.topk_indices(Q, K, Pq, Pk, 7, False, 0.5))


@pytest.mark.parametrize("causal", [False, True])
def test_all_blocks_kept_is_dense_attention(causal):
    Q, K, V, Pq, Pk = _blk_inputs(29, 5, 3, 2)
    idx = O.block_topk_indices(Q, K, Pq, Pk, 4, 8, causal, 0.5)     # 8 blocks of 4 >= 29
    got = O.gather_attention(Q, K, V, idx, 0.4)
    np.testing.assert_allclose(got, O.dense_attention(Q, K, V, 0.4, causal=causal),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_block_selection_by_enumeration(causal):
    """The kept blocks beat every other candidate block (ties to the lower
    block), found by enumerating all subsets of blocks."""
    Q, K, V, Pq, Pk = _blk_inputs(26, 5, 3, 3)
    block, kb = 4, 3
    kbar = O.block_means(O.project(O.f64(K[0, 0]), O.f64(Pk)), block)
    SB = np.round(O.score_rows(O.project(O.f64(Q[0, 0]), O.f64(Pq)), kbar, 0.5), 1)  # force ties
    idx = O.block_topk_indices(Q, K, Pq, Pk, block, kb, causal, 0.5,
                               block_scores=lambda b, h: SB)
    for i in range(26):
        own = i // block
        cands = list(range(own)) if causal else list(range(SB.shape[1]))
        want_n = min(kb - 1, len(cands)) if causal else min(kb, len(cands))
        want = O.brute_force_topk(list(SB[i]), [J in cands for J in range(SB.shape[1])], want_n) \
            if want_n > 0 else []
        if causal:
            want = sorted(want + [own])
        keys = [j for J in want for j in range(J * block, min(26, J * block + block))
                if not causal or j <= i]
        assert [int(x) for x in idx[0, 0, i] if x >= 0] == keys, i
