"""Pins of the fp64 oracle against things other than itself.

Each test ties one oracle step to an independent fact: the hand-derived
worked example (tests/golden), brute-force enumeration, dense attention
computed without index lists, closed forms (single key, constant V, equal
logits) and invariances (key permutation, idx-entry permutation).  A
mistake in the oracle such as a dropped scale, a transposed projection, a
wrong tie rule, a missing mask or an off-by-one band edge fails at least one
of them.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _ex():
    with open(GOLDEN) as f:
        ex = json.load(f)
    arr = lambda name: np.asarray(ex[name], dtype=np.float64)
    Q = arr("Q")[None, None]
    K = arr("K")[None, None]
    V = arr("V")[None, None]
    return ex, Q, K, V, arr("Pq"), arr("Pk")


# ------------------------------------------------------- worked example ---

@pytest.mark.parametrize("causal", [False, True])
def test_worked_example_indices(causal):
    ex, Q, K, V, Pq, Pk = _ex()
    idx = O.topk_indices(Q, K, Pq, Pk, ex["k"], causal, ex["score_scale"])
    want = ex["idx_causal" if causal else "idx_noncausal"]
    np.testing.assert_array_equal(idx[0, 0], np.asarray(want))


def test_worked_example_outputs():
    ex, Q, K, V, Pq, Pk = _ex()
    for case in ex["cases"]:
        idx, out = O.sparse_attn_fwd(Q, K, V, Pq, Pk, ex["k"], case["causal"],
                                     ex["score_scale"], case["softmax_scale"])
        np.testing.assert_allclose(out[0, 0], np.asarray(case["O"]), rtol=0, atol=1e-15)


# ------------------------------------------------------------ selection ---

@settings(max_examples=200, deadline=None)
@given(n=st.integers(1, 9), k=st.integers(1, 5), seed=st.integers(0, 2**31 - 1),
       causal_row=st.one_of(st.none(), st.integers(0, 8)))
def test_topk_matches_brute_force(n, k, seed, causal_row):
    rng = np.random.default_rng(seed)
    s = rng.integers(-3, 4, size=n).astype(np.float64)   # small range: many ties
    valid = np.ones(n, dtype=bool)
    if causal_row is not None:
        valid[min(causal_row, n - 1) + 1:] = False
    got = O.topk_row(s, valid, k)
    want = O.brute_force_topk(list(s), list(valid), k)
    kept = min(k, int(valid.sum()))
    assert list(got[:kept]) == want
    assert np.all(got[kept:] == -1)


def test_topk_keeps_all_valid_when_fewer_than_k():
    s = np.array([0.3, -1.0, 2.0, 5.0, 1.0])
    got = O.topk_row(s, O.valid_keys(5, 2, causal=True), 4)
    np.testing.assert_array_equal(got, [0, 1, 2, -1])


def test_topk_tie_goes_to_lower_index_including_signed_zero():
    s = np.array([0.0, -0.0, 1.0, 0.0])
    np.testing.assert_array_equal(O.topk_row(s, np.ones(4, bool), 2), [0, 2])
    s = np.array([-0.0, 0.0, 1.0])
    np.testing.assert_array_equal(O.topk_row(s, np.ones(3, bool), 2), [0, 2])


def test_selection_every_kept_beats_every_dropped():
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((1, 2, 300, 16))
    K = rng.standard_normal((1, 2, 300, 16))
    Pq = rng.standard_normal((16, 8))
    Pk = rng.standard_normal((16, 8))
    for causal in (False, True):
        idx = O.topk_indices(Q, K, Pq, Pk, 20, causal, 8 ** -0.5)
        for h in range(2):
            S = O.scores(Q, K, Pq, Pk, 8 ** -0.5, 0, h)
            for i in range(0, 300, 7):
                valid = O.valid_keys(300, i, causal)
                kept = idx[0, h, i][idx[0, h, i] >= 0]
                O.row_invariants(idx[0, h, i], 20, int(valid.sum()), 299)
                dropped = np.setdiff1d(np.nonzero(valid)[0], kept)
                if dropped.size:
                    assert S[i, kept].min() >= S[i, dropped].max()


def test_identity_scorer_ranks_keys_like_dense_attention_probabilities():
    """With Pq = Pk = I_D and score_scale = softmax_scale = D^-1/2 the scorer
    is the attention logit itself ("scorer v1" on page mhpq.cn/news/1098205,
    section 2.2).  Dense attention with V = I_N returns the probability
    matrix P, computed without the scorer: the oracle's scores must equal
    log P up to a per-row constant (pins scale and orientation), and the
    kept sets must be the k largest probabilities."""
    rng = np.random.default_rng(2)
    N, D, k = 64, 8, 10
    Q = rng.standard_normal((1, 1, N, D))
    K = rng.standard_normal((1, 1, N, D))
    eye = np.eye(D)
    c = D ** -0.5
    S = O.scores(Q, K, eye, eye, c, 0, 0)
    P = O.dense_attention(Q, K, np.eye(N)[None, None], c)[0, 0]
    d = S - np.log(P)
    np.testing.assert_allclose(d - d[:, :1], 0.0, atol=1e-12)
    idx = O.topk_indices(Q, K, eye, eye, k, False, c)[0, 0]
    for i in range(N):
        want = np.sort(np.argsort(-P[i], kind="stable")[:k])
        np.testing.assert_array_equal(idx[i], want)


def test_projection_orientation_and_per_head_inputs():
    """Scores use Q·Pq with Pq of shape [D, d_proj] and each head's own Q, K:
    a rank-one projection onto coordinate 0 reduces S to a product of the
    first coordinates."""
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((2, 3, 5, 4))
    K = rng.standard_normal((2, 3, 5, 4))
    P = np.zeros((4, 2)); P[0, 0] = 1.0
    for b in range(2):
        for h in range(3):
            S = O.scores(Q, K, P, P, 0.5, b, h)
            np.testing.assert_allclose(S, 0.5 * np.outer(Q[b, h, :, 0], K[b, h, :, 0]),
                                       atol=1e-15)


# ------------------------------------------------------------ attention ---

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_k_equal_n_is_dense_attention(causal):
    B, H, N, D, dp = 1, 2, 48, 16, 4
    Q, K, V = _rand((B, H, N, D), 4), _rand((B, H, N, D), 5), _rand((B, H, N, D), 6)
    Pq, Pk = _rand((D, dp), 7), _rand((D, dp), 8)
    _, out = O.sparse_attn_fwd(Q, K, V, Pq, Pk, N, causal, dp ** -0.5, D ** -0.5)
    want = O.dense_attention(Q, K, V, D ** -0.5, causal=causal)
    np.testing.assert_allclose(out, want, atol=1e-12)


@pytest.mark.parametrize("w_left,w_right", [(5, 5), (64, 64), (0, 3), (7, 0)])
def test_band_indices_equal_local_mask_and_dense_masked_attention(w_left, w_right):
    N, D = 150, 8
    idx = O.band_indices(N, w_left, w_right, w_left + w_right + 1)
    allowed = np.zeros((N, N), bool)
    for i in range(N):
        row = idx[i][idx[i] >= 0]
        assert np.all(np.diff(row) > 0)
        allowed[i, row] = True
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    np.testing.assert_array_equal(allowed, (j >= i - w_left) & (j <= i + w_right))
    if w_left == w_right:
        np.testing.assert_array_equal(allowed, O.local_mask(N, w_left))
    Q, K, V = _rand((1, 2, N, D), 9), _rand((1, 2, N, D), 10), _rand((1, 2, N, D), 11)
    full = np.broadcast_to(idx, (1, 2, N, idx.shape[1]))
    got = O.gather_attention(Q, K, V, full, D ** -0.5)
    want = O.dense_attention(Q, K, V, D ** -0.5, mask=allowed)
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_band_edges_are_clipped_not_wrapped():
    idx = O.band_indices(10, 2, 2, 5)
    np.testing.assert_array_equal(idx[0], [0, 1, 2, -1, -1])
    np.testing.assert_array_equal(idx[9], [7, 8, 9, -1, -1])
    np.testing.assert_array_equal(idx[5], [3, 4, 5, 6, 7])


def test_softmax_weights_sum_to_one_and_constant_v():
    N, D, k = 40, 8, 7
    rng = np.random.default_rng(12)
    Q, K = rng.standard_normal((1, 1, N, D)), rng.standard_normal((1, 1, N, D))
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(N)])[None, None]
    ones = np.ones((1, 1, N, D))
    np.testing.assert_allclose(O.gather_attention(Q, K, ones, idx, 0.3), 1.0, atol=1e-14)
    const = np.full((1, 1, N, D), -2.5)
    np.testing.assert_allclose(O.gather_attention(Q, K, const, idx, 0.3), -2.5, atol=1e-14)


def test_single_key_and_equal_logits_and_empty_row():
    rng = np.random.default_rng(13)
    N, D = 12, 4
    Q, K, V = rng.standard_normal((1, 1, N, D)), rng.standard_normal((1, 1, N, D)), \
        rng.standard_normal((1, 1, N, D))
    idx = np.full((1, 1, N, 3), -1, dtype=np.int32)
    idx[0, 0, :, 0] = np.arange(N)[::-1]
    out = O.gather_attention(Q, K, V, idx, 0.7)
    np.testing.assert_array_equal(out[0, 0], V[0, 0, ::-1])          # exact copy
    Qz = np.zeros_like(Q)                                            # all logits 0
    idx2 = np.tile(np.array([1, 4, 9], dtype=np.int32), (1, 1, N, 1))
    out2 = O.gather_attention(Qz, K, V, idx2, 0.7)
    np.testing.assert_allclose(out2[0, 0], np.tile(V[0, 0, [1, 4, 9]].mean(0), (N, 1)),
                               atol=1e-15)
    empty = np.full((1, 1, N, 3), -1, dtype=np.int32)
    assert np.all(O.gather_attention(Q, K, V, empty, 0.7) == 0.0)


def test_output_invariant_to_key_order_and_idx_order():
    rng = np.random.default_rng(14)
    B, H, N, D, dp, k = 1, 1, 60, 8, 4, 9
    Q, K, V = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    Pq, Pk = rng.standard_normal((D, dp)), rng.standard_normal((D, dp))
    idx, out = O.sparse_attn_fwd(Q, K, V, Pq, Pk, k, False, 0.5, 0.35)
    perm = rng.permutation(N)                     # new position p holds old key perm[p]
    inv = np.argsort(perm)
    Kp, Vp = K[:, :, perm], V[:, :, perm]
    idx_p, out_p = O.sparse_attn_fwd(Q, Kp, Vp, Pq, Pk, k, False, 0.5, 0.35)
    np.testing.assert_allclose(out_p, out, atol=1e-12)
    # the kept sets are the same keys (tie-free inputs), renamed
    for i in range(N):
        np.testing.assert_array_equal(np.sort(perm[idx_p[0, 0, i]]), idx[0, 0, i])
    shuffled = idx.copy()
    for i in range(N):
        shuffled[0, 0, i] = rng.permutation(shuffled[0, 0, i])
    np.testing.assert_allclose(O.gather_attention(Q, K, V, shuffled, 0.35), out, atol=1e-12)
    del inv


def test_duplicates_count_twice():
    rng = np.random.default_rng(15)
    N, D = 6, 3
    Q, K, V = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    idx = np.tile(np.array([2, 2, 5], dtype=np.int32), (1, 1, N, 1))
    got = O.gather_attention(Q, K, V, idx, 1.0)[0, 0]
    for i in range(N):
        want = O.brute_force_attention(Q[0, 0, i], K[0, 0, [2, 2, 5]], V[0, 0, [2, 2, 5]], 1.0)
        np.testing.assert_allclose(got[i], want, atol=1e-14)


@settings(max_examples=60, deadline=None)
@given(n=st.integers(2, 12), d=st.integers(1, 5), k=st.integers(1, 12),
       seed=st.integers(0, 2**31 - 1), scale=st.floats(0.05, 3.0))
def test_gather_matches_pure_python_summation(n, d, k, seed, scale):
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    sel = rng.integers(-1, n, size=(n, k)).astype(np.int32)
    got = O.gather_attention(Q, K, V, sel[None, None], scale)[0, 0]
    for i in range(n):
        rows = [int(j) for j in sel[i] if j >= 0]
        if not rows:
            assert np.all(got[i] == 0)
            continue
        want = O.brute_force_attention(Q[0, 0, i], [K[0, 0, j] for j in rows],
                                       [V[0, 0, j] for j in rows], scale)
        np.testing.assert_allclose(got[i], want, rtol=1e-12, atol=1e-12)


def test_f64_upcast_is_exact_for_bf16():
    torch = pytest.importorskip("torch")
    x = torch.tensor([1.0, -2.5, 3.140625, 1e-3], dtype=torch.bfloat16)
    got = O.f64(x)
    want = np.array([float(v) for v in x.float()])
    np.testing.assert_array_equal(got, want)


# -------------------------------------------------------------- overlap ---

def test_overlap_excuses_only_near_ties():
    S = np.array([[5.0, 4.0, 3.0, 2.9995, 1.0, 0.0]])
    A = np.array([[0, 1, 2]])
    G_tie = np.array([[0, 1, 3]])           # swap 2 (3.0) for 3 (2.9995): excused
    G_bad = np.array([[0, 1, 4]])           # swap 2 for 4 (1.0): not excused
    assert O.set_overlap(S, A, G_tie)["overlap"] == 1.0
    assert O.set_overlap(S, A, G_tie)["raw_overlap"] == pytest.approx(2 / 3)
    r = O.set_overlap(S, A, G_bad)
    assert r["overlap"] == pytest.approx(2 / 3) and r["unexcused"] == 1


def test_row_invariants_catch_malformed_rows():
    O.row_invariants(np.array([1, 5, 9, -1]), 4, 3, 9)
    for bad in ([5, 1, 9, -1], [1, 1, 9, -1], [1, 5, -1, 9], [1, 5, 10, -1]):
        with pytest.raises(AssertionError):
            O.row_invariants(np.array(bad), 4, 3, 9)
