"""Pins of the oracle's backward (page "mhpq.cn/news/1098205", §2.3: hard
top-k forward; selected positions' gradients flow, unselected ones get zero;
the scorer's gradient goes through the selected positions' attention weights)
against things other than the oracle itself:

  * torch.autograd in float64 on an independent forward: dense masked
    attention whose logits of kept pairs carry S - S.detach() (value zero,
    gradient one: the straight-through reading) - for dQ, dK, dV, dPq, dPk;
  * torch.autograd on a gather formulation with -1 entries and repeated
    entries (list semantics) for the attention path;
  * central finite differences of the oracle's own forward (attention over
    fixed index sets), which are true gradients there;
  * k = N against autograd of plain dense softmax attention;
  * closed-form invariants: the dV rows sum to the dO rows, unselected keys
    get nothing, each row's logit gradients sum to zero.
"""
import numpy as np
import pytest
import torch

import oracle as O


def _inputs(B, H, N, D, dp, seed):
    g = np.random.default_rng(seed)
    Q, K, V = (g.standard_normal((B, H, N, D)) for _ in range(3))
    Pq, Pk = (g.standard_normal((D, dp)) / np.sqrt(D) for _ in range(2))
    dO = g.standard_normal((B, H, N, D))
    return Q, K, V, Pq, Pk, dO


def _surrogate_grads(Q, K, V, Pq, Pk, idx, dO, sscale, ascale, scorer):
    """Autograd of sum(O * dO) where O is dense attention restricted to the
    kept pairs, whose logits gain S - S.detach() when `scorer` is set."""
    t = {n: torch.tensor(a, requires_grad=True) for n, a in
         dict(Q=Q, K=K, V=V, Pq=Pq, Pk=Pk).items()}
    B, H, N, D = Q.shape
    keep = torch.zeros(B, H, N, N, dtype=torch.bool)
    for b in range(B):
        for h in range(H):
            for i in range(N):
                for j in idx[b, h, i]:
                    if j >= 0:
                        keep[b, h, i, j] = True
    logits = ascale * t["Q"] @ t["K"].transpose(-1, -2)
    if scorer:
        S = sscale * (t["Q"] @ t["Pq"]) @ (t["K"] @ t["Pk"]).transpose(-1, -2)
        logits = logits + (S - S.detach())
    logits = logits.masked_fill(~keep, float("-inf"))
    P = torch.softmax(logits, dim=-1)
    P = torch.nan_to_num(P)          # rows without kept keys give O = 0
    out = P @ t["V"]
    (out * torch.tensor(dO)).sum().backward()
    return {n: (v.grad.numpy() if v.grad is not None else np.zeros(v.shape))
            for n, v in t.items()}


@pytest.mark.parametrize("causal,k,seed", [(False, 3, 0), (True, 4, 1), (False, 9, 2),
                                           (True, 12, 3)])
def test_backward_matches_autograd_of_straight_through_surrogate(causal, k, seed):
    B, H, N, D, dp = 2, 2, 10, 6, 4
    Q, K, V, Pq, Pk, dO = _inputs(B, H, N, D, dp, seed)
    sscale, ascale = dp ** -0.5, D ** -0.5
    idx = O.topk_indices(Q, K, Pq, Pk, k, causal, sscale)
    got = O.sparse_attn_backward(Q, K, V, Pq, Pk, idx, dO, sscale, ascale, scorer_grad=True)
    want = _surrogate_grads(Q, K, V, Pq, Pk, idx, dO, sscale, ascale, scorer=True)
    for name, g in zip(("Q", "K", "V", "Pq", "Pk"), got):
        np.testing.assert_allclose(g, want[name], rtol=1e-10, atol=1e-12, err_msg=name)
    # without the scorer path: the attention gradients alone, and zero for P
    got = O.sparse_attn_backward(Q, K, V, Pq, Pk, idx, dO, sscale, ascale, scorer_grad=False)
    want = _surrogate_grads(Q, K, V, Pq, Pk, idx, dO, sscale, ascale, scorer=False)
    for name, g in zip(("Q", "K", "V"), got[:3]):
        np.testing.assert_allclose(g, want[name], rtol=1e-10, atol=1e-12, err_msg=name)
    assert not got[3].any() and not got[4].any()


def test_attention_backward_with_repeats_and_padding_matches_autograd_gather():
    """List semantics: -1 entries are skipped, a repeated entry counts twice,
    a row without entries has no gradient."""
    B, H, N, D, k = 1, 1, 7, 5, 5
    Q, K, V, Pq, Pk, dO = _inputs(B, H, N, D, 3, 4)
    idx = np.array([[[[0, 3, 3, -1, 6], [-1, -1, -1, -1, -1], [1, 2, 4, 5, 6],
                      [2, 2, 2, 2, 2], [6, 5, 4, -1, 0], [3, -1, 1, -1, 3],
                      [0, 1, 2, 3, 4]]]])
    ascale = 0.7
    got = O.sparse_attn_backward(Q, K, V, Pq, Pk, idx, dO, 0.5, ascale, scorer_grad=False)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    loss = 0.0
    for i in range(N):
        sel = torch.tensor([j for j in idx[0, 0, i] if j >= 0], dtype=torch.long)
        if sel.numel() == 0:
            continue
        lg = ascale * tk[0, 0, sel] @ tq[0, 0, i]
        o = torch.softmax(lg, 0) @ tv[0, 0, sel]
        loss = loss + (o * torch.tensor(dO[0, 0, i])).sum()
    loss.backward()
    for g, t in zip(got[:3], (tq, tk, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12)
    assert not got[0][0, 0, 1].any()


def test_attention_backward_matches_finite_differences():
    """Central differences of the oracle's forward over fixed index sets."""
    B, H, N, D, dp, k = 1, 2, 9, 4, 3, 4
    Q, K, V, Pq, Pk, dO = _inputs(B, H, N, D, dp, 5)
    ascale = 0.6
    idx = O.topk_indices(Q, K, Pq, Pk, k, False, 1.0)
    dQ, dK, dV, _, _ = O.sparse_attn_backward(Q, K, V, Pq, Pk, idx, dO, 1.0, ascale,
                                              scorer_grad=False)

    def loss(Qx, Kx, Vx):
        return float((O.gather_attention(Qx, Kx, Vx, idx, ascale) * dO).sum())

    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, arr, grad in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for _ in range(12):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            xp, xm = arr.copy(), arr.copy()
            xp[pos] += eps
            xm[pos] -= eps
            args_p = {"Q": Q, "K": K, "V": V}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd = (loss(args_p["Q"], args_p["K"], args_p["V"])
                  - loss(args_m["Q"], args_m["K"], args_m["V"])) / (2 * eps)
            assert abs(fd - grad[pos]) <= 1e-7 * max(1.0, abs(fd)), (name, pos, fd, grad[pos])


@pytest.mark.parametrize("causal", [False, True])
def test_k_equal_N_is_dense_attention_backward(causal):
    B, H, N, D, dp = 1, 2, 8, 5, 3
    Q, K, V, Pq, Pk, dO = _inputs(B, H, N, D, dp, 6)
    ascale = D ** -0.5
    idx = O.topk_indices(Q, K, Pq, Pk, N, causal, 1.0)
    got = O.sparse_attn_backward(Q, K, V, Pq, Pk, idx, dO, 1.0, ascale, scorer_grad=False)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (Q, K, V))
    mask = torch.tril(torch.ones(N, N, dtype=torch.bool)) if causal else None
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=ascale)
    (out * torch.tensor(dO)).sum().backward()
    for g, t in zip(got[:3], (tq, tk, tv)):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-9, atol=1e-11)


def test_backward_invariants():
    B, H, N, D, dp, k = 2, 3, 11, 6, 4, 3
    Q, K, V, Pq, Pk, dO = _inputs(B, H, N, D, dp, 7)
    idx = O.topk_indices(Q, K, Pq, Pk, k, True, 0.5)
    dQ, dK, dV, dPq, dPk = O.sparse_attn_backward(Q, K, V, Pq, Pk, idx, dO, 0.5, 0.4)
    # softmax weights of a row sum to one: the dV rows of a head sum to its dO rows
    np.testing.assert_allclose(dV.sum(axis=2), dO.sum(axis=2), rtol=1e-12, atol=1e-12)
    # keys no row kept get no gradient at all
    for b in range(B):
        for h in range(H):
            kept = set(int(j) for j in idx[b, h].ravel() if j >= 0)
            for j in range(N):
                if j not in kept:
                    assert not dV[b, h, j].any() and not dK[b, h, j].any()
    # each row's logit gradients sum to zero
    for i in range(N):
        _, _, _, dl = O.attend_row_backward(O.f64(Q)[0, 0, i], O.f64(K)[0, 0], O.f64(V)[0, 0],
                                            idx[0, 0, i].astype(np.int64), 0.4, dO[0, 0, i])
        assert abs(dl.sum()) < 1e-12
