"""Parity of the index variants (through the C ABI) with the fp64 oracle:
dilated wrap-around windows, per-sample band radii and boundary smoothing
of the top-k.  Index work is compared bit for bit; attention over the
indices against the oracle's attention, max-abs 1e-5 (fp32) / 2e-2 (bf16)."""
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


@pytest.mark.parametrize("N,window,dilation,k", [(4096, 129, 4, 129), (1000, 50, 37, 64),
                                                 (300, 40, 9, 40), (17, 9, 5, 12), (1, 3, 2, 3)])
def test_dilated_indices_match_oracle(N, window, dilation, k):
    idx = _np(sa.sparse_attn_dilated_indices(2, 3, N, window, dilation, k))
    want = O.dilated_indices(N, window, dilation, k)
    for b in range(2):
        for h in range(3):
            np.testing.assert_array_equal(idx[b, h], want)


def test_dilated_window_attention_band_workload_size():
    """The band workload's shape (2 x 8 heads, N = 4096, D = 64, fp32) with a
    129-entry window at dilation 4: attention against the oracle's, and
    against dense attention under the same mask (no repeats at this size)."""
    w = W.get("band_fp32")
    x = W.make_inputs(w, 0)
    g = {n: t.cuda() for n, t in x.items()}
    idx = sa.sparse_attn_dilated_indices(w.B, w.H, w.N, 129, 4, 129)
    out = _np(sa.sparse_attn_gather(g["Q"], g["K"], g["V"], idx))
    scale = w.D ** -0.5
    i = np.arange(w.N)[:, None]
    j = np.arange(w.N)[None, :]
    off = (j - i) % w.N
    mask = (off % 4 == 0) & (off // 4 < 129)
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            want = O.dense_attention(x["Q"][b:b + 1, h:h + 1], x["K"][b:b + 1, h:h + 1],
                                     x["V"][b:b + 1, h:h + 1], scale, mask=mask)[0, 0]
            worst = max(worst, float(np.abs(out[b, h] - want).max()))
    assert worst <= 1e-5, worst


def test_band_per_batch_matches_oracle_and_dense_attention():
    B, H, N, D = 4, 2, 2000, 64
    radii = torch.tensor([0, 16, 200, 511], dtype=torch.int32)
    k = 2 * 511 + 1
    idx = sa.sparse_attn_band_indices_per_batch(H, N, radii.cuda(), k)
    want = O.band_indices_per_batch(B, H, N, radii.tolist(), k)
    np.testing.assert_array_equal(_np(idx), want)
    gen = torch.Generator().manual_seed(3)
    Q, K, V = (torch.randn(B, H, N, D, generator=gen) for _ in range(3))
    out = _np(sa.sparse_attn_gather(Q.cuda(), K.cuda(), V.cuda(), idx))
    for b, r in enumerate(radii.tolist()):
        ref = O.dense_attention(Q[b:b + 1], K[b:b + 1], V[b:b + 1], D ** -0.5,
                                mask=O.local_mask(N, r))
        assert np.abs(out[b:b + 1] - ref).max() <= 1e-5
    # a negative radius counts as 0; rows are truncated to k entries
    neg = sa.sparse_attn_band_indices_per_batch(1, 50, torch.tensor([-3, 7], dtype=torch.int32,
                                                                    device="cuda"), 5)
    np.testing.assert_array_equal(_np(neg)[0, 0], O.band_indices(50, 0, 0, 5))
    np.testing.assert_array_equal(_np(neg)[1, 0], O.band_indices(50, 7, 7, 5))


def _smooth_case(w, gap, seed, filter_dtype=None):
    x = W.make_inputs(w, seed)
    g = {n: t.cuda() for n, t in x.items()}
    idx = _np(sa.sparse_attn_scores_topk_smoothed(g["Q"], g["K"], g["Pq"], g["Pk"], w.k, gap,
                                                  w.causal, filter_dtype=filter_dtype))
    S = _np(sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], 0, w.N, w.causal))
    rows = list(range(w.N))
    kept_extra = 0
    for b in range(w.B):
        for h in range(w.H):
            want = O.smoothed_topk_rows(S[b, h].astype(np.float64), rows, w.k, w.causal,
                                        float(np.float32(gap)))
            np.testing.assert_array_equal(idx[b, h], want)
            kept_extra += int((want[:, w.k] >= 0).sum())
    return x, g, idx, kept_extra


@pytest.mark.parametrize("N,k,dp,D,dtype,causal,gap", [
    (3000, 64, 16, 64, "f32", False, 0.02),
    (4099, 48, 64, 128, "bf16", True, 0.05),
    (2500, 1, 32, 64, "bf16", False, 0.1),
    (700, 699, 16, 64, "f32", False, 0.5),      # rows hold every key
    (5000, 200, 64, 128, "bf16", False, 0.0),   # no smoothing: plain top-k
])
def test_smoothed_topk_all_rows(N, k, dp, D, dtype, causal, gap):
    w = W.Workload("smooth", 1, 2, N, D, dtype, d_proj=dp, k=k, causal=causal)
    x, g, idx, extra = _smooth_case(w, gap, seed=N + k)
    if gap == 0.0:
        plain = _np(sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], k, causal))
        np.testing.assert_array_equal(idx[..., :k], plain)
        assert np.all(idx[..., k] == -1)
    elif N > k + 1:
        assert extra > 0, "no row kept a (k+1)-th key: the case tests nothing"
    # attention over the smoothed rows (list semantics handle the -1 tail)
    out = _np(sa.sparse_attn_gather(g["Q"], g["K"], g["V"], torch.from_numpy(idx).cuda()).float())
    want = O.gather_attention(x["Q"], x["K"], x["V"], idx, D ** -0.5)
    assert np.abs(out - want).max() <= TOL[w.torch_dtype]


def test_smoothed_topk_infinite_gap_is_top_k_plus_one():
    w = W.Workload("smooth", 1, 2, 3000, 64, "f32", d_proj=16, k=40)
    x = W.make_inputs(w, 8)
    g = {n: t.cuda() for n, t in x.items()}
    sm = sa.sparse_attn_scores_topk_smoothed(g["Q"], g["K"], g["Pq"], g["Pk"], 40, float("inf"))
    plus = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], 41)
    assert torch.equal(sm, plus)
