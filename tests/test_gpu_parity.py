"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Bars (stated in the method's contract):
  * idx: bit-exact equality with the oracle's top-k recomputed from the
    library's own dumped fp32 scores (same tie rule), on every checked row;
    hard invariants on every row; set overlap >= 0.999 against the oracle's
    fp64 scores, pairs whose fp64 scores differ by < 1e-3 excused.
  * O: max-abs error vs the oracle's fp64 attention over the library's idx
    <= 1e-5 for fp32 I/O and <= 2e-2 for bf16 I/O (fp32 accumulation).
Small cases are checked on every row; the full-size workloads on sampled
row ranges.
"""
import numpy as np
import pytest
import torch

import dynamic_top_sparse_amd as sa
import oracle as O
from dynamic_top_sparse_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def _cuda(x):
    return {k: v.cuda() for k, v in x.items()}


def _rows_np(t):
    return t.detach().cpu().numpy()


def check_idx_rows(idx_rows, S_dump, S64, rows, k, causal, N):
    """idx_rows [R,k] from the GPU; S_dump [R,N] its fp32 scores; S64 [R,N]
    the oracle's fp64 scores for the same rows."""
    want = O.topk_rows(S_dump.astype(np.float64), rows, k, causal)
    np.testing.assert_array_equal(idx_rows, want)
    for r, i in enumerate(rows):
        nv = int(i) + 1 if causal else N
        O.row_invariants(idx_rows[r], k, nv, N - 1 if not causal else int(i))
    ora = O.topk_rows(S64, rows, k, causal)
    ov = O.set_overlap(S64, ora, idx_rows)
    assert ov["overlap"] >= 0.999, ov
    return ov


def run_case(w: W.Workload, seed=0, rows=None, check_all=True):
    x = W.make_inputs(w, seed)
    g = _cuda(x)
    B, H, N, D = w.B, w.H, w.N, w.D
    ws = sa.allocate_workspace(g["Q"], w.d_proj, w.k, w.causal, with_idx=False)
    idx = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k, w.causal,
                                     workspace=ws)
    out, idx2 = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, w.causal,
                                   return_idx=True)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "fused and split paths disagree"
    stats = sa.sparse_attn_workspace_stats(ws)
    # the exact fallback keeps results right even when the filter is broken,
    # so a flood of fallbacks must fail the test on its own
    if w.N >= 4096:
        assert stats["fallback_queries"] <= 0.05 * w.queries, stats
    idx_np = _rows_np(idx)
    if rows is None:
        ranges = [(0, N)]
    else:
        ranges = rows
    sscale = sa.default_score_scale(w.d_proj)
    ascale = sa.default_softmax_scale(D)
    for (r0, rc) in ranges:
        S = sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], r0, rc, w.causal)
        S_np = _rows_np(S)
        rr = list(range(r0, r0 + rc))
        for b in range(B):
            for h in range(H):
                S64 = O.scores(x["Q"], x["K"], x["Pq"], x["Pk"], sscale, b, h, rr)
                if w.causal:
                    S64 = np.where(np.arange(N)[None, :] <= np.asarray(rr)[:, None], S64, -np.inf)
                check_idx_rows(idx_np[b, h, r0:r0 + rc], S_np[b, h], S64, rr, w.k, w.causal, N)
        want = O.gather_attention(x["Q"], x["K"], x["V"], idx_np[:, :, r0:r0 + rc], ascale, rr)
        got = _rows_np(out[:, :, r0:r0 + rc].float())
        err = np.abs(got - want).max()
        assert err <= TOL[w.torch_dtype], (err, w)
    return stats


# ------------------------------------------------------------- gather ---

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("k", [1, 7, 100])
def test_gather_random_index_lists(dtype, D, k):
    B, H, N = 1, 3, 517
    gen = torch.Generator().manual_seed(D * 1000 + k)
    Q, K, V = (torch.randn(B, H, N, D, generator=gen).to(dtype) for _ in range(3))
    idx = torch.randint(-1, N, (B, H, N, k), generator=gen, dtype=torch.int32)
    idx[0, 0, 5] = -1                      # an empty row
    if k > 2:
        idx[0, 1, 3, :3] = 11               # duplicates count twice
    got = sa.sparse_attn_gather(Q.cuda(), K.cuda(), V.cuda(), idx.cuda(), 0.3)
    want = O.gather_attention(Q, K, V, idx.numpy(), 0.3)
    err = np.abs(_rows_np(got.float()) - want).max()
    assert err <= TOL[dtype], err
    assert torch.all(got[0, 0, 5] == 0)
    assert sa.sparse_attn_check_status() == 0


def test_gather_flags_out_of_range_index():
    Q = torch.randn(1, 1, 64, 64).cuda()
    idx = torch.zeros(1, 1, 64, 4, dtype=torch.int32)
    idx[0, 0, 10, 2] = 64                   # == N: skipped and flagged
    got = sa.sparse_attn_gather(Q, Q, Q, idx.cuda(), 0.125)
    assert sa.sparse_attn_check_status() == -7
    assert sa.sparse_attn_check_status() == 0       # the flag is cleared
    want = O.gather_attention(Q.cpu(), Q.cpu(), Q.cpu(),
                              np.where(idx.numpy() >= 64, -1, idx.numpy()), 0.125)
    assert np.abs(_rows_np(got) - want).max() <= 1e-5


@pytest.mark.parametrize("w_left,w_right,N", [(64, 64, 4096), (5, 5, 1024), (0, 7, 300),
                                              (9, 0, 301)])
def test_band_indices_match_oracle(w_left, w_right, N):
    idx = sa.sparse_attn_band_indices(2, 3, N, w_left, w_right)
    want = O.band_indices(N, w_left, w_right, w_left + w_right + 1)
    got = _rows_np(idx)
    for b in range(2):
        for h in range(3):
            np.testing.assert_array_equal(got[b, h], want)


def test_band_workload_equals_dense_sliding_window_attention():
    """Band mode at its full size: 2 x 8 heads, N=4096, D=64, window +-64
    (129 keys, clipped), fp32 - compared with dense masked attention."""
    w = W.get("band_fp32")
    x = W.make_inputs(w, 0)
    g = _cuda(x)
    idx = sa.sparse_attn_band_indices(w.B, w.H, w.N, w.window, w.window)
    out = sa.sparse_attn_gather(g["Q"], g["K"], g["V"], idx)
    got = _rows_np(out)
    mask = O.local_mask(w.N, w.window)
    scale = w.D ** -0.5
    worst = 0.0
    for b in range(w.B):
        for h in range(w.H):
            want = O.dense_attention(x["Q"][b:b + 1, h:h + 1], x["K"][b:b + 1, h:h + 1],
                                     x["V"][b:b + 1, h:h + 1], scale, mask=mask)[0, 0]
            worst = max(worst, float(np.abs(got[b, h] - want).max()))
    assert worst <= 1e-5, worst


# ------------------------------------------------------------ scores ---

@pytest.mark.parametrize("causal", [False, True])
def test_scores_dump_close_to_fp64(causal):
    w = W.get("tiny_fp32", N=700, H=2, causal=causal)
    x = W.make_inputs(w, 3)
    g = _cuda(x)
    S = _rows_np(sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], 0, 700, causal))
    for h in range(2):
        S64 = O.scores(x["Q"], x["K"], x["Pq"], x["Pk"], 0.25, 0, h)
        if causal:
            tri = np.tril(np.ones((700, 700), bool))
            assert np.all(np.isneginf(S[0, h][~tri]))
            np.testing.assert_allclose(S[0, h][tri], S64[tri], atol=2e-5, rtol=0)
        else:
            np.testing.assert_allclose(S[0, h], S64, atol=2e-5, rtol=0)


# ----------------------------------------------------- top-k + forward ---

def test_tiny_fp32_workload_all_rows():
    """Tiny fp32 workload: B=1 H=1 N=1024 D=64 d_proj=16 k=32."""
    run_case(W.get("tiny_fp32"))


@pytest.fixture(params=[torch.float16, torch.bfloat16], ids=["filter_f16", "filter_bf16"])
def filter_dtype(request):
    """Runs a test with each 16-bit operand type of the MFMA filter; the
    indices must not depend on it."""
    before = sa.sparse_attn_get_filter_dtype()
    sa.sparse_attn_set_filter_dtype(request.param)
    yield request.param
    sa.sparse_attn_set_filter_dtype(before)


@pytest.mark.parametrize("N,k,dp,D,dtype,causal", [
    (5000, 64, 16, 64, "f32", False),       # sample + filter path, ragged tail
    (5000, 64, 64, 128, "bf16", False),
    (4099, 48, 32, 64, "bf16", True),       # causal: early rows keep all keys
    (3001, 200, 64, 128, "f32", True),
    (2500, 1, 16, 64, "f32", False),        # k = 1
    (600, 700, 16, 64, "f32", False),       # k > N: all keys, -1 padding
    (1, 5, 16, 64, "f32", True),            # a single query
    (5000, 96, 128, 64, "bf16", True),      # d_proj 128
])
def test_topk_and_forward_small_shapes_all_rows(N, k, dp, D, dtype, causal, filter_dtype):
    w = W.Workload("case", 1, 2, N, D, dtype, d_proj=dp, k=k, causal=causal)
    run_case(w, seed=N + k)


def test_largest_k_with_key_range_gather_all_rows():
    """k at its maximum (2048, lists of 2048 entries per half) past the
    threshold path's minimum N and the key-range gather's, d_proj 128."""
    w = W.Workload("case", 1, 1, 9000, 128, "bf16", d_proj=128, k=2048)
    run_case(w, seed=77)


def test_mixture_causal_small_all_rows(filter_dtype):
    w = W.get("causal_mixture", B=2, H=2, N=6000, k=64)
    run_case(w, seed=5)


def test_exact_ties_go_to_lower_index(filter_dtype):
    """Duplicated key rows give bit-identical scores; the lower index wins."""
    w = W.Workload("ties", 1, 1, 3000, 64, "f32", d_proj=16, k=40)
    x = W.make_inputs(w, 9)
    K = x["K"].clone()
    K[0, 0, 2000:2600] = K[0, 0, 0:600]     # keys 2000.. repeat keys 0..
    x["K"] = K
    g = _cuda(x)
    idx = _rows_np(sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k))
    S = _rows_np(sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], 0, 3000))
    assert np.array_equal(S[0, 0][:, 2000:2600], S[0, 0][:, 0:600])
    want = O.topk_rows(S[0, 0].astype(np.float64), list(range(3000)), w.k, False)
    np.testing.assert_array_equal(idx[0, 0], want)


def test_repeated_runs_are_bit_identical():
    w = W.get("bf16_32k", N=8192, H=2, k=128)
    g = _cuda(W.make_inputs(w, 4))
    a = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, return_idx=True)
    b = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, return_idx=True)
    assert torch.equal(a[1], b[1]) and torch.equal(a[0], b[0])


def test_small_workspace_runs_head_by_head():
    w = W.get("bf16_32k", N=4096, H=3, k=64)
    g = _cuda(W.make_inputs(w, 6))
    full = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k)
    ws1 = sa.allocate_workspace(g["Q"], w.d_proj, w.k, False, heads_per_chunk=1)
    one = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k, workspace=ws1)
    assert torch.equal(full, one)


def test_fused_forward_same_bits_per_chunk_size_and_stream():
    """The fused forward with the key-range gather (N > 8192) gives the same
    indices and outputs whether the heads go one at a time or all together,
    and when it runs on a side stream."""
    w = W.get("bf16_32k", N=8200, H=3, k=64)
    g = _cuda(W.make_inputs(w, 8))

    def fwd(ws=None):
        return sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k,
                                  workspace=ws, return_idx=True)

    ref_o, ref_i = fwd(sa.allocate_workspace(g["Q"], w.d_proj, w.k, False, heads_per_chunk=3))
    one_o, one_i = fwd(sa.allocate_workspace(g["Q"], w.d_proj, w.k, False, heads_per_chunk=1))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ws = sa.allocate_workspace(g["Q"], w.d_proj, w.k, False)
        s_o, s_i = fwd(ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(ref_i, one_i) and torch.equal(ref_o, one_o)
    assert torch.equal(ref_i, s_i) and torch.equal(ref_o, s_o)


# ------------------------------------------------- full-size workloads ---

def _ranges(N, causal):
    r = [(0, 8), (N // 3, 8), (N - 8, 8)]
    if causal:
        r.insert(1, (500, 24))              # rows around i = k: fewer than k valid keys
    return r


@pytest.mark.parametrize("dtype,D,causal,k", [("f32", 64, False, 64), ("bf16", 128, False, 64),
                                               ("bf16", 128, True, 64), ("bf16", 64, False, 512),
                                               ("bf16", 128, True, 512)])
def test_fused_forward_key_range_gather(dtype, D, causal, k):
    """Past N = 8192 the fused forward gathers by key range (partials per
    range, then a merge); ragged N, empty ranges and, causally, rows whose
    keys all fall in the first ranges.  With k = 512 a range holds enough of
    a row's keys for whole blocks of row loads, not only a last partial one."""
    w = W.get("bf16_32k", N=8200, H=2, D=D, dtype=dtype, d_proj=64 if D == 128 else 16,
              k=k, causal=causal)
    run_case(w, seed=5, rows=[(0, 300), (4000, 200), (8000, 200)])


@pytest.mark.parametrize("name", ["bf16_32k", "headline_128k", "causal_mixture"])
def test_full_size_workloads_sampled_rows(name):
    w = W.get(name)
    stats = run_case(w, rows=_ranges(w.N, w.causal))
    print(name, stats)
    assert stats["queries"] == w.queries
    assert stats["fallback_queries"] <= 0.01 * w.queries


def test_filter_dtype_does_not_change_indices():
    w = W.get("bf16_32k", N=6000, H=2, k=96)
    g = _cuda(W.make_inputs(w, 11))
    before = sa.sparse_attn_get_filter_dtype()
    try:
        sa.sparse_attn_set_filter_dtype(torch.float16)
        a = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k)
        sa.sparse_attn_set_filter_dtype(torch.bfloat16)
        b = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k)
    finally:
        sa.sparse_attn_set_filter_dtype(before)
    assert torch.equal(a, b)
