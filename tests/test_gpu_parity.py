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


def run_case(w: W.Workload, seed=0, rows=None, check_all=True, filter_dtype=None, x=None):
    x = W.make_inputs(w, seed) if x is None else x
    g = _cuda(x)
    B, H, N, D = w.B, w.H, w.N, w.D
    ws = sa.allocate_workspace(g["Q"], w.d_proj, w.k, w.causal, with_idx=False)
    idx = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k, w.causal,
                                     workspace=ws, filter_dtype=filter_dtype)
    out, idx2 = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, w.causal,
                                   return_idx=True, filter_dtype=filter_dtype)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "fused and split paths disagree"
    stats = sa.sparse_attn_workspace_stats(ws)
    # every exactly re-scored key lies in the interval the filter's margin
    # gives it: the no-miss argument's rounding bound holds on these inputs
    assert stats["margin_violations"] == 0, stats
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


@pytest.mark.parametrize("dtype,D", [(torch.float32, 64), (torch.float32, 128),
                                     (torch.bfloat16, 128), (torch.bfloat16, 64)])
def test_gather_by_key_range_mixed_rows(dtype, D):
    """sparse_attn_gather_ws just past the key-range threshold (N = 8200):
    rows of ascending keys with -1 tails, repeated keys, keys crowded into
    one range and an empty row take the key-range path; an unordered row, a
    -1 before a valid entry and an entry >= N go through the single pass (the
    entry >= N skipped and flagged).  Every row against the oracle, and the
    one-pass gather within the same bound."""
    B, H, N, k = 1, 2, 8200, 64
    gen = torch.Generator().manual_seed(D + 7)
    Q, K, V = (torch.randn(B, H, N, D, generator=gen).to(dtype) for _ in range(3))
    idx = torch.sort(torch.randint(0, N, (B, H, N, k), generator=gen, dtype=torch.int32),
                     dim=-1).values
    for i in range(0, N, 5):                    # -1 tails of 0 .. 16 entries
        t = i % 17
        if t:
            idx[:, :, i, k - t:] = -1
    idx[0, 0, 3] = -1                           # empty row
    idx[0, 1, 20] = torch.sort(torch.randint(0, 100, (k,), generator=gen,
                                             dtype=torch.int32)).values   # one range only
    idx[0, 0, 30, :5] = idx[0, 0, 30, 0]        # repeats, still ascending
    for i in (7, 100, 5000):                    # unordered
        idx[0, 0, i] = idx[0, 0, i].flip(0)
    idx[0, 1, 11, 10] = -1                      # a valid entry after a -1
    idx[0, 1, 13, k - 1] = N                    # out of range: skipped, flagged
    assert sa.sparse_attn_check_status() == 0
    g = {n: t.cuda() for n, t in (("Q", Q), ("K", K), ("V", V))}
    gi = idx.cuda()
    got = sa.sparse_attn_gather(g["Q"], g["K"], g["V"], gi, 0.2)
    assert sa.sparse_attn_check_status() == -7
    one = sa.sparse_attn_gather(g["Q"], g["K"], g["V"], gi, 0.2, by_range=False)
    assert sa.sparse_attn_check_status() == -7
    want = O.gather_attention(Q, K, V, np.where(idx.numpy() >= N, -1, idx.numpy()), 0.2)
    got_np = _rows_np(got.float())
    err = np.abs(got_np - want).max()
    assert err <= TOL[dtype], err
    assert np.abs(got_np - _rows_np(one.float())).max() <= TOL[dtype]
    assert torch.all(got[0, 0, 3] == 0)


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
    """Each 16-bit operand type of the MFMA filter (passed per call); the
    indices must not depend on it."""
    return request.param


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
    run_case(w, seed=N + k, filter_dtype=filter_dtype)


def test_largest_k_with_key_range_gather_all_rows():
    """k at its maximum (2048, lists of 2048 entries per half) past the
    threshold path's minimum N and the key-range gather's, d_proj 128."""
    w = W.Workload("case", 1, 1, 9000, 128, "bf16", d_proj=128, k=2048)
    run_case(w, seed=77)


@pytest.mark.parametrize("N,k,causal", [(1100, 512, False), (9000, 512, True), (20000, 640, False)])
def test_long_candidate_lists_ranked_from_memory_all_rows(N, k, causal):
    """With fp16 filter operands the re-rank's LDS room (1024 candidates at
    k = 512 and 640, so that four waves share a SIMD) is smaller than a
    query's two lists (640 or 832 entries each): queries with more candidates
    are ranked from their lists in memory.  N = 1100: every query keeps all
    its keys (1100 candidates); causal N = 9000: all-key rows on both sides of
    the room and threshold rows; N = 20000, k = 640: threshold rows, many
    above the room (three row ranges checked)."""
    w = W.Workload("case", 1, 2, N, 64, "bf16", d_proj=64, k=k, causal=causal)
    rows = [(0, 384), (9000, 384), (N - 384, 384)] if N > 10000 else None
    stats = run_case(w, seed=N + 3, rows=rows, filter_dtype=torch.float16)
    print(stats, flush=True)
    assert stats["wide_queries"] > 0, stats
    if N == 1100:
        assert stats["wide_queries"] == w.queries, stats


def test_mixture_causal_small_all_rows(filter_dtype):
    w = W.get("causal_mixture", B=2, H=2, N=6000, k=64)
    run_case(w, seed=5, filter_dtype=filter_dtype)


def test_exact_ties_go_to_lower_index(filter_dtype):
    """Duplicated key rows give bit-identical scores; the lower index wins."""
    w = W.Workload("ties", 1, 1, 3000, 64, "f32", d_proj=16, k=40)
    x = W.make_inputs(w, 9)
    K = x["K"].clone()
    K[0, 0, 2000:2600] = K[0, 0, 0:600]     # keys 2000.. repeat keys 0..
    x["K"] = K
    g = _cuda(x)
    idx = _rows_np(sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k,
                                              filter_dtype=filter_dtype))
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

def _sample_ranges(N, causal, k, seed, n_ranges=64, width=16):
    """Seeded random row ranges (n_ranges x width rows) plus the first and last
    rows and, causally, the rows around i = k where the valid-key count
    crosses k; overlapping ranges are trimmed so every row is checked once."""
    rng = np.random.default_rng(seed)
    starts = set(int(x) for x in rng.choice(N - width, n_ranges, replace=False))
    starts |= {0, N - width}
    if causal:
        starts.add(max(0, k - width // 2))
    out, last = [], -1
    for s0 in sorted(starts):
        a, b = max(s0, last + 1), min(s0 + width, N)
        if b > a:
            out.append((a, b - a))
            last = b - 1
    return out


def check_sampled_heads(w, x, idx, out, heads, ranges):
    """idx and O of the full-size call, on the given (b, h) heads and row
    ranges: bit-exact idx against the oracle's top-k of the dumped fp32
    scores, overlap against fp64 scores, O against the oracle's attention."""
    sscale = sa.default_score_scale(w.d_proj)
    ascale = sa.default_softmax_scale(w.D)
    for (b, h) in heads:
        sl = {n: x[n][b:b + 1, h:h + 1].contiguous() for n in ("Q", "K", "V")}
        gq, gk = sl["Q"].cuda(), sl["K"].cuda()
        gpq, gpk = x["Pq"].cuda(), x["Pk"].cuda()
        ws = sa.allocate_workspace(gq, w.d_proj, 1, w.causal)
        k_low = O.project(O.f64(sl["K"][0, 0]), O.f64(x["Pk"]))
        q_all = O.f64(sl["Q"][0, 0])
        idx_h = _rows_np(idx[b, h])
        out_h = _rows_np(out[b, h].float())
        print(f"checking head ({b}, {h}): {sum(c for _, c in ranges)} rows", flush=True)
        for (r0, rc) in ranges:
            rr = list(range(r0, r0 + rc))
            S = _rows_np(sa.sparse_attn_scores_dump(gq, gk, gpq, gpk, r0, rc, w.causal,
                                                    workspace=ws))[0, 0]
            S64 = O.score_rows(O.project(q_all[r0:r0 + rc], O.f64(x["Pq"])), k_low, sscale)
            if w.causal:
                S64 = np.where(np.arange(w.N)[None, :] <= np.asarray(rr)[:, None], S64, -np.inf)
            check_idx_rows(idx_h[r0:r0 + rc], S, S64, rr, w.k, w.causal, w.N)
            want = O.gather_attention(sl["Q"], sl["K"], sl["V"], idx_h[None, None, r0:r0 + rc],
                                      ascale, rr)[0, 0]
            err = np.abs(out_h[r0:r0 + rc] - want).max()
            assert err <= TOL[w.torch_dtype], (err, (b, h), r0)


@pytest.mark.parametrize("name", ["bf16_32k", "headline_128k", "causal_mixture"])
def test_full_size_workloads_sampled_rows(name):
    """The three large workloads at their full sizes, in the launch setup the
    benchmark times (all heads in one fused call): 1024+ seeded random rows
    on each of two heads, plus the edges and (causal) the rows near i = k."""
    w = W.get(name)
    x = W.make_inputs(w, 0)
    g = _cuda(x)
    ws = sa.allocate_workspace(g["Q"], w.d_proj, w.k, w.causal, with_idx=False,
                               heads_per_chunk=w.B * w.H)
    out, idx = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, w.causal,
                                  workspace=ws, return_idx=True)
    torch.cuda.synchronize()
    stats = sa.sparse_attn_workspace_stats(ws)
    print(name, stats, flush=True)
    assert stats["queries"] == w.queries
    assert stats["fallback_queries"] <= 0.01 * w.queries
    assert stats["margin_violations"] == 0, stats
    del g
    heads = [(0, 0), (w.B - 1, w.H - 1)]
    check_sampled_heads(w, x, idx, out, heads, _sample_ranges(w.N, w.causal, w.k, seed=17))


# ------------------------------------------ retry and fallback paths ---

def _tied_keys(w, seed, copies, all_same_head=None):
    """Inputs whose key rows repeat: in every head, `copies` positions hold the
    very same row (bit-identical scores for every query, so top lists of tied
    keys overflow), and head `all_same_head` has one row for all its keys."""
    x = W.make_inputs(w, seed)
    K = x["K"].clone()
    rng = np.random.default_rng(seed)
    for b in range(w.B):
        for h in range(w.H):
            if h == all_same_head:
                K[b, h] = K[b, h, 0].clone()
            else:
                pos = rng.choice(w.N, copies, replace=False)
                K[b, h, torch.as_tensor(pos)] = K[b, h, int(pos[0])].clone()
    x["K"] = K.contiguous()
    return x


@pytest.mark.parametrize("N,k,causal,dtype", [(3000, 64, False, "f32"), (3000, 64, True, "bf16"),
                                              (3000, 700, False, "bf16"), (2600, 900, True, "f32")])
def test_retry_and_fallback_paths_all_rows(N, k, causal, dtype, filter_dtype):
    """Repeated key rows make lists overflow on the first pass and again on
    the retry with a proven threshold, so the exact fallback resolves those
    queries (its radix select and its ordering of tied keys across threads),
    while other queries of the same call take the retry path.  Every row is
    checked: idx bit-exact against the oracle's top-k of the dumped scores
    (ties to the lower index), O against the oracle's attention; causally
    with rows below and above k valid keys."""
    w = W.Workload("ties", 1, 3, N, 64 if dtype == "f32" else 128, dtype,
                   d_proj=16 if dtype == "f32" else 64, k=k, causal=causal)
    x = _tied_keys(w, seed=N + k, copies=N // 3, all_same_head=2)
    stats = run_case(w, x=x, filter_dtype=filter_dtype)
    print(stats, flush=True)
    assert stats["fallback_queries"] > 0, stats
    assert stats["retried"] > 0, stats
    assert stats["queries"] == w.queries


# ------------------------------------------------ projection precision ---

def _score_error_bound(Q, K, Pq, Pk, scale, rows):
    """Elementwise bound on |S_library - S_exact| for fp32 projections and an
    fp32 score: each projection is a sum of D exact products (or fp32
    products) rounded in some order, so its error is at most
    gamma_D * sum_d |x_d P_dc| (gamma_n = n u / (1 - n u), u = 2^-24); the
    score adds the projections' errors times the other factor, and its own
    sum of d_proj products at most gamma_dp * sum_c |q_c k_c|."""
    u = 2.0 ** -24
    D, dp = Pq.shape

    def gam(n):
        return n * u / (1 - n * u)

    Qa, Ka = O.f64(Q)[rows], O.f64(K)
    Pqa, Pka = O.f64(Pq), O.f64(Pk)
    q, kk = Qa @ Pqa, Ka @ Pka
    Eq = gam(D + 1) * (np.abs(Qa) @ np.abs(Pqa))
    Ek = gam(D + 1) * (np.abs(Ka) @ np.abs(Pka))
    aq, ak = np.abs(q) + Eq, np.abs(kk) + Ek
    bound = Eq @ np.abs(kk).T + np.abs(q) @ Ek.T + Eq @ Ek.T + gam(dp + 1) * (aq @ ak.T)
    return scale * bound * (1 + 1e-6) + 1e-30


@pytest.mark.parametrize("dtype,D,dp", [("bf16", 128, 64), ("bf16", 64, 32), ("f32", 128, 128)])
def test_scores_dump_within_rounding_bound_of_fp64(dtype, D, dp):
    """The library's fp32 scores (bf16 rows on the MFMA projection, fp32 rows
    on FMAs) lie within the rounding bound of the exact fp64 scores, element
    by element; a projection or score rounded through a 16-bit type would
    miss it by orders of magnitude."""
    w = W.Workload("proj", 1, 2, 2500, D, dtype, d_proj=dp, k=8)
    x = W.make_inputs(w, 21)
    g = _cuda(x)
    scale = sa.default_score_scale(dp)
    S = _rows_np(sa.sparse_attn_scores_dump(g["Q"], g["K"], g["Pq"], g["Pk"], 0, w.N))
    rows = np.arange(w.N)
    worst = 0.0
    for h in range(w.H):
        S64 = O.scores(x["Q"], x["K"], x["Pq"], x["Pk"], scale, 0, h)
        bound = _score_error_bound(x["Q"][0, h], x["K"][0, h], x["Pq"], x["Pk"], scale, rows)
        err = np.abs(S[0, h].astype(np.float64) - S64)
        assert np.all(err <= bound), (float((err / bound).max()), h)
        worst = max(worst, float((err / bound).max()))
    print(f"largest error / bound: {worst:.3g}")


def test_filter_dtype_does_not_change_indices():
    w = W.get("bf16_32k", N=6000, H=2, k=96)
    g = _cuda(W.make_inputs(w, 11))
    a = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k,
                                   filter_dtype=torch.float16)
    b = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], w.k,
                                   filter_dtype=torch.bfloat16)
    assert torch.equal(a, b)
