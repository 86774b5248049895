"""Backward (through the C ABI) against the fp64 oracle's backward
(page "mhpq.cn/news/1098205", §2.3: hard top-k forward, gradients through
the kept positions only, the scorer reached through the kept positions'
attention weights).  Every gradient is fp32; the bound is fp32 accumulation
over the entries that feed one output: |err| <= 1e-5 * max(1, max|ref|) for
dQ, dK, dV and 1e-4 * max|ref| for dPq, dPk, which sum over every row of
every head."""
import numpy as np
import pytest
import torch

import dynamic_top_sparse_amd as sa
import oracle as O
from dynamic_top_sparse_amd import workloads as W

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _close(got, want, rel, name):
    scale = max(1.0, float(np.abs(want).max()))
    err = float(np.abs(got.astype(np.float64) - want).max())
    assert err <= rel * scale, (name, err, scale)
    return err / scale


@pytest.mark.parametrize("N,k,D,dp,dtype,causal", [
    (1500, 32, 64, 16, "f32", False),
    (1200, 48, 128, 64, "bf16", True),
    (900, 900, 64, 32, "bf16", False),       # every key kept: dense attention's gradient
    (2000, 7, 128, 128, "f32", True),
    (8500, 40, 64, 16, "f32", True),
    (1501, 33, 128, 32, "bf16", True),       # ragged: N and k not multiples of the tiles
])
def test_backward_matches_oracle(N, k, D, dp, dtype, causal):
    w = W.Workload("bwd", 1, 2, N, D, dtype, d_proj=dp, k=k, causal=causal)
    x = W.make_inputs(w, N + k)
    gen = torch.Generator().manual_seed(N)
    dO = torch.randn(1, 2, N, D, generator=gen, dtype=torch.float32).to(w.torch_dtype)
    g = {n: t.cuda() for n, t in x.items()}
    idx = sa.sparse_attn_scores_topk(g["Q"], g["K"], g["Pq"], g["Pk"], k, causal)
    sscale, ascale = sa.default_score_scale(dp), sa.default_softmax_scale(D)
    want = O.sparse_attn_backward(x["Q"], x["K"], x["V"], x["Pq"], x["Pk"], _np(idx), dO,
                                  sscale, ascale, scorer_grad=True)
    want0 = O.sparse_attn_backward(x["Q"], x["K"], x["V"], x["Pq"], x["Pk"], _np(idx), dO,
                                   sscale, ascale, scorer_grad=False)
    for parts in ("whole", "split"):      # one wave per row / key, or key-range parts
        got = sa.sparse_attn_bwd(g["Q"], g["K"], g["V"], dO.cuda(), idx, g["Pq"], g["Pk"],
                                 parts=parts)
        for name, a, b in zip(("dQ", "dK", "dV"), got[:3], want[:3]):
            _close(_np(a), b, 1e-5, (parts, name))
        for name, a, b in zip(("dPq", "dPk"), got[3:], want[3:]):
            _close(_np(a), b, 1e-4, (parts, name))
        # the attention path alone
        att = sa.sparse_attn_bwd(g["Q"], g["K"], g["V"], dO.cuda(), idx, scorer_grad=False,
                                 parts=parts)
        for name, a, b in zip(("dQ", "dK", "dV"), att, want0[:3]):
            _close(_np(a), b, 1e-5, (parts, name))


def test_backward_list_semantics():
    """-1 entries skipped, repeats counted twice, rows without entries give
    nothing, keys no row kept get zero."""
    B, H, N, D, k = 1, 2, 600, 64, 12
    gen = torch.Generator().manual_seed(1)
    Q, K, V, dO = (torch.randn(B, H, N, D, generator=gen, dtype=torch.float32) for _ in range(4))
    idx = torch.randint(-1, N // 2, (B, H, N, k), generator=gen, dtype=torch.int32)
    idx[0, 0, 5] = -1
    idx[0, 1, 7, :4] = 3
    got = sa.sparse_attn_bwd(Q.cuda(), K.cuda(), V.cuda(), dO.cuda(), idx.cuda(),
                             scorer_grad=False)
    want = O.sparse_attn_backward(Q, K, V, np.zeros((D, 16)), np.zeros((D, 16)), idx.numpy(),
                                  dO, 1.0, D ** -0.5, scorer_grad=False)
    for name, a, b in zip(("dQ", "dK", "dV"), got, want[:3]):
        _close(_np(a), b, 1e-5, name)
    assert torch.all(got[0][0, 0, 5] == 0)
    assert torch.all(got[1][:, :, N // 2:] == 0) and torch.all(got[2][:, :, N // 2:] == 0)
    assert sa.sparse_attn_check_status() == 0


def test_backward_full_size_bf16_32k_sampled():
    """The bf16 32K workload (32 heads, N = 32768, k = 256) through the fused
    forward's index sets: per head, the dV rows sum to the dO rows (softmax
    weights sum to one); sampled dQ rows and sampled keys' dK, dV rows
    against the oracle, which gathers the rows that kept each sampled key."""
    w = W.get("bf16_32k")
    x = W.make_inputs(w, 0)
    gen = torch.Generator().manual_seed(2)
    dO = torch.randn(w.B, w.H, w.N, w.D, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    g = {n: t.cuda() for n, t in x.items()}
    _, idx = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, return_idx=True)
    dQ, dK, dV = sa.sparse_attn_bwd(g["Q"], g["K"], g["V"], dO.cuda(), idx, scorer_grad=False)
    # the key-range parts give the same gradients up to fp32 rounding
    sQ, sK, sV = sa.sparse_attn_bwd(g["Q"], g["K"], g["V"], dO.cuda(), idx, scorer_grad=False,
                                    parts="split")
    for name, a, b in (("dQ", sQ, dQ), ("dK", sK, dK), ("dV", sV, dV)):
        _close(_np(a), _np(b).astype(np.float64), 1e-5, ("split", name))
    torch.cuda.synchronize()
    dVs = _np(dV.double().sum(dim=2))
    dOs = dO.double().sum(dim=2).numpy()
    assert np.abs(dVs - dOs).max() <= 1e-5 * w.N, np.abs(dVs - dOs).max()
    ascale = w.D ** -0.5
    rng = np.random.default_rng(0)
    for h in (0, w.H - 1):
        Qh, Kh, Vh, dOh = (O.f64(t[0, h]) for t in (x["Q"], x["K"], x["V"], dO))
        idx_h = _np(idx[0, h]).astype(np.int64)
        for i in rng.choice(w.N, 16, replace=False):
            dq, _, _, _ = O.attend_row_backward(Qh[i], Kh, Vh, idx_h[i], ascale, dOh[i])
            _close(_np(dQ[0, h, i]), dq, 1e-5, "dQ")
        for j in rng.choice(w.N, 4, replace=False):
            rows, ts = np.nonzero(idx_h == j)
            dk = np.zeros(w.D)
            dv = np.zeros(w.D)
            for i, t in zip(rows, ts):
                _, dKr, dVr, _ = O.attend_row_backward(Qh[i], Kh, Vh, idx_h[i], ascale, dOh[i])
                dk += dKr[t]
                dv += dVr[t]
            _close(_np(dK[0, h, j]), dk, 1e-5, "dK")
            _close(_np(dV[0, h, j]), dv, 1e-5, "dV")


@pytest.mark.parametrize("N,k,H", [(8200, 1024, 1), (3000, 64, 2)])
def test_backward_split_path_list_semantics(N, k, H):
    """The passes in key-range parts: rows whose valid entries are an
    ascending prefix are cut into segments, other rows are scanned whole by
    every part; the key pass takes its parts from groups of row slices.
    Mixed rows: sorted ones, reversed ones, -1 entries in the middle,
    repeats; every element against the oracle."""
    B, D = 1, 64
    gen = torch.Generator().manual_seed(N + k)
    Q, K, V, dO = (torch.randn(B, H, N, D, generator=gen, dtype=torch.float32) for _ in range(4))
    idx = torch.randint(0, N, (B, H, N, k), generator=gen, dtype=torch.int32)
    idx, _ = torch.sort(idx, dim=-1)                       # ascending rows with repeats
    idx[0, 0, 1::3] = idx[0, 0, 1::3].flip(-1)              # every third row descending
    idx[0, H - 1, 5::7, k // 2] = -1                        # -1 inside a row
    idx[0, H - 1, 2::5, k - 3:] = -1                        # valid prefix, then -1
    idx[0, 0, 11] = -1                                      # a row with no valid entry
    got = sa.sparse_attn_bwd(Q.cuda(), K.cuda(), V.cuda(), dO.cuda(), idx.cuda(),
                             scorer_grad=False, parts="split")
    want = O.sparse_attn_backward(Q, K, V, np.zeros((D, 16)), np.zeros((D, 16)), idx.numpy(),
                                  dO, 1.0, D ** -0.5, scorer_grad=False)
    for name, a, b in zip(("dQ", "dK", "dV"), got, want[:3]):
        _close(_np(a), b, 1e-5, name)
    assert torch.all(got[0][0, 0, 11] == 0)
    assert sa.sparse_attn_check_status() == 0



@pytest.mark.parametrize("N,D,k", [(65600, 128, 16), (131200, 64, 8)])
def test_backward_two_launch_key_pass_every_element(N, D, k):
    """A head of more than 2^23 row elements (N = 65600 at D = 128, N =
    131200 at D = 64) takes the key pass in two launches, dV from the dO
    rows, then H from the Q rows; sorted rows, descending rows, -1 inside and
    at the end of rows, every element against the oracle."""
    B, H = 1, 1
    gen = torch.Generator().manual_seed(N + D)
    Q, K, V, dO = (torch.randn(B, H, N, D, generator=gen, dtype=torch.float32) for _ in range(4))
    idx = torch.randint(0, N, (B, H, N, k), generator=gen, dtype=torch.int32)
    idx, _ = torch.sort(idx, dim=-1)
    idx[0, 0, 1::5] = idx[0, 0, 1::5].flip(-1)
    idx[0, 0, 3::7, k // 2] = -1
    idx[0, 0, 2::9, k - 2:] = -1
    got = sa.sparse_attn_bwd(Q.cuda(), K.cuda(), V.cuda(), dO.cuda(), idx.cuda(),
                             scorer_grad=False)
    want = O.sparse_attn_backward(Q, K, V, np.zeros((D, 16)), np.zeros((D, 16)), idx.numpy(),
                                  dO, 1.0, D ** -0.5, scorer_grad=False)
    for name, a, b in zip(("dQ", "dK", "dV"), got, want[:3]):
        _close(_np(a), b, 1e-5, name)
    assert sa.sparse_attn_check_status() == 0


def test_backward_full_size_headline_128k_sampled():
    """The 128K headline sizes (32 heads, N = 131072, D = 128, k = 512, bf16)
    through the fused forward's index sets, in the launch setup the benchmark
    times (key-range parts, the key pass in two launches): every element
    against the whole-row passes (one wave per query and per key, no parts);
    per head, the dV rows sum to the dO rows; sampled dQ rows and sampled
    keys' dK, dV rows of two heads against the oracle."""
    w = W.get("headline_128k")
    x = W.make_inputs(w, 0)
    gen = torch.Generator().manual_seed(3)
    dO = torch.randn(w.B, w.H, w.N, w.D, generator=gen, dtype=torch.float32).to(torch.bfloat16)
    g = {n: t.cuda() for n, t in x.items()}
    gdO = dO.cuda()
    _, idx = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, return_idx=True)
    dQ, dK, dV = sa.sparse_attn_bwd(g["Q"], g["K"], g["V"], gdO, idx, scorer_grad=False)
    print("parts backward done", flush=True)
    whole = sa.sparse_attn_bwd(g["Q"], g["K"], g["V"], gdO, idx, scorer_grad=False,
                               parts="whole")
    for name, a, b in (("dQ", dQ, whole[0]), ("dK", dK, whole[1]), ("dV", dV, whole[2])):
        err = (a - b).abs().max().item()
        ref = max(1.0, b.abs().max().item())
        assert err <= 1e-5 * ref, ("whole", name, err, ref)
    del whole
    torch.cuda.synchronize()
    dVs = dV.double().sum(dim=2).cpu().numpy()
    dOs = dO.double().sum(dim=2).numpy()
    assert np.abs(dVs - dOs).max() <= 1e-5 * w.N, np.abs(dVs - dOs).max()
    ascale = w.D ** -0.5
    rng = np.random.default_rng(1)
    for h in (0, w.H - 1):
        Qh, Kh, Vh, dOh = (O.f64(t[0, h]) for t in (x["Q"], x["K"], x["V"], dO))
        idx_h = _np(idx[0, h]).astype(np.int64)
        for i in rng.choice(w.N, 16, replace=False):
            dq, _, _, _ = O.attend_row_backward(Qh[i], Kh, Vh, idx_h[i], ascale, dOh[i])
            _close(_np(dQ[0, h, i]), dq, 1e-5, "dQ")
        for j in rng.choice(w.N, 3, replace=False):
            rows, ts = np.nonzero(idx_h == j)
            dk = np.zeros(w.D)
            dv = np.zeros(w.D)
            for i, t in zip(rows, ts):
                _, dKr, dVr, _ = O.attend_row_backward(Qh[i], Kh, Vh, idx_h[i], ascale, dOh[i])
                dk += dKr[t]
                dv += dVr[t]
            _close(_np(dK[0, h, j]), dk, 1e-5, "dK")
            _close(_np(dV[0, h, j]), dv, 1e-5, "dV")
        print(f"head {h}: sampled rows and keys match the oracle", flush=True)
    assert sa.sparse_attn_check_status() == 0
