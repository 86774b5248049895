"""Every row of several heads of the large workloads, at full size and in
the launch setup the benchmark times (all heads in one fused call).

For each checked head, in chunks of rows:
- idx equals, row by row, the top-k of the library's own dumped fp32 scores
  by (score descending, key ascending), masked keys excluded and every valid
  key kept when fewer than k are valid: that definition is evaluated here
  with plain torch ops on the GPU (the k-th largest value from torch.topk,
  then the keys above it and the lowest-index keys equal to it), so every
  row is covered, not a sample;
- each row lists its keys ascending, then -1 only;
- O equals fp32 attention over the row's keys, computed with torch
  (gathered rows, fp32 products, softmax, weighted sum).

The dumped scores are themselves checked against the fp64 oracle within the
rounding bound (test_gpu_parity), and sampled rows of the same calls against
the oracle's own top-k and attention."""
import pytest
import torch

import dynamic_top_sparse_amd as sa
from dynamic_top_sparse_amd import workloads as W
from topk_definition import actual_mask, check_row_form, expected_mask

pytestmark = pytest.mark.gpu

TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
CHUNK = 1024


def attention_rows(q, K, V, idx_rows, scale):
    """fp32 softmax(q·K_selᵀ·scale)·V_sel over each row's valid entries."""
    valid = idx_rows >= 0
    j = idx_rows.clamp(min=0).long()
    Ks = K[j]                                   # [R, k, D] fp32, contiguous
    Vs = V[j]
    logit = torch.bmm(Ks, q[:, :, None])[:, :, 0] * scale
    logit = logit.masked_fill(~valid, float("-inf"))
    p = torch.softmax(logit, dim=1)
    return torch.bmm(p[:, None, :], Vs)[:, 0, :]


# eight heads of each workload (a quarter of its heads), spread over b and h;
# and the headline once more with bf16 filter operands (the benchmark times
# that forward too), on four heads
CASES = {
    "bf16_32k": [(0, h) for h in (0, 4, 9, 13, 18, 22, 27, 31)],
    "headline_128k": [(0, h) for h in (0, 5, 7, 12, 19, 24, 26, 31)],
    "causal_mixture": [(0, 0), (0, 6), (1, 3), (1, 7), (2, 1), (2, 5), (3, 2), (3, 7)],
    "headline_128k/bf16 filter": [(0, h) for h in (2, 11, 20, 29)],
}


@pytest.mark.parametrize("name", list(CASES))
def test_every_row_of_sampled_heads(name):
    wname, _, variant = name.partition("/")
    fdt = torch.bfloat16 if variant == "bf16 filter" else None
    w = W.get(wname)
    x = W.make_inputs(w, 0)
    g = {n: t.cuda() for n, t in x.items()}
    ws = sa.allocate_workspace(g["Q"], w.d_proj, w.k, w.causal, with_idx=False,
                               heads_per_chunk=w.B * w.H)
    out, idx = sa.sparse_attn_fwd(g["Q"], g["K"], g["V"], g["Pq"], g["Pk"], w.k, w.causal,
                                  workspace=ws, return_idx=True, filter_dtype=fdt)
    st = sa.sparse_attn_workspace_stats(ws)
    assert st["margin_violations"] == 0, st
    torch.cuda.synchronize()
    del ws
    ascale = sa.default_softmax_scale(w.D)
    for (b, h) in CASES[name]:
        print(f"{name}: head ({b}, {h}), all {w.N} rows", flush=True)
        gq = g["Q"][b:b + 1, h:h + 1].contiguous()
        gk = g["K"][b:b + 1, h:h + 1].contiguous()
        dws = sa.allocate_workspace(gq, w.d_proj, 1, w.causal)
        Q32, K32, V32 = (g[n][b, h].float().contiguous() for n in ("Q", "K", "V"))
        S = torch.empty(1, 1, CHUNK, w.N, dtype=torch.float32, device="cuda")
        worst = 0.0
        for r0 in range(0, w.N, CHUNK):
            rc = min(CHUNK, w.N - r0)
            Sc = S[:, :, :rc] if rc == CHUNK else \
                torch.empty(1, 1, rc, w.N, dtype=torch.float32, device="cuda")
            sa.sparse_attn_scores_dump(gq, gk, g["Pq"], g["Pk"], r0, rc, w.causal, S=Sc,
                                       workspace=dws)
            rows = torch.arange(r0, r0 + rc, device="cuda")
            want, kk = expected_mask(Sc[0, 0], rows, w.k, w.causal)
            ir = idx[b, h, r0:r0 + rc]
            check_row_form(ir, kk)
            got = actual_mask(ir, w.N)
            if not torch.equal(got, want):
                bad = (got != want).any(1).nonzero()[:5, 0] + r0
                raise AssertionError(f"{name} head ({b}, {h}): idx differs at rows {bad.tolist()}")
            o_ref = attention_rows(Q32[r0:r0 + rc], K32, V32, ir, ascale)
            err = (out[b, h, r0:r0 + rc].float() - o_ref).abs().max().item()
            worst = max(worst, err)
        print(f"  idx exact on all rows; O max-abs error {worst:.3g}", flush=True)
        assert worst <= TOL[w.torch_dtype], (name, (b, h), worst)
