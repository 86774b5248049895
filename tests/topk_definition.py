"""The top-k selection rule written with plain torch ops, for checking every
row of large GPU results on the GPU itself: keep the keys by (score
descending, key index ascending), masked keys (causally j > i) never kept,
every valid key kept when fewer than k are valid (page "mhpq.cn/news/1098205",
§3.2: top-k of the scores with masked positions excluded first).  The
functions work on any device; tests/test_topk_definition_cpu.py checks them
against the oracle's topk_rows."""
import torch


def expected_mask(S, rows, k, causal):
    """[R, N] bool: the keys the definition keeps for each row of S."""
    R, N = S.shape
    if causal:
        S = S.masked_fill(torch.arange(N, device=S.device)[None, :] > rows[:, None], float("-inf"))
    valid = S > float("-inf")
    n_valid = valid.sum(1)
    kk = torch.clamp(n_valid, max=k)
    kq = min(k, N)
    kth = torch.topk(S, kq, dim=1).values[:, kq - 1]          # k-th largest value per row
    greater = S > kth[:, None]
    eq = (S == kth[:, None]) & valid
    need = (kk - greater.sum(1))[:, None]                      # ties still to take
    take_eq = eq & (torch.cumsum(eq.to(torch.int32), 1, dtype=torch.int32) <= need)
    keep = (greater | take_eq) & valid
    # rows with fewer than k valid keys keep every valid key
    return torch.where((n_valid < k)[:, None], valid, keep), kk


def actual_mask(idx_rows, N):
    R, k = idx_rows.shape
    col = torch.where(idx_rows >= 0, idx_rows.long(), torch.full_like(idx_rows, N).long())
    m = torch.zeros(R, N + 1, dtype=torch.bool, device=idx_rows.device)
    m.scatter_(1, col, True)
    return m[:, :N]


def check_row_form(idx_rows, kk):
    """ascending keys, then -1 only, as many keys as the row keeps"""
    R, k = idx_rows.shape
    pos = torch.arange(k, device=idx_rows.device)[None, :]
    is_key = idx_rows >= 0
    assert torch.equal(is_key, pos < kk[:, None]), "keys not a prefix of the row"
    assert bool(((idx_rows == -1) | is_key).all())
    if k > 1:
        both = is_key[:, 1:] & is_key[:, :-1]
        assert bool(((idx_rows[:, 1:] > idx_rows[:, :-1]) | ~both).all()), "keys not ascending"
