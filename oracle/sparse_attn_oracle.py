"""fp64 CPU oracle for dynamic top-k sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code with the HIP library.

The oracle is the plain definition of what the method computes, written in
float64 with NumPy, one step per statement, following the pages:

  1. Scorer (page "mhpq.cn/news/1098205", §2.2, LightweightScorer): each
     head's queries and keys are projected to a low dimension d_proj,
     q_low = Q·Pq and k_low = K·Pk, and every query-key pair is scored with a
     scaled dot product, S_ij = score_scale · q_low_i · k_low_j
     (score_scale defaults to d_proj^-1/2, as in that section).
  2. Selection (same page, §1.3 two-step allocation and §3.2 torch.topk):
     each query keeps the k highest-scoring keys.  Keys excluded by a mask
     (j > i when causal) are removed before selection (§3.2, third
     implementation note).  With fewer than k valid keys the query keeps all
     of them (§3.2, second implementation note: fall back to full
     attention).  Ties go to the lower key index.  A row is written in
     ascending key order and padded with -1.
  3. Attention over the kept keys (same page §1.2 formula and §3.2 forward;
     page "Attention机制优化：原理、挑战与工程实践", §1.1 scaled dot-product
     steps): logits softmax_scale · q·k_j, a max-subtracted softmax, and the
     weighted sum of the kept V rows.  softmax_scale defaults to D^-1/2.
  4. Band mode (page "Attention机制改进：稀疏注意力应用", create_local_mask;
     page "nxmr.cn/news/163144", §2.2): query i keeps keys
     max(0, i-w_left) .. min(N-1, i+w_right).

  6. Index variants feeding the same attention:
     - boundary smoothing (page "mhpq.cn/news/1098205", §4.2): when the gap
       between the k-th and (k+1)-th scores is below a threshold, both are
       kept, so a row holds k or k+1 keys;
     - dilated window with wrap-around (page "Attention机制优化：原理、挑战与
       工程实践", §3.3): query i keeps (i + t·dilation) mod N for
       t = 0 .. window-1, repeats included;
     - a window radius per batch sample (page "nxmr.cn/news/163144", §6,
       adaptive attention: each sample gets its own window size w).
  8. Block-granular selection (the SSA page's _block_sparsify works on
     blocks of the mask; page "mhpq.cn/news/1098205", §2.1 block-sparse
     attention computes only some block pairs).  Reading taken here: keys
     are cut into blocks of `block` consecutive rows, each block is scored
     as a whole with its mean k_low (so its score is the mean of its keys'
     scores), each query keeps its kb best blocks and attends to every
     valid key in them.  Causally a query always keeps its own block (the
     keys up to itself) and picks kb-1 more among the blocks wholly before
     it.
  7. Decode (page "mhpq.cn/news/1098205", §3.4, inference over the KV
     cache): one new query against the cached keys; with the cache holding
     keys 0..n-1 this is the causal forward's row n-1.
  5. Backward (same page, §2.3, top-k selection and gradient flow): the
     forward keeps the hard top-k; in the backward the selected positions'
     gradients flow normally and unselected positions get zero; the scorer
     receives its gradient through the selected positions' attention
     weights.  Reading taken here (a straight-through estimator): the
     scorer score S_ij of a selected pair receives the gradient of that
     pair's attention logit, dS_ij = dlogit_ij, and unselected pairs receive
     nothing; from there the chain rule runs through S = score_scale ·
     (Q·Pq)·(K·Pk)ᵀ to Pq, Pk, Q and K.

Every function below is pinned by tests against things other than itself
(brute force, closed forms, dense attention, a hand-derived example, torch
autograd and finite differences for the backward); see
tests/test_oracle_pins.py and tests/test_oracle_backward.py.  Nothing here
is "parity unpinned".
"""
from __future__ import annotations

import itertools
import math
from typing import Iterable, Optional, Sequence

import numpy as np


# ---------------------------------------------------------------- inputs ---

def f64(x) -> np.ndarray:
    """Exact upcast of a stored tensor (numpy or torch, fp32 or bf16) to fp64."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    try:  # torch tensor: bf16 -> fp32 is exact, fp32 -> fp64 is exact
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float32).numpy().astype(np.float64)
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------- 1. scorer ---

def project(X: np.ndarray, P: np.ndarray) -> np.ndarray:
    """Low-dimensional projection X·P for X [..., D], P [D, d_proj]
    (page "mhpq.cn/news/1098205", §2.2: q_proj / k_proj to d_proj)."""
    return np.matmul(X, P)


def valid_keys(N: int, i: int, causal: bool) -> np.ndarray:
    """Boolean mask of the keys query i may select: all N, or j <= i when
    causal (masked keys are excluded before selection, §3.2 of the same page)."""
    m = np.ones(N, dtype=bool)
    if causal:
        m[i + 1:] = False
    return m


def score_rows(q_low: np.ndarray, k_low: np.ndarray, score_scale: float) -> np.ndarray:
    """S[r, j] = score_scale · q_low[r] · k_low[j] for the given query rows
    (one head): q_low [R, d_proj], k_low [N, d_proj] -> [R, N]."""
    return score_scale * np.matmul(q_low, k_low.T)


def scores(Q, K, Pq, Pk, score_scale: float, b: int, h: int,
           rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """fp64 scores of head (b, h) for the requested query rows (all rows if
    None) against every key: [R, N].  Masking is not applied here."""
    Qh = f64(Q[b, h])
    Kh = f64(K[b, h])
    q_low = project(Qh if rows is None else Qh[np.asarray(rows)], f64(Pq))
    k_low = project(Kh, f64(Pk))
    return score_rows(q_low, k_low, score_scale)


# -------------------------------------------------------- 2. selection ---

def topk_row(s: np.ndarray, valid: np.ndarray, k: int) -> np.ndarray:
    """Top-k of one score row by (score descending, key index ascending),
    over valid keys only; returned in ascending key order, padded with -1
    up to k entries."""
    cand = np.nonzero(valid)[0]
    keep = min(k, cand.size)
    # np.lexsort sorts by the last key first: -score ascending (score
    # descending), then key index ascending for equal scores.
    order = np.lexsort((cand, -s[cand]))
    chosen = np.sort(cand[order[:keep]])
    out = np.full(k, -1, dtype=np.int32)
    out[:keep] = chosen
    return out


def topk_rows(S: np.ndarray, rows: Sequence[int], k: int, causal: bool) -> np.ndarray:
    """Apply topk_row to score rows S [R, N] of query rows ``rows``."""
    N = S.shape[1]
    return np.stack([topk_row(S[r], valid_keys(N, int(i), causal), k)
                     for r, i in enumerate(rows)])


def topk_indices(Q, K, Pq, Pk, k: int, causal: bool, score_scale: float,
                 rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """idx [B, H, R, k] (R = N when rows is None) of the full method's
    selection, computed from fp64 scores."""
    B, H, N = Q.shape[0], Q.shape[1], Q.shape[2]
    rows = list(range(N)) if rows is None else [int(r) for r in rows]
    out = np.empty((B, H, len(rows), k), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            S = scores(Q, K, Pq, Pk, score_scale, b, h, rows)
            out[b, h] = topk_rows(S, rows, k, causal)
    return out


def brute_force_topk(s: Sequence[float], valid: Sequence[bool], k: int) -> list:
    """Pure-Python enumeration for tiny rows: the unique subset of
    min(k, #valid) valid keys in which every member beats every non-member,
    where a beats b iff s_a > s_b, or s_a == s_b and a < b."""
    keys = [j for j, ok in enumerate(valid) if ok]
    size = min(k, len(keys))

    def beats(a, b):
        return s[a] > s[b] or (s[a] == s[b] and a < b)

    found = []
    for subset in itertools.combinations(keys, size):
        inside = set(subset)
        if all(beats(a, b) for a in subset for b in keys if b not in inside):
            found.append(sorted(subset))
    assert len(found) == 1, "the order is total, so exactly one subset qualifies"
    return found[0]


# ------------------------------------------------ 3. attention on a set ---

def attend_row(q: np.ndarray, Kh: np.ndarray, Vh: np.ndarray, sel: np.ndarray,
               softmax_scale: float) -> np.ndarray:
    """One query's output over the key list ``sel`` (entries < 0 skipped,
    repeated entries counted as often as they appear): logits, a
    max-subtracted softmax, weighted sum of V rows.  No valid entry -> 0."""
    sel = sel[sel >= 0]
    if sel.size == 0:
        return np.zeros(Vh.shape[1])
    logits = softmax_scale * (Kh[sel] @ q)
    w = np.exp(logits - logits.max())
    return (w @ Vh[sel]) / w.sum()


def gather_attention(Q, K, V, idx, softmax_scale: float,
                     rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """O [B, H, R, D]: attention of each query row over its idx row.
    ``idx`` is [B, H, R, k] for the given rows (all rows when None)."""
    Qa, Ka, Va = f64(Q), f64(K), f64(V)
    idx = np.asarray(idx)
    B, H, N, D = Qa.shape
    rows = list(range(N)) if rows is None else [int(r) for r in rows]
    O = np.zeros((B, H, len(rows), D))
    for b in range(B):
        for h in range(H):
            for r, i in enumerate(rows):
                O[b, h, r] = attend_row(Qa[b, h, i], Ka[b, h], Va[b, h],
                                        idx[b, h, r].astype(np.int64), softmax_scale)
    return O


def sparse_attn_fwd(Q, K, V, Pq, Pk, k: int, causal: bool, score_scale: float,
                    softmax_scale: float, rows: Optional[Sequence[int]] = None):
    """The whole forward: selection then attention.  Returns (idx, O)."""
    idx = topk_indices(Q, K, Pq, Pk, k, causal, score_scale, rows)
    O = gather_attention(Q, K, V, idx, softmax_scale, rows)
    return idx, O


# ------------------------------------------------------- 4. band mode ---

def band_indices(N: int, w_left: int, w_right: int, width: int) -> np.ndarray:
    """idx [N, width]: keys max(0, i-w_left) .. min(N-1, i+w_right) in
    ascending order, then -1 padding."""
    out = np.full((N, width), -1, dtype=np.int32)
    for i in range(N):
        lo, hi = max(0, i - w_left), min(N - 1, i + w_right)
        keys = np.arange(lo, hi + 1)[:width]
        out[i, :keys.size] = keys
    return out


# ------------------------------------------------------------ 7. decode ---

def decode_step(q, Kc, Vc, Pq, Pk, k: int, length: int, score_scale: float,
                softmax_scale: float):
    """One decode step of one head (page "mhpq.cn/news/1098205", §3.4): the
    new query q [D] scores the cached keys Kc[0:length] with the scorer,
    keeps its top-k (ties to the lower index, ascending, -1 padded) and
    attends over them.  Returns (idx [k], o [D])."""
    qa = f64(q)
    Ka, Va = f64(Kc)[:length], f64(Vc)[:length]
    s = score_rows(project(qa[None, :], f64(Pq)), project(Ka, f64(Pk)), score_scale)[0]
    idx = topk_row(s, np.ones(length, dtype=bool), k)
    return idx, attend_row(qa, Ka, Va, idx.astype(np.int64), softmax_scale)


# ------------------------------------------- 8. block-granular selection ---

def block_means(k_low: np.ndarray, block: int) -> np.ndarray:
    """Mean of each block of `block` consecutive rows of k_low [N, d_proj]
    (the last block may be shorter): [ceil(N / block), d_proj]."""
    N = k_low.shape[0]
    nb = (N + block - 1) // block
    return np.stack([k_low[J * block:min(N, (J + 1) * block)].mean(axis=0) for J in range(nb)])


def block_select_row(sb: np.ndarray, i: int, block: int, kb: int, causal: bool) -> np.ndarray:
    """Blocks kept by query i from its block scores sb [n_blocks]: the kb
    best by (score descending, block ascending); causally its own block plus
    the kb-1 best among the blocks that end before it.  Ascending."""
    nb = sb.shape[0]
    if causal:
        own = i // block
        cand = np.arange(own)
        take = min(kb - 1, cand.size)
        order = cand[np.lexsort((cand, -sb[cand]))]
        return np.sort(np.concatenate([order[:take], [own]])).astype(np.int64)
    cand = np.arange(nb)
    order = cand[np.lexsort((cand, -sb[cand]))]
    return np.sort(order[:min(kb, nb)]).astype(np.int64)


def block_keys_row(blocks: np.ndarray, i: int, N: int, block: int, width: int,
                   causal: bool) -> np.ndarray:
    """The keys of the kept blocks (causally only j <= i), ascending, -1
    padded to `width` entries."""
    keys = [j for J in blocks for j in range(J * block, min(N, (J + 1) * block))
            if not causal or j <= i]
    out = np.full(width, -1, dtype=np.int32)
    out[:len(keys)] = keys
    return out


def block_topk_indices(Q, K, Pq, Pk, block: int, kb: int, causal: bool, score_scale: float,
                       rows: Optional[Sequence[int]] = None, block_scores=None) -> np.ndarray:
    """idx [B, H, R, kb*block] of block-granular selection.  block_scores,
    when given, is a callable (b, h) -> [R, n_blocks] used instead of the
    fp64 block scores (to recompute the selection from other values)."""
    B, H, N = Q.shape[0], Q.shape[1], Q.shape[2]
    rows = list(range(N)) if rows is None else [int(r) for r in rows]
    out = np.empty((B, H, len(rows), kb * block), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            if block_scores is None:
                q_low = project(f64(Q[b, h])[np.asarray(rows)], f64(Pq))
                kbar = block_means(project(f64(K[b, h]), f64(Pk)), block)
                SB = score_rows(q_low, kbar, score_scale)
            else:
                SB = block_scores(b, h)
            for r, i in enumerate(rows):
                kept = block_select_row(SB[r], i, block, kb, causal)
                out[b, h, r] = block_keys_row(kept, i, N, block, kb * block, causal)
    return out


# -------------------------------------------------- 6. index variants ---

def smoothed_topk_row(s: np.ndarray, valid: np.ndarray, k: int, gap: float) -> np.ndarray:
    """Boundary smoothing of one row (page "mhpq.cn/news/1098205", §4.2):
    order the valid keys by (score descending, index ascending); keep the
    first k, and also the (k+1)-th when score_k - score_(k+1) < gap.  Output
    in ascending key order, padded with -1 to k + 1 entries."""
    cand = np.nonzero(valid)[0]
    order = cand[np.lexsort((cand, -s[cand]))]
    keep = min(k, order.size)
    if order.size > k and (s[order[k - 1]] - s[order[k]]) < gap:
        keep = k + 1
    out = np.full(k + 1, -1, dtype=np.int32)
    out[:keep] = np.sort(order[:keep])
    return out


def smoothed_topk_rows(S: np.ndarray, rows: Sequence[int], k: int, causal: bool,
                       gap: float) -> np.ndarray:
    """smoothed_topk_row over score rows S [R, N] of query rows ``rows``."""
    N = S.shape[1]
    return np.stack([smoothed_topk_row(S[r], valid_keys(N, int(i), causal), k, gap)
                     for r, i in enumerate(rows)])


def dilated_indices(N: int, window: int, dilation: int, width: int) -> np.ndarray:
    """idx [N, width]: row i holds (i + t*dilation) mod N for t = 0 ..
    window-1 (in t order, repeats kept), then -1 padding (page
    "Attention机制优化：原理、挑战与工程实践", §3.3 sliding window with
    dilation, wrapped modulo the sequence length)."""
    out = np.full((N, width), -1, dtype=np.int32)
    for i in range(N):
        for t in range(min(window, width)):
            out[i, t] = (i + t * dilation) % N
    return out


def band_indices_per_batch(B: int, H: int, N: int, radii: Sequence[int], width: int) -> np.ndarray:
    """idx [B, H, N, width]: band_indices with radius radii[b] for every head
    of batch sample b (page "nxmr.cn/news/163144", §6: one window size per
    sample)."""
    out = np.empty((B, H, N, width), dtype=np.int32)
    for b in range(B):
        rows = band_indices(N, int(radii[b]), int(radii[b]), width)
        for h in range(H):
            out[b, h] = rows
    return out


# --------------------------------- independent dense references (pins) ---

def dense_attention(Q, K, V, softmax_scale: float, mask: Optional[np.ndarray] = None,
                    causal: bool = False) -> np.ndarray:
    """Full softmax(Q·Kᵀ·scale [masked]) · V in fp64 over [B,H,N,D]: the
    standard scaled dot-product attention of page "mhpq.cn/news/1098205"
    §1.2 and page "Attention机制优化：原理、挑战与工程实践" §1.1, with the
    -inf masking of page "Attention机制改进：稀疏注意力应用" (mask [N,N],
    True = allowed).  Written without any index list."""
    Qa, Ka, Va = f64(Q), f64(K), f64(V)
    N = Qa.shape[2]
    logits = np.matmul(Qa, np.swapaxes(Ka, -1, -2)) * softmax_scale
    allowed = np.ones((N, N), dtype=bool) if mask is None else np.asarray(mask, bool)
    if causal:
        allowed = allowed & np.tril(np.ones((N, N), dtype=bool))
    logits = np.where(allowed, logits, -np.inf)
    mx = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - mx)
    p = e / e.sum(axis=-1, keepdims=True)
    return np.matmul(p, Va)


def local_mask(N: int, w: int) -> np.ndarray:
    """Band mask: key j allowed for query i iff i-w <= j <= i+w."""
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    return (j >= i - w) & (j <= i + w)


def brute_force_attention(q: Sequence[float], Krows: Iterable[Sequence[float]],
                          Vrows: Iterable[Sequence[float]], softmax_scale: float) -> list:
    """Direct summation in pure Python floats (tiny inputs only)."""
    Krows, Vrows = list(Krows), list(Vrows)
    logits = [softmax_scale * sum(a * b for a, b in zip(q, kr)) for kr in Krows]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    tot = sum(w)
    D = len(Vrows[0])
    return [sum(w[t] * Vrows[t][d] for t in range(len(w))) / tot for d in range(D)]


# -------------------------------------------------------- 5. backward ---

def attend_row_backward(q, Kh, Vh, sel, softmax_scale, dO_row):
    """Gradients of one query's output over the key list ``sel`` (entries < 0
    skipped, repeats counted as often as they appear), for an upstream
    gradient dO_row: returns (dq [D], dK_rows [k, D], dV_rows [k, D],
    dlogit [k]) with zero rows for skipped entries.  Softmax backward: with
    weights p_t and dp_t = dO·V_t, dlogit_t = p_t (dp_t - sum_u p_u dp_u)."""
    k = sel.shape[0]
    D = Kh.shape[1]
    dq = np.zeros(D)
    dK = np.zeros((k, D))
    dV = np.zeros((k, Vh.shape[1]))
    dlogit = np.zeros(k)
    ok = sel >= 0
    if not np.any(ok):
        return dq, dK, dV, dlogit
    js = sel[ok]
    logits = softmax_scale * (Kh[js] @ q)
    w = np.exp(logits - logits.max())
    p = w / w.sum()
    dp = Vh[js] @ dO_row
    dl = p * (dp - np.dot(p, dp))
    dlogit[ok] = dl
    dq = softmax_scale * (dl @ Kh[js])
    dK[ok] = softmax_scale * np.outer(dl, q)
    dV[ok] = np.outer(p, dO_row)
    return dq, dK, dV, dlogit


def sparse_attn_backward(Q, K, V, Pq, Pk, idx, dO, score_scale: float, softmax_scale: float,
                         scorer_grad: bool = True):
    """Backward of the whole forward for fixed index sets ``idx`` [B,H,N,k].

    Attention path: dQ, dK, dV of softmax attention over each row's kept
    keys; a key receives gradient only from the rows that kept it.
    Scorer path (scorer_grad, the straight-through reading of §2.3): the
    score of each kept pair (i, j) receives that pair's logit gradient,
    dS_ij = dlogit_ij, and with q_low = Q·Pq, k_low = K·Pk,
    S = score_scale · q_low·k_lowᵀ:
      dq_low_i = score_scale · sum_j dS_ij k_low_j,
      dk_low_j = score_scale · sum_i dS_ij q_low_i,
      dPq = sum over heads and rows of Qᵀ·dq_low, dPk likewise with K,
      and dQ += dq_low·Pqᵀ, dK += dk_low·Pkᵀ.
    Returns dQ, dK, dV [B,H,N,D] and dPq, dPk [D, d_proj] (zeros without
    the scorer path), all float64."""
    Qa, Ka, Va, dOa = f64(Q), f64(K), f64(V), f64(dO)
    Pqa, Pka = f64(Pq), f64(Pk)
    idx = np.asarray(idx).astype(np.int64)
    B, H, N, D = Qa.shape
    dQ = np.zeros_like(Qa)
    dK = np.zeros_like(Ka)
    dV = np.zeros_like(Va)
    dPq = np.zeros_like(Pqa)
    dPk = np.zeros_like(Pka)
    for b in range(B):
        for h in range(H):
            q_low = project(Qa[b, h], Pqa)
            k_low = project(Ka[b, h], Pka)
            dq_low = np.zeros_like(q_low)
            dk_low = np.zeros_like(k_low)
            for i in range(N):
                sel = idx[b, h, i]
                dq, dKr, dVr, dl = attend_row_backward(Qa[b, h, i], Ka[b, h], Va[b, h], sel,
                                                        softmax_scale, dOa[b, h, i])
                dQ[b, h, i] += dq
                for t, j in enumerate(sel):
                    if j < 0:
                        continue
                    dK[b, h, j] += dKr[t]
                    dV[b, h, j] += dVr[t]
                    if scorer_grad:
                        dq_low[i] += score_scale * dl[t] * k_low[j]
                        dk_low[j] += score_scale * dl[t] * q_low[i]
            if scorer_grad:
                dPq += Qa[b, h].T @ dq_low
                dPk += Ka[b, h].T @ dk_low
                dQ[b, h] += dq_low @ Pqa.T
                dK[b, h] += dk_low @ Pka.T
    return dQ, dK, dV, dPq, dPk
