/*
 * sparse_attn.h - C ABI of the MI355X (gfx950) dynamic top-k sparse
 * attention library, libsparse_attn.so.
 *
 * The method (page "mhpq.cn/news/1098205", §1.3 two-step allocation, §2.2
 * LightweightScorer, §3.2 DynamicSparseAttention forward):
 *   1. a lightweight scorer projects each head's queries and keys to d_proj
 *      dimensions, q_low = Q·Pq and k_low = K·Pk, and scores every pair as
 *      S_ij = score_scale · q_low_i · k_low_j;
 *   2. each query keeps its k highest-scoring keys;
 *   3. softmax(q·K_selᵀ · softmax_scale) · V_sel runs over those keys only.
 * A band (sliding window) is the same attention over a fixed index set
 * (page "Attention机制改进：稀疏注意力应用", create_local_mask; page
 * "nxmr.cn/news/163144", §2.2 local attention).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers on the current HIP device, 16-byte
 *   aligned.  Q, K, V, O are [B, H, N, D] contiguous (D fastest), the
 *   [batch, heads, seq_len, ·] layout of the pages' scorer.  Pq, Pk are
 *   [D, d_proj] row-major and shared by all heads: q_low = Q·Pq.
 *   idx is [B, H, N, k] int32.
 * - dtype: SA_F32 or SA_BF16; Q, K, V, Pq, Pk and O all share it (mixing
 *   precisions is an error, not a silent cast).  Arithmetic is fp32
 *   throughout (logits, softmax and accumulation: page
 *   "Attention机制优化：原理、挑战与工程实践", §4.2 keep fp32 before softmax);
 *   bf16 outputs are rounded to nearest even.
 * - Supported sizes: D in {64, 128}; d_proj in {16, 32, 64, 128};
 *   1 <= k <= SA_K_MAX; B, H, N >= 1 and N * k < 2^31.
 * - Ownership: the caller allocates and owns every buffer, including the
 *   workspace; the library allocates no device memory in these calls.
 * - Execution: asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream).  Arguments are validated on the host before anything is
 *   enqueued; on a negative return value nothing was enqueued.
 * - Calls that share a workspace must not overlap in time.
 * - The library keeps no mutable state between calls: everything a call
 *   depends on is in its arguments (the options below included), so calls
 *   from several host threads on different workspaces are independent.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_K_MAX 2048

typedef enum { SA_F32 = 0, SA_BF16 = 1, SA_F16 = 2 } sa_dtype;  /* SA_F16: filter only */

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = -1,         /* a required pointer is NULL                   */
  SA_ERR_SHAPE = -2,        /* B, H, N < 1, k < 1, N*k too large, row range  */
  SA_ERR_UNSUPPORTED = -3,  /* D, d_proj, dtype or k outside the supported set */
  SA_ERR_ALIGN = -4,        /* a pointer is not 16-byte aligned             */
  SA_ERR_WORKSPACE = -5,    /* workspace smaller than sparse_attn_workspace_size */
  SA_ERR_HIP = -6,          /* a HIP launch or query failed                 */
  SA_ERR_DEVICE_INDEX = -7  /* check_status: a kernel saw idx >= N          */
} sa_status;

/* Shape of Q, K, V, O: [B, H, N, D]. */
typedef struct { int32_t B, H, N, D; } sa_dims;

/*
 * Per-kernel timing record, owned by the caller (created and destroyed with
 * sparse_attn_profile_create / _destroy).  A call given one brackets each of
 * its kernel launches with a pair of HIP events on the launch stream; its
 * own mutex makes it safe to share between threads.
 */
typedef struct sa_profile sa_profile;

/*
 * Options of a compute call, read while the call runs and never kept.
 * Passing NULL is the same as { SA_F16, NULL, SA_BWD_PARTS_AUTO }.
 *   filter_dtype: operand type of the 16-bit MFMA filter inside
 *     sparse_attn_scores_topk and sparse_attn_fwd, SA_F16 or SA_BF16.  Rows
 *     are scaled by powers of two before rounding (one exponent per query
 *     row, one per key head), so either type covers the fp32 range.  The
 *     returned indices are the same for both: the filter only discards keys
 *     that provably cannot be in the top-k, and the final choice uses the
 *     exact fp32 score.  fp16 keeps 11 significant bits instead of 8, which
 *     shrinks the band of keys that must be re-scored exactly.
 *   profile: NULL, or a timing record that receives this call's launches.
 *   bwd_parts: how sparse_attn_bwd lays out its row and key passes.
 *     SA_BWD_PARTS_AUTO picks by size; SA_BWD_PARTS_WHOLE runs one wave per
 *     whole row and per whole key; SA_BWD_PARTS_SPLIT cuts both into eight
 *     key (row) ranges, one per XCD, and adds the parts.  The results agree
 *     to fp32 rounding; only the time and the workspace differ (the size
 *     query takes the same options).
 */
enum { SA_BWD_PARTS_AUTO = 0, SA_BWD_PARTS_WHOLE = 1, SA_BWD_PARTS_SPLIT = 2 };
typedef struct {
  int32_t filter_dtype;
  sa_profile* profile;
  int32_t bwd_parts;
} sa_options;

/*
 * Bytes of workspace that sparse_attn_scores_topk, sparse_attn_fwd and
 * sparse_attn_scores_dump need for these arguments (with_idx != 0 adds room
 * for the index rows sparse_attn_fwd keeps internally when the caller passes
 * no idx buffer).  The library works through the (b, h) heads in chunks; a
 * larger workspace than this minimum lets it use larger chunks (see
 * sparse_attn_workspace_size_for_chunk).  Returns 0 for unsupported
 * arguments.
 */
size_t sparse_attn_workspace_size(sa_dims d, int32_t d_proj, int32_t k, int32_t causal,
                                  int32_t dtype, int32_t with_idx);

/* Workspace bytes for processing `heads_per_chunk` (b, h) heads at a time. */
size_t sparse_attn_workspace_size_for_chunk(sa_dims d, int32_t d_proj, int32_t k,
                                            int32_t causal, int32_t dtype,
                                            int32_t with_idx, int32_t heads_per_chunk);

/*
 * Index sets of the method (steps 1-2).
 * page "mhpq.cn/news/1098205", §2.2 (scorer) and §3.2 (torch.topk, masks).
 *   Q, K: [B,H,N,D]; Pq, Pk: [D,d_proj]; idx (out): [B,H,N,k] int32.
 *   causal != 0: query i may only select keys j <= i (masked keys are
 *   removed before selection).
 *   score_scale: multiplies q_low·k_low (d_proj^-1/2 in the scorer of the
 *   pages; any positive value gives the same idx).
 * Row i of idx holds the k_i = min(k, #valid keys) keys with the highest
 * scores, ties going to the lower key index, written in ascending key order
 * and followed by k - k_i entries of -1.  The score that decides the
 * selection is the fp32 value reported by sparse_attn_scores_dump, and the
 * result is exactly the top-k of those values.
 */
int sparse_attn_scores_topk(const void* Q, const void* K, const void* Pq, const void* Pk,
                            sa_dims d, int32_t d_proj, int32_t k, int32_t causal,
                            float score_scale, int32_t dtype, int32_t* idx,
                            void* ws, size_t ws_bytes, const sa_options* opts, void* stream);

/*
 * Attention over index sets (step 3).
 * page "mhpq.cn/news/1098205", §3.2 (gather, matmul·scale, softmax, matmul)
 * and §1.2 (softmax(QKᵀ/√d_k)V).
 *   Q, K, V: [B,H,N,D]; idx: [B,H,N,k] int32; O (out): [B,H,N,D].
 *   O_i = Σ_t w_t V[idx_t], w = softmax(softmax_scale · q_i·K[idx_t]) over the
 *   entries idx_t >= 0 of row i.  Entries < 0 are skipped; repeated entries
 *   count as often as they appear; a row without entries gives O_i = 0.
 *   An entry >= N is skipped and sets a sticky device flag that
 *   sparse_attn_check_status reports.
 */
int sparse_attn_gather(const void* Q, const void* K, const void* V, const int32_t* idx,
                       int32_t k, sa_dims d, float softmax_scale, int32_t dtype, void* O,
                       const sa_options* opts, void* stream);

/*
 * sparse_attn_gather with a workspace, for large N: the same attention
 * (same entry rules, same sticky flag), computed by key range where a row
 * allows it, so that each XCD's L2 serves one range of the head's K and V
 * rows, as the fused forward does.  A row qualifies when its valid entries
 * (0 <= j < N) form an ascending prefix (repeats allowed) followed by
 * negative entries only, which is what sparse_attn_scores_topk,
 * sparse_attn_block_topk, the smoothed top-k and the band writers return;
 * every other row is attended in one pass as by sparse_attn_gather.  O
 * agrees with sparse_attn_gather's to fp32 rounding (the ranges' partial
 * softmax sums are merged), not bit for bit.
 *   ws: sparse_attn_gather_workspace_size(d, k, dtype) bytes (about 40 bytes
 *   per row plus 8·(D+4)·4 bytes per query of one head).  When that size is
 *   0 (N <= 8192, a head's K rows beyond 32-bit byte offsets, or more than
 *   2^31 - 1 rows in all) the call is sparse_attn_gather and ws may be NULL.  The workspace's contents need
 *   not start at zero.
 */
size_t sparse_attn_gather_workspace_size(sa_dims d, int32_t k, int32_t dtype);
int sparse_attn_gather_ws(const void* Q, const void* K, const void* V, const int32_t* idx,
                          int32_t k, sa_dims d, float softmax_scale, int32_t dtype, void* O,
                          void* ws, size_t ws_bytes, const sa_options* opts, void* stream);

/*
 * The whole forward, the two-step allocation of page "mhpq.cn/news/1098205"
 * §1.3 (score every pair cheaply, then attend only to each query's best k)
 * as run by the §3.2 forward: sparse_attn_scores_topk followed by
 * sparse_attn_gather, head chunk by head chunk.
 *   Q, K, V: [B,H,N,D]; Pq, Pk: [D,d_proj]; O (out): [B,H,N,D].
 *   idx_or_null receives the index sets when not NULL; otherwise they live
 *   in the workspace (size it with with_idx = 1).
 *   O and idx are exactly those of the two separate calls with the same
 *   arguments.  Errors: as for those two calls.
 */
int sparse_attn_fwd(const void* Q, const void* K, const void* V, const void* Pq,
                    const void* Pk, sa_dims d, int32_t d_proj, int32_t k, int32_t causal,
                    float score_scale, float softmax_scale, int32_t dtype, void* O,
                    int32_t* idx_or_null, void* ws, size_t ws_bytes, const sa_options* opts,
                    void* stream);

/*
 * Band (sliding-window) index sets: the fixed-index special case.
 * page "Attention机制改进：稀疏注意力应用" (create_local_mask: i-w <= j <= i+w)
 * and page "nxmr.cn/news/163144" §2.2 (window [i-w, i+w]).
 *   idx (out): [B,H,N,k] int32.  Row i holds keys max(0, i-w_left) ..
 *   min(N-1, i+w_right) in ascending order (clipped at the ends, not
 *   wrapped), truncated to k entries, then -1 padding.  d.D is ignored.
 */
int sparse_attn_band_indices(sa_dims d, int32_t w_left, int32_t w_right, int32_t* idx,
                             int32_t k, const sa_options* opts, void* stream);

/*
 * Backward of the forward for given index sets (page "mhpq.cn/news/1098205",
 * §2.3: the forward keeps the hard top-k; in the backward the selected
 * positions' gradients flow as usual, the unselected ones get zero, and the
 * scorer receives its gradient through the selected positions' attention
 * weights).
 *   Q, K, V, dO (upstream gradient of O): [B,H,N,D] of dtype; idx:
 *   [B,H,N,k] int32 (list semantics as in sparse_attn_gather: -1 skipped,
 *   repeats counted; entries >= N are skipped and set the sticky flag).
 *   Out, fp32 whatever the dtype: dQ, dK, dV [B,H,N,D] (overwritten).
 *   Attention path: with p = softmax(softmax_scale · q_i·K[idx_t]) and
 *   dl_t = p_t (dO_i·V[idx_t] - sum_u p_u dO_i·V[idx_u]):
 *   dQ_i = softmax_scale · sum_t dl_t K[idx_t]; each kept key j gets
 *   dV_j += p_t dO_i and dK_j += softmax_scale · dl_t q_i from every row i
 *   that kept it; keys no row kept get zero.
 *   Scorer path, when dPq and dPk are given ([D,d_proj] fp32, overwritten;
 *   Pq, Pk then required): the straight-through reading of §2.3, each kept
 *   pair's score score_scale · q_low_i·k_low_j receives its logit's
 *   gradient dl_t, which the chain rule takes through q_low = Q·Pq and
 *   k_low = K·Pk to dPq, dPk (summed over every head and row) and into dQ,
 *   dK.  With dPq = dPk = NULL only the attention path is computed.
 *   dK and dV add each key's contributions in an order that can differ
 *   from run to run (the entry lists are grouped by key through LDS
 *   atomics), so they agree between runs to fp32 rounding, not bit for bit.
 *   ws: sparse_attn_bwd_workspace_size(d, d_proj, k, scorer, opts) bytes
 *   (about 20 bytes per idx entry, plus the parts' records when the passes
 *   are split: about 8·(2·D + 4)·4 bytes per row).
 *   Errors: SA_ERR_SHAPE for a bwd_parts value other than the three above.
 */
size_t sparse_attn_bwd_workspace_size(sa_dims d, int32_t d_proj, int32_t k, int32_t scorer_grad,
                                      const sa_options* opts);
int sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* Pq, const void* Pk,
                    const void* dO, const int32_t* idx, sa_dims d, int32_t d_proj, int32_t k,
                    float score_scale, float softmax_scale, int32_t dtype, float* dQ, float* dK,
                    float* dV, float* dPq, float* dPk, void* ws, size_t ws_bytes,
                    const sa_options* opts, void* stream);

/*
 * Decode: one new query per (b, h) against the keys cached so far (page
 * "mhpq.cn/news/1098205", §3.4: at inference the selection runs for each
 * generated token over the KV cache, and how often a key is selected can
 * decide which cache entries are kept; page
 * "Attention机制优化：原理、挑战与工程实践", §4.3: a preallocated cache
 * updated in place at each step).
 *
 * The caller owns the caches: K and V caches [B,H,Ncap,D] (dtype), and a
 * k_low cache [B,H,Ncap,d_proj] fp32 holding each cached key's projection
 * K·Pk.  sparse_attn_decode_append_keys writes the projections of T new keys
 * K_new [B,H,T,D] (d.N = T) at cache rows pos .. pos+T-1 (0 <= pos,
 * pos + T <= Ncap), with the arithmetic of the prefill's projection, so the
 * cached values equal the prefill's bit for bit.
 *
 * sparse_attn_decode (d.N = Ncap): q [B,H,1,D]; the query of each (b, h)
 * attends to cache rows 0 .. len-1 (1 <= len <= Ncap; append the query's
 * own key first for a causal step).  The selection is the top-k of the
 * exact fp32 scores score_scale · q_low·k_low_j (the prefill's arithmetic:
 * the index row equals the causal prefill's row len-1 over the same keys),
 * ties to the lower key index, ascending, -1 padded when len < k.
 *   O (out): [B,H,1,D]; idx_or_null (out, optional): [B,H,k] int32;
 *   counts_or_null (in/out, optional): [B,H,Ncap] int32, each selected key's
 *   count is incremented (selection frequency for cache eviction).
 *   ws: sparse_attn_decode_workspace_size(d, d_proj, k) bytes (about 6 bytes
 *   per cache row and head: its score and its share of the slots for the
 *   keys collected near the k-th score); its contents need not start at
 *   zero (the call clears what it counts into).
 */
size_t sparse_attn_decode_workspace_size(sa_dims d, int32_t d_proj, int32_t k);
int sparse_attn_decode_append_keys(const void* K_new, const void* Pk, sa_dims d, int32_t d_proj,
                                   int32_t dtype, float* klow_cache, int32_t Ncap, int32_t pos,
                                   const sa_options* opts, void* stream);
int sparse_attn_decode(const void* q, const void* Kc, const void* Vc, const float* klow_cache,
                       const void* Pq, sa_dims d, int32_t d_proj, int32_t len, int32_t k,
                       float score_scale, float softmax_scale, int32_t dtype, void* O,
                       int32_t* idx_or_null, int32_t* counts_or_null, void* ws, size_t ws_bytes,
                       const sa_options* opts, void* stream);

/*
 * Block-granular selection (block-sparse attention: the SSA page's
 * _block_sparsify works on blocks of the mask; page "mhpq.cn/news/1098205"
 * §2.1, block-sparse attention computes only some block pairs).  Keys are cut
 * into blocks of `block` consecutive rows (the last one may be shorter).
 * Each block is scored as a whole with its mean projected key,
 *   kbar_J = fl(sum of the block's k_low rows, in key order) / n_J,
 *   score_iJ = score_scale · q_low_i·kbar_J (the fixed-order fp32 dot
 *   product of the token scores),
 * so a block's score is, up to rounding, the mean of its keys' scores.
 * Query i keeps its kb best blocks by (score descending, block ascending);
 * causally it keeps its own block (keys up to i) plus the kb-1 best blocks
 * that end before it.  idx (out) [B,H,N,kb*block] int32 lists the keys of
 * the kept blocks in ascending order (causally only j <= i), then -1; it
 * feeds sparse_attn_gather.  1 <= kb <= 32, kb*block <= SA_K_MAX.
 * sparse_attn_block_scores_dump writes the block scores of query rows
 * [row_begin, row_begin+row_count): S [B,H,row_count,ceil(N/block)] fp32.
 * Both take ws of sparse_attn_block_workspace_size(d, d_proj, block, kb)
 * bytes (the dump: kb = 1).
 */
size_t sparse_attn_block_workspace_size(sa_dims d, int32_t d_proj, int32_t block, int32_t kb);
int sparse_attn_block_topk(const void* Q, const void* K, const void* Pq, const void* Pk,
                           sa_dims d, int32_t d_proj, int32_t block, int32_t kb, int32_t causal,
                           float score_scale, int32_t dtype, int32_t* idx, void* ws,
                           size_t ws_bytes, const sa_options* opts, void* stream);
int sparse_attn_block_scores_dump(const void* Q, const void* K, const void* Pq, const void* Pk,
                                  sa_dims d, int32_t d_proj, int32_t block, float score_scale,
                                  int32_t dtype, int32_t row_begin, int32_t row_count, float* S,
                                  void* ws, size_t ws_bytes, const sa_options* opts,
                                  void* stream);

/*
 * sparse_attn_decode without any allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Arguments and results are
 * those of sparse_attn_decode; the workspace is instead a device-resident
 * array inside the library, one per GPU, held until the process ends and
 * found once per device (the first call on a device looks up its address).
 * Its size is sparse_attn_decode_noalloc_max_bytes() (32 MiB); a call whose
 * sparse_attn_decode_workspace_size exceeds it returns SA_ERR_WORKSPACE with
 * nothing enqueued (about 6 bytes per cache row and head: 32 heads of 128K
 * keys fit).  The call allocates nothing and records no timing events.
 * All calls on one GPU share that array: calls that overlap in time on one
 * GPU (other streams, other threads) race and must be ordered by the
 * caller.  Nothing in the array needs to start at zero: each call clears
 * the part it counts into with a fill kernel of its own.
 */
size_t sparse_attn_decode_noalloc_max_bytes(void);
int sparse_attn_decode_noalloc(const void* q, const void* Kc, const void* Vc,
                               const float* klow_cache, const void* Pq, sa_dims d,
                               int32_t d_proj, int32_t len, int32_t k, float score_scale,
                               float softmax_scale, int32_t dtype, void* O, int32_t* idx_or_null,
                               int32_t* counts_or_null, void* stream);

/*
 * Index variants feeding sparse_attn_gather.
 *
 * Boundary smoothing of the top-k (page "mhpq.cn/news/1098205", §4.2: when
 * the gap between the k-th and the (k+1)-th scores is below a threshold,
 * both keys are kept, so the number of kept keys varies a little from row
 * to row).
 *   Arguments as for sparse_attn_scores_topk, plus gap; idx (out) is
 *   [B,H,N,k+1] int32 and the workspace must be sized for k + 1
 *   (sparse_attn_workspace_size with k + 1).  Row i holds the keys of the
 *   top-k of the exact fp32 scores (those sparse_attn_scores_dump reports;
 *   ties to the lower key index), plus the (k+1)-th key when
 *   s_k - s_(k+1) < gap, the difference taken exactly (in double precision);
 *   ascending key order, -1 padding to k + 1 entries.  Rows with at most k
 *   valid keys keep them all.  1 <= k < SA_K_MAX; a NaN gap is SA_ERR_SHAPE.
 */
int sparse_attn_scores_topk_smoothed(const void* Q, const void* K, const void* Pq,
                                     const void* Pk, sa_dims d, int32_t d_proj, int32_t k,
                                     int32_t causal, float score_scale, float gap, int32_t dtype,
                                     int32_t* idx, void* ws, size_t ws_bytes,
                                     const sa_options* opts, void* stream);

/*
 * Dilated sliding window wrapped around the sequence (page
 * "Attention机制优化：原理、挑战与工程实践", §3.3: offsets t·dilation,
 * t < window, taken modulo the sequence length).
 *   idx (out): [B,H,N,k] int32; entry t of row i is (i + t·dilation) mod N
 *   for t < min(window, k), then -1.  Keys repeat when window·dilation > N
 *   and then count as often as they appear in the attention.  d.D is
 *   ignored.  window >= 0 and dilation >= 1, else SA_ERR_SHAPE.
 */
int sparse_attn_dilated_indices(sa_dims d, int32_t window, int32_t dilation, int32_t* idx,
                                int32_t k, const sa_options* opts, void* stream);

/*
 * Band with one radius per batch sample (page "nxmr.cn/news/163144", §6
 * adaptive attention: the window size is a per-sample value computed by the
 * model, so it is read from device memory).
 *   radii: DEVICE pointer to B int32 radii (a negative radius counts as 0);
 *   idx (out): [B,H,N,k] int32, row i of sample b holds keys
 *   max(0, i-w_b) .. min(N-1, i+w_b) ascending, truncated to k entries,
 *   then -1 padding.  d.D is ignored.
 */
int sparse_attn_band_indices_per_batch(sa_dims d, const int32_t* radii, int32_t* idx,
                                       int32_t k, const sa_options* opts, void* stream);

/*
 * The scorer's output for chosen query rows: the fp32 scores the selection
 * uses (page "mhpq.cn/news/1098205" §2.2, LightweightScorer: the scaled dot
 * product d_proj^-1/2 · q_low·k_lowᵀ), written out so that the top-k can be
 * recomputed from them; that page's troubleshooting notes (§4.4) suggest
 * comparing the selected top-k indices across runs, which needs exactly
 * these values.
 *   Rows [row_begin, row_begin + row_count) of every head: S (out) is
 *   [B,H,row_count,N] fp32, S[.., r, j] = fl(score_scale · fl(q_low_i ·
 *   k_low_j)) with the dot product accumulated in a fixed order; pairs
 *   excluded by the causal mask are -inf.
 *   Needs the same workspace as sparse_attn_scores_topk.  A row range
 *   outside [0, N) is SA_ERR_SHAPE.
 */
int sparse_attn_scores_dump(const void* Q, const void* K, const void* Pq, const void* Pk,
                            sa_dims d, int32_t d_proj, int32_t causal, float score_scale,
                            int32_t dtype, int32_t row_begin, int32_t row_count, float* S,
                            void* ws, size_t ws_bytes, const sa_options* opts, void* stream);

/*
 * Synchronizes `stream`, then reports and clears the sticky device flag:
 * SA_ERR_DEVICE_INDEX if a gather saw an index >= N since the last check,
 * SA_ERR_HIP if synchronization failed, SA_OK otherwise.
 */
int sparse_attn_check_status(void* stream);

/*
 * Diagnostics of the last sparse_attn_scores_topk / sparse_attn_fwd call
 * that used workspace `ws` (synchronizes `stream`).  Writes up to n values to
 * out: [0] queries resolved by the exact fallback path, [1] queries whose
 * first candidate list overflowed, [2] total candidates written, [3] total
 * keys re-scored exactly, [4] queries resolved, [5] queries filtered a second
 * time with a proven threshold, [6] re-scored keys whose exact score fell
 * outside the interval the filter's margin gives for it (0 unless the
 * margin's rounding bound is wrong), [7] queries the re-rank ranked from
 * their candidate lists in memory because they held more candidates than its
 * LDS room, summed over all head chunks of the call.  Returns the number of
 * values written or a negative status.
 */
int sparse_attn_workspace_stats(const void* ws, size_t ws_bytes, int64_t* out, int32_t n,
                                void* stream);

/*
 * Per-kernel timing for benchmarks, in a caller-owned record.
 * sparse_attn_profile_create returns a new, empty record (NULL if host
 * memory or HIP events cannot be had); the caller passes it in
 * sa_options.profile and frees it with sparse_attn_profile_destroy (NULL is
 * ignored).  sparse_attn_profile_read synchronizes the events of the
 * launches recorded so far and writes up to n (kernel name, milliseconds)
 * records in launch order, then forgets all of them; it returns the number
 * written or a negative status.  Recording costs two event records per
 * launch; a record not passed to a call costs nothing.
 */
typedef struct { char name[48]; float ms; } sa_kernel_time;
sa_profile* sparse_attn_profile_create(void);
void sparse_attn_profile_destroy(sa_profile* prof);
int sparse_attn_profile_read(sa_profile* prof, sa_kernel_time* out, int32_t n);

/* Static description of a status code. */
const char* sparse_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
