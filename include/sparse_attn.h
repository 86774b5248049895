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
                            void* ws, size_t ws_bytes, void* stream);

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
                       void* stream);

/*
 * The whole forward: sparse_attn_scores_topk followed by sparse_attn_gather,
 * head chunk by head chunk.  idx_or_null receives the index sets when not
 * NULL; otherwise they live in the workspace (size it with with_idx = 1).
 */
int sparse_attn_fwd(const void* Q, const void* K, const void* V, const void* Pq,
                    const void* Pk, sa_dims d, int32_t d_proj, int32_t k, int32_t causal,
                    float score_scale, float softmax_scale, int32_t dtype, void* O,
                    int32_t* idx_or_null, void* ws, size_t ws_bytes, void* stream);

/*
 * Band (sliding-window) index sets: the fixed-index special case.
 * page "Attention机制改进：稀疏注意力应用" (create_local_mask: i-w <= j <= i+w)
 * and page "nxmr.cn/news/163144" §2.2 (window [i-w, i+w]).
 *   idx (out): [B,H,N,k] int32.  Row i holds keys max(0, i-w_left) ..
 *   min(N-1, i+w_right) in ascending order (clipped at the ends, not
 *   wrapped), truncated to k entries, then -1 padding.  d.D is ignored.
 */
int sparse_attn_band_indices(sa_dims d, int32_t w_left, int32_t w_right, int32_t* idx,
                             int32_t k, void* stream);

/*
 * The fp32 scores the selection uses, for query rows [row_begin,
 * row_begin + row_count) of every head: S (out) is [B,H,row_count,N] fp32.
 * S[.., r, j] = fl(score_scale · fl(q_low_i · k_low_j)) with the dot product
 * accumulated in a fixed order; pairs excluded by the causal mask are -inf.
 * Needs the same workspace as sparse_attn_scores_topk.
 */
int sparse_attn_scores_dump(const void* Q, const void* K, const void* Pq, const void* Pk,
                            sa_dims d, int32_t d_proj, int32_t causal, float score_scale,
                            int32_t dtype, int32_t row_begin, int32_t row_count, float* S,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * Operand type of the 16-bit MFMA filter inside sparse_attn_scores_topk and
 * sparse_attn_fwd: SA_F16 (default) or SA_BF16.  Rows are scaled by powers
 * of two before rounding (one exponent per query row, one per key head), so
 * either type covers the fp32 range.  The returned indices are the same for
 * both: the filter only discards keys that provably cannot be in the top-k,
 * and the final choice uses the exact fp32 score.  fp16 keeps 11 significant
 * bits instead of 8, which shrinks the band of keys that must be re-scored
 * exactly.  Process-wide; affects calls made after it returns.
 * Returns SA_OK or SA_ERR_UNSUPPORTED.
 */
int sparse_attn_set_filter_dtype(int32_t dtype);
int sparse_attn_get_filter_dtype(void);

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
 * time with a proven threshold, summed over all head chunks of the call.
 * Returns the number of values written or a negative status.
 */
int sparse_attn_workspace_stats(const void* ws, size_t ws_bytes, int64_t* out, int32_t n,
                                void* stream);

/*
 * Per-kernel timing for benchmarks.  While enabled, every kernel the library
 * launches is bracketed by a pair of HIP events recorded on the launch
 * stream; sparse_attn_profile_read synchronizes those events and returns
 * (kernel name, milliseconds) records in launch order, then forgets them.
 * Disabled by default; enabling it costs two event records per launch.
 */
typedef struct { char name[48]; float ms; } sa_kernel_time;
int sparse_attn_profile_enable(int32_t on);
int sparse_attn_profile_read(sa_kernel_time* out, int32_t n);

/* Static description of a status code. */
const char* sparse_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
