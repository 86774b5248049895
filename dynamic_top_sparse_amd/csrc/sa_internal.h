// Host-side plan of one scores/top-k pass and the kernel launch wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "sa_common.h"
#include "sparse_attn.h"

namespace sa {

// Tunables of the selection pipeline.
constexpr int kQueriesPerBlock = 256;   // scorer workgroup: 4 waves x 64 queries
constexpr int kKeysPerChunk = 128;      // keys staged in LDS per step
constexpr int kMaxSampleStride = 16;    // the threshold sample takes every s-th key, s <= 16
constexpr int kRowPad = 2048;           // N is padded to a multiple of this
constexpr float kTauBeta = 1.3f;        // sample rank slack (see threshold kernel)
constexpr int kFallbackBlocks = 256;    // workgroups of the exact fallback
constexpr int kKMax = 2048;             // largest supported k
constexpr int kGatherRanges = 8;        // key ranges of the split gather (a multiple of 8)
constexpr int kRetrySplit = 8;          // key segments of the retry filter (capH is a multiple of 64)

// Key ranges of the split gather: range r holds keys [b[r], b[r + 1]),
// b[0] = 0, b[kGatherRanges] = N.  Each range is served by one XCD, so the
// ranges should carry equal work.  A non-causal row may select any key: the
// ranges are equal.  A causal row i selects among keys 0..i; if it picks them
// evenly, key j is read by about k * ln(N / j) rows, and the work in [0, uN)
// is a fraction u * (1 - ln u) of the whole, so range r ends where that
// fraction reaches (r + 1) / kGatherRanges.
struct GatherRanges {
  int b[kGatherRanges + 1];
};

inline GatherRanges gather_ranges(int N, int causal) {
  static_assert(kGatherRanges == 8, "causal range table is for 8 ranges");
  // u with u * (1 - ln u) = r / 8, r = 0..8
  static const double kCausalFrac[kGatherRanges + 1] = {
      0.0, 0.027132, 0.067702, 0.120268, 0.186682, 0.271132, 0.382404, 0.543687, 1.0};
  GatherRanges g;
  const int L = (N + kGatherRanges - 1) / kGatherRanges;
  for (int r = 0; r <= kGatherRanges; ++r) {
    const long long x = causal ? static_cast<long long>(kCausalFrac[r] * N + 0.5)
                               : static_cast<long long>(r) * L;
    g.b[r] = static_cast<int>(x < N ? x : N);
  }
  g.b[kGatherRanges] = N;
  return g;
}

// Start of range r (wave-uniform table, lane-varying r): a select chain, so
// the kernel argument is never indexed by a lane value.
__device__ __forceinline__ int gather_range_start(const GatherRanges& g, int r) {
  int x = g.b[0];
#pragma unroll
  for (int t = 1; t <= kGatherRanges; ++t) x = r == t ? g.b[t] : x;
  return x;
}

// A candidate entry's key field.  The filter's accumulator r of tile-half h
// of the 32-key tile starting at key 32T covers key 32T + 4h + r + (r & 12);
// the entry stores x = 32T + 16h + r (one add in the filter), and the key is
// x + (x & 12) - 12 * ((x >> 4) & 1).
__device__ __forceinline__ int candidate_key(unsigned x) {
  return static_cast<int>(x + (x & 12u) - 12u * ((x >> 4) & 1u));
}

// Byte offsets of one head chunk's buffers inside the workspace.
struct Plan {
  int B, H, N, D, dp, k, causal, dtype;
  int filt;       // 16-bit filter operands: 0 = fp16, 1 = bf16
  int BH;         // B*H heads
  int hc;         // heads per chunk
  int Npad;       // N rounded up to kRowPad
  int sstride;    // sample stride s: a power of two, about beta*k/32, in [1, 16]
  int Ns;         // sample keys: ceil(N / s)
  int Nspad;      // Npad / s
  int NB;         // block maxima per query: 2 * ceil(Ns / 32)
  int capH;       // candidate capacity of one query half
  int with_idx;   // room for idx rows of the chunk
  int gsplit;     // the fused forward gathers by key range (N > 8192)
  size_t off_hdr, off_qlo32, off_klo32, off_qlo16, off_klo16, off_ksamp, off_qstat,
      off_kstat, off_bm, off_tau, off_thr, off_cand, off_cnt, off_rcnt, off_rlist, off_rcount, off_fblist,
      off_fbscratch, off_idx, off_seg, off_part, total;
};

// Fills every field from the arguments and heads_per_chunk; returns false
// when the sizes do not fit the index arithmetic.
// filt: the filter operand type (0 = fp16, 1 = bf16).
bool make_plan(Plan& p, int B, int H, int N, int D, int dp, int k, int causal, int dtype,
               int with_idx, int heads_per_chunk, int filt);

// Threshold sample: rank r of the sample maxima that sets a query's
// threshold (about beta * k keys are expected above it; the sample stride is
// chosen so that r is near 48), and the size B of the sample blocks whose
// maxima are kept for it: the largest power of two that leaves at least 4r
// blocks, so that the top samples rarely share a block.  Blocks of up to 16
// samples lie within one 32-sample tile (a lane sees 16 of its samples);
// larger ones span B/16 tiles.  The kernels that use these must agree.
__host__ __device__ inline int sample_rank(int k_i, int ns_valid, int n_valid, float beta) {
  const int r = static_cast<int>(ceilf(beta * static_cast<float>(k_i) *
                                       static_cast<float>(ns_valid) /
                                       static_cast<float>(n_valid)));
  return r < 1 ? 1 : r;
}
__host__ __device__ inline int sample_block(int ns_valid, int r) {
  int B = 1;
  while (ns_valid / (2 * B) >= 4 * r) B *= 2;
  return B;
}
// Maxima a query keeps: one per block of its valid sample tiles.
__host__ __device__ inline int sample_blocks(int ns_valid, int B) {
  const int tiles = (ns_valid + 31) / 32;
  return B <= 16 ? tiles * (32 / B) : 2 * ((tiles + B / 16 - 1) / (B / 16));
}

// Number of kstat words per head.
constexpr int kKeyStatWords = 4;

// Pointers of the chunk buffers for a given workspace base.
struct Bufs {
  WsHeader* hdr;
  float* qlo32;
  float* klo32;
  bf16_t* qlo16;
  bf16_t* klo16;
  bf16_t* ksamp;
  float4* qstat;        // per query: ||q_low||, ||q_low - q~||, 2^-e_q (norms rounded up)
  uint32_t* kstat;      // per head: max ||k_low||, max ||k_low - k~||, max |k_low|_inf (fp32 bits)
  uint16_t* bm;         // sample block maxima, top 16 bits of their order keys [NB][hc][Npad]
  float* tau;           // per-query threshold [hc][Npad]
  float* thr;           // the filter's threshold on the raw MFMA sum, as used [hc][Npad]
  uint2* cand;          // candidates [hc][Npad][2][capH] = (key, raw MFMA sum bits)
  int* cnt;             // candidates per query half [hc][Npad][2]
  int* rcnt;            // retry pass: candidates per query half and key segment [hc][Npad][2][kRetrySplit]
  int* rlist;           // per head: queries to filter again with a proven threshold
  int* rcount;          // per head: entries of rlist
  int* fblist;          // queries queued for the exact fallback
  float* fbscratch;     // [kFallbackBlocks][Npad] exact scores
  int32_t* idx;         // optional idx rows [hc][N][k]
  int* seg;             // split gather: key-range starts of each row [hc][Npad][kGatherRanges + 1]
  float* part;          // split gather, one head: partials [Npad][kGatherRanges][D + 4]
};
Bufs bufs_of(const Plan& p, void* ws);

// ---------------------------------------------------------- launches ---
// All return hipSuccess or the launch error.  `h0` is the first head of the
// chunk, `nh` the number of heads in it; Q, K, V are the full tensors.
hipError_t launch_init_chunk(const Plan& p, const Bufs& b, int first_chunk, hipStream_t s);
hipError_t launch_project(const Plan& p, const Bufs& b, const void* Q, const void* K,
                          const void* Pq, const void* Pk, int h0, int nh, hipStream_t s);
hipError_t launch_pack_keys(const Plan& p, const Bufs& b, int nh, hipStream_t s);
hipError_t launch_sample_maxima(const Plan& p, const Bufs& b, int nh, float score_scale,
                                hipStream_t s);
hipError_t launch_threshold(const Plan& p, const Bufs& b, int nh, float score_scale,
                            hipStream_t s);
// retry = false: every query; retry = true: the queries listed in rlist.
hipError_t launch_filter(const Plan& p, const Bufs& b, int nh, float score_scale, bool retry,
                         hipStream_t s);
// seg: null, or where the kernels that write idx rows also write each row's
// key-range starts for the split gather ([nh][Npad][kGatherRanges + 1]).
hipError_t launch_finalize(const Plan& p, const Bufs& b, int nh, float score_scale,
                           int32_t* idx_chunk, bool retry, int* seg, hipStream_t s);
hipError_t launch_fallback(const Plan& p, const Bufs& b, int nh, float score_scale,
                           int32_t* idx_chunk, int* seg, hipStream_t s);
hipError_t launch_dump(const Plan& p, const Bufs& b, int nh, float score_scale,
                       int row_begin, int row_count, float* S_chunk, hipStream_t s);
hipError_t launch_gather(const void* Q, const void* K, const void* V, const int32_t* idx,
                         int k, int nheads, int N, int D, float softmax_scale, int dtype,
                         void* O, hipStream_t s);
// Gather with Nq query rows and Nk key rows per head (Q, idx, O rows of head
// h at h*Nq; K, V rows at h*Nk).
hipError_t launch_gather_rows(const void* Q, const void* K, const void* V, const int32_t* idx,
                              int k, int nheads, int Nq, int Nk, int D, float softmax_scale,
                              int dtype, void* O, hipStream_t s);
// sparse_attn_gather_ws: per row (nheads*N of them) the key-range segment
// starts seg[row][0..8] of a row the range kernels can take, else -1s and
// the row's number h*N + q appended to list (count at *count, zeroed here);
// then the listed rows through the single-pass kernel.
hipError_t launch_gather_check(const int32_t* idx, int k, int nheads, int N, int* seg,
                               int* list, int* count, hipStream_t s);
hipError_t launch_gather_list(const void* Q, const void* K, const void* V, const int32_t* idx,
                              int k, int N, int D, float softmax_scale, int dtype, const int* list,
                              const int* count, void* O, hipStream_t s);
// Projection of `rows` rows of each of nh heads (X rows of head h at
// h*rows), written at row h*out_stride of lo32 (and lo16 / qstat for
// queries); nothing beyond `rows` is written.
hipError_t launch_project_rows(const void* X, const void* P, int nh, int rows, int out_stride,
                               int D, int dp, int dtype, int is_key, float* lo32, uint16_t* lo16,
                               float4* qstat, hipStream_t s);
// Decode (decode.hip), one query per head against the first `len` rows of
// a k_low cache (head stride Ncap rows):
//   clear:   zeroes the per-head histograms of the scores' leading bits;
//   scores:  exact scores [nh][Ncap] and, added to those histograms, the
//            count of keys per leading 11-bit bin of the order key;
//   collect: per slice of kDecodeSliceKeys keys, the keys at or above the
//            bin of the head's k-th largest score, in index order (at most
//            kDecodeCandCap per slice, the full count in ccount);
//   select:  the top-k per head, ascending, -1 padded; counts (optional)
//            gains one per selected key;
//   gather:  attention over the selected rows in kGatherRanges parts of the
//            index row, then their merge.
constexpr int kDecodeHistBins = 2048;
constexpr int kDecodeSliceKeys = 2048;
constexpr int kDecodeCandCap = 512;
__host__ __device__ inline int decode_slices(int len) { return (len + kDecodeSliceKeys - 1) / kDecodeSliceKeys; }
hipError_t launch_decode_clear(uint32_t* hist, int nh, hipStream_t s);
hipError_t launch_decode_scores(const float* qlo, int q_stride, const float* klow, int Ncap,
                                int len, int nh, int dp, float scale, float* scores,
                                uint32_t* hist, hipStream_t s);
hipError_t launch_decode_collect(const float* scores, int Ncap, int len, int nh, int k,
                                 const uint32_t* hist, uint2* cand, int* ccount, int2* selinfo,
                                 hipStream_t s);
hipError_t launch_decode_select(const float* scores, int len, int nh, int k, const uint2* cand,
                                const int* ccount, const int2* selinfo, int32_t* idx,
                                int32_t* counts, int Ncap, hipStream_t s);
hipError_t launch_decode_gather_part(const void* q, const void* Kc, const void* Vc,
                                     const int32_t* idx, int k, int len, int nh, int Ncap, int D,
                                     float softmax_scale, int dtype, float* part, hipStream_t s);
hipError_t launch_decode_gather_merge(const float* part, int nh, int D, int dtype, void* O,
                                      hipStream_t s);
// The no-allocation decode's device-resident workspace: its size, and its
// address on the current device (looked up once per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** out);

// Block-granular selection (block.hip): block means of k_low (kbar
// [nh][NB][dp]), each query's kept blocks (sel [nh][N][kb], best first; none
// written when sel is null), their keys as idx rows [nh][N][kb*block], and
// the block scores of chosen rows.  q32/k32 rows of head h at h*N.
hipError_t launch_block_select(const float* q32, const float* k32, int nh, int N, int dp,
                               int block, int kb, int causal, float scale, float* kbar,
                               int32_t* sel, hipStream_t s);
hipError_t launch_block_expand(const int32_t* sel, int nh, int N, int block, int kb, int causal,
                               int32_t* idx, hipStream_t s);
hipError_t launch_block_dump(const float* q32, const float* kbar, int nh, int N, int NB, int dp,
                             float scale, int row_begin, int row_count, float* S, hipStream_t s);

// Backward of the gather attention (gather.hip, the two wave passes) and its
// helpers (bwd.hip).  dp = 0 leaves out the scorer's gradient.
// One idx entry as the key pass reads it: e = i*k + t within the head, and
// the row pass's p_t and dl_t (12 bytes, one 3-dword access).
struct BwdEntry {
  int e;
  float p, dl;
};
struct BwdArgs {
  int pass;             // 0: row pass, 1: key pass
  int dtype, D, k, N, nh;
  int scorer;           // scorer gradients follow: store the sums unscaled
  float scale;
  const void *Q, *K, *V, *dO;
  const int32_t* idx;
  float *dQ, *dK, *dV;
  float2* epd;                  // (logit, dp_t) of every idx entry, in idx's layout
  float4* stats;                // per row: (max logit, 1/S, delta)
  const int *seg_off, *seg_cnt; // key pass: each key's segment of `rec`
  const BwdEntry* rec;          // per head, the entries grouped by key
  // key-range split of the passes (bwd.hip)
  int split_rows, split_keys, slices;
  const int* row_seg;           // per row: part starts (kGatherRanges + 1), or -1
  const int* bounds;            // per head: part key bounds (kGatherRanges + 1)
  const int* slice_pre;         // per slice and key: entries of the earlier slices
  float* part;                  // the parts' records
  // split key pass: -1 sums dV and H in one launch; 0 only dV (dO rows),
  // 1 only H (Q rows), for heads large enough that two launches are faster
  int keys_which;
};
hipError_t launch_bwd_pass(const BwdArgs& a, hipStream_t s);
// Whether the split key pass runs as two launches (dV, then H).
bool bwd_keys_two_launches(int N, int D);
// Device address of the sticky out-of-range index flag (gather.hip) on the
// current device.
hipError_t index_error_flag(int** out);
// Key segments of the entry list, built from idx alone: per-slice counts of
// each key (LDS histograms over windows of keys), their prefix over slices,
// each key's segment start, then the entries written into their segments.
int bwd_slices(int N, int k);
hipError_t launch_bwd_hist(const int32_t* idx, int nh, int N, int k, int S, int* cnt_s,
                           hipStream_t s);
hipError_t launch_bwd_slice_prefix(int* cnt_s, int S, long long total, int* cnt, hipStream_t s);
hipError_t launch_bwd_scan(const int* cnt, int nh, int N, int* off, hipStream_t s);
hipError_t launch_bwd_fill(const int32_t* idx, const float2* lpd, const float4* stats, int nh,
                           int N, int k, int S, const int* cnt_s, const int* off, BwdEntry* rec,
                           hipStream_t s);
hipError_t launch_bwd_bounds(const int* off, const int* cnt, int nh, int N, int* bounds,
                             hipStream_t s);
hipError_t launch_bwd_fill_parts(const int32_t* idx, const float2* lpd, const float4* stats,
                                 const int* row_seg, const int* bounds, int nh, int N, int k,
                                 int S, const int* cnt_s, const int* off, BwdEntry* rec,
                                 hipStream_t s);
hipError_t launch_bwd_row_ranges(const int32_t* idx, const int* bounds, int nh, int N, int k,
                                 int* seg, hipStream_t s);
hipError_t launch_bwd_rows_merge(const float* part, int nh, int N, int D, float out_scale,
                                 float* dQ, float4* stats, hipStream_t s);
hipError_t launch_bwd_keys_merge(const float* part, int nh, int N, int D, float out_scale,
                                 float* dK, float* dV, hipStream_t s);
// out[r][d] = pre * out[r][d] + sum_c lo[r][c] * P[d][c] over rows r (P [D][dp] of dtype)
hipError_t launch_rows_times_pt(const float* lo, const void* P, int dtype, long long rows, int D,
                                int dp, float pre, float* out, hipStream_t s);
// out[r][c] = alpha * sum_d X[r][d] * P[d][c] over rows r (X fp32, P [D][dp] of dtype)
hipError_t launch_rows_times_p(const float* X, const void* P, int dtype, long long rows, int D,
                               int dp, float alpha, float* out, hipStream_t s);
// dP[d][c] = sum_r X[r][d] * lo[r][c] over all rows (X of dtype), in a
// fixed order through per-chunk partials
hipError_t launch_outer_sum(const void* X, int dtype, const float* lo, long long rows, int D,
                            int dp, float* partial, int nchunks, float* dP, hipStream_t s);
int outer_sum_chunks(long long rows);

// Split gather of one head whose idx rows are ascending (the fused forward's).
// seg[q][r] (r = 0..kGatherRanges) is the first position of row q whose key
// is >= gather_ranges(N, causal).b[r]; the re-rank and fallback kernels write it
// beside the rows.
hipError_t launch_gather_split(const void* Q, const void* K, const void* V, const int32_t* idx,
                               int k, int N, int D, float softmax_scale, int dtype, const int* seg,
                               float* part, void* O, sa_profile* prof, hipStream_t s);
hipError_t launch_band(int nheads, int N, int w_left, int w_right, int32_t* idx, int k,
                       hipStream_t s);
// Index variants (variants.hip).
hipError_t launch_dilated(int nheads, int N, int window, int dilation, int32_t* idx, int k,
                          hipStream_t s);
hipError_t launch_band_batch(int B, int H, int N, const int32_t* radii, int32_t* idx, int k,
                             hipStream_t s);
// Boundary smoothing of a chunk's top-(k+1) rows (p.k is k+1), in place.
hipError_t launch_smooth(const Plan& p, const Bufs& b, int nh, float score_scale, float gap,
                         int32_t* idx_chunk, hipStream_t s);

// Optional per-launch timing into a caller-owned record (NULL: none).
// prof_begin records the start event and returns the slot that prof_end
// closes (-1 when nothing was recorded).
int prof_begin(sa_profile* prof, const char* name, hipStream_t s);
void prof_end(sa_profile* prof, int token, hipStream_t s);

// Sets a kernel's dynamic-LDS limit once per device (thread-safe); `flags`
// is a per-kernel array of kMaxDevices flags.
constexpr int kMaxDevices = 64;
hipError_t set_lds_limit_once(const void* kernel, int bytes, std::atomic<int>* flags);

// Sticky device flag set by the gather when an index is >= N.
hipError_t read_and_clear_device_flag(int* value, hipStream_t s);

}  // namespace sa
