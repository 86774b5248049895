// Host-side plan of one scores/top-k pass and the kernel launch wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sa_common.h"

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
bool make_plan(Plan& p, int B, int H, int N, int D, int dp, int k, int causal, int dtype,
               int with_idx, int heads_per_chunk);

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
// Split gather of one head whose idx rows are ascending (the fused forward's).
// seg[q][r] (r = 0..kGatherRanges) is the first position of row q whose key
// is >= gather_ranges(N, causal).b[r]; the re-rank and fallback kernels write it
// beside the rows.
hipError_t launch_gather_split(const void* Q, const void* K, const void* V, const int32_t* idx,
                               int k, int N, int D, float softmax_scale, int dtype, const int* seg,
                               float* part, void* O, hipStream_t s);
hipError_t launch_band(int nheads, int N, int w_left, int w_right, int32_t* idx, int k,
                       hipStream_t s);

// Optional per-launch timing (see sparse_attn_profile_enable).  Launch
// wrappers call prof_begin before and prof_end after a launch.
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);

// Sticky device flag set by the gather when an index is >= N.
hipError_t read_and_clear_device_flag(int* value, hipStream_t s);

}  // namespace sa
