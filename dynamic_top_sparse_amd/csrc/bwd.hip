// Helpers of the backward (page "mhpq.cn/news/1098205", §2.3, gradients of
// the top-k attention): the key segments of the entry list, and the scorer's
// projection gradients.
//
// Key segments (a counting sort of idx's entries by key, per head): the
// rows are cut into S slices and the keys into windows of kHistWindow; one
// workgroup per (head, slice, window) counts its keys in an LDS histogram.
// The counts are added up over slices (each slice keeps its running prefix),
// scanned over keys into each key's segment start, and a second pass with
// the same grid places every entry (its index i*k + t within the head) at
// its slice's next free position of its key's segment, again through LDS
// counters, copying the row pass's (p, dl) beside it.  No global atomics; the
// order of entries within one slice's part of a segment is the order of the
// LDS atomics.
//
// Scorer: with q_low = Q·Pq and k_low = K·Pk, the straight-through gradient
// reaches dq_low = score_scale·G·Pk and dk_low = score_scale·H·Pq, where G and
// H are the row and key passes' unscaled sums (gather.hip; rows_times_p), then
//   dQ = scale·G + dq_low·Pqᵀ, dK = scale·H + dk_low·Pkᵀ   (rows_times_pt),
//   dPq = sum over every row of Qᵀ·dq_low, dPk likewise  (outer_sum: fixed
//   row chunks, then the chunks' partial sums added in chunk order, so the
//   result does not depend on scheduling).
#include <algorithm>
#include <type_traits>

#include "rows.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kOuterRows = 2048;    // rows per outer-sum chunk
constexpr int kStageRows = 32;      // rows staged in LDS at a time

constexpr int kHistThreads = 1024;
constexpr int kHistWindow = 32768;  // keys per window: 128 KB of LDS counters

// Calls fn(g, idx[g]) for the entries g in [a, b) of the 16-byte aligned
// array idx, spread over the workgroup: 16-byte loads on the aligned
// interior, single entries at the two ends.
template <typename Fn>
__device__ __forceinline__ void for_entries(const int32_t* __restrict__ idx, long long a,
                                            long long b, Fn fn) {
  const long long a4 = min(b, (a + 3) & ~3LL);
  const long long b4 = max(a4, b & ~3LL);
  const int tid = threadIdx.x;
  if (tid < a4 - a) fn(a + tid, idx[a + tid]);
  if (tid < b - b4) fn(b4 + tid, idx[b4 + tid]);
  const int4* v = reinterpret_cast<const int4*>(idx);
  for (long long q = a4 / 4 + tid; q < b4 / 4; q += kHistThreads) {
    const int4 x = v[q];
    fn(4 * q, x.x);
    fn(4 * q + 1, x.y);
    fn(4 * q + 2, x.z);
    fn(4 * q + 3, x.w);
  }
}

struct SliceWindow {
  int s, w0, W, i0, i1;
};

__device__ __forceinline__ SliceWindow slice_window(int N, int S, int rows_per_slice) {
  SliceWindow r;
  r.s = static_cast<int>(blockIdx.x) % S;
  r.w0 = static_cast<int>(blockIdx.x) / S * kHistWindow;
  r.W = min(kHistWindow, N - r.w0);
  r.i0 = min(N, r.s * rows_per_slice);
  r.i1 = min(N, r.i0 + rows_per_slice);
  return r;
}

// cnt_s[s][h][j] = entries of key j in the rows of slice s (keys outside
// 0..N-1, -1 included, are skipped).
__global__ __launch_bounds__(kHistThreads) void bwd_hist_kernel(const int32_t* __restrict__ idx,
                                                                int N, int k, int S,
                                                                int rows_per_slice, int nh,
                                                                int* __restrict__ cnt_s) {
  extern __shared__ int hist[];
  const SliceWindow sw = slice_window(N, S, rows_per_slice);
  const int h = blockIdx.y;
  for (int t = threadIdx.x; t < sw.W; t += kHistThreads) hist[t] = 0;
  __syncthreads();
  const long long hk = static_cast<long long>(h) * N * k;
  const unsigned w0 = static_cast<unsigned>(sw.w0), W = static_cast<unsigned>(sw.W);
  for_entries(idx, hk + static_cast<long long>(sw.i0) * k, hk + static_cast<long long>(sw.i1) * k,
              [&](long long, int j) {
                const unsigned u = static_cast<unsigned>(j) - w0;
                if (u < W) atomicAdd(&hist[u], 1);
              });
  __syncthreads();
  int* out = cnt_s + (static_cast<size_t>(sw.s) * nh + h) * N + sw.w0;
  for (int t = threadIdx.x; t < sw.W; t += kHistThreads) out[t] = hist[t];
}

// Per key: the total over slices into cnt, and each slice's count replaced by
// the sum of the earlier slices' counts.
__global__ void bwd_slice_prefix_kernel(int* __restrict__ cnt_s, int S, long long total,
                                        int* __restrict__ cnt) {
  for (long long x = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; x < total;
       x += static_cast<long long>(gridDim.x) * blockDim.x) {
    int run = 0;
    for (int s = 0; s < S; ++s) {
      const int v = cnt_s[s * total + x];
      cnt_s[s * total + x] = run;
      run += v;
    }
    cnt[x] = run;
  }
}

// Places the entries of one (head, slice, window) in their key segments.
__global__ __launch_bounds__(kHistThreads) void bwd_fill_kernel(const int32_t* __restrict__ idx,
                                                                const float2* __restrict__ lpd,
                                                                const float4* __restrict__ stats,
                                                                int N, int k, int S,
                                                                int rows_per_slice, int nh,
                                                                const int* __restrict__ cnt_s,
                                                                const int* __restrict__ off,
                                                                BwdEntry* __restrict__ rec) {
  extern __shared__ int cur[];
  const SliceWindow sw = slice_window(N, S, rows_per_slice);
  const int h = blockIdx.y;
  const size_t hN = static_cast<size_t>(h) * N;
  const int* before = cnt_s + (static_cast<size_t>(sw.s) * nh + h) * N + sw.w0;
  for (int t = threadIdx.x; t < sw.W; t += kHistThreads) cur[t] = off[hN + sw.w0 + t] + before[t];
  __syncthreads();
  const long long hk = static_cast<long long>(h) * N * k;
  BwdEntry* rh = rec + hk;
  const unsigned w0 = static_cast<unsigned>(sw.w0), W = static_cast<unsigned>(sw.W);
  for_entries(idx, hk + static_cast<long long>(sw.i0) * k, hk + static_cast<long long>(sw.i1) * k,
              [&](long long g, int j) {
                const unsigned u = static_cast<unsigned>(j) - w0;
                if (u < W) {
                  // p_t and dl_t from the logit, dp_t and the row's statistics
                  const float2 ld = lpd[g];
                  const int e = static_cast<int>(g - hk);
                  const float4 st = stats[hN + static_cast<unsigned>(e) / static_cast<unsigned>(k)];
                  BwdEntry r;
                  r.e = e;
                  r.p = ld.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ld.x - st.x) * st.y;
                  r.dl = r.p != 0.0f ? r.p * (ld.y - st.z) : 0.0f;
                  rh[atomicAdd(&cur[u], 1)] = r;
                }
              });
}

// The fill when the row pass ran in key-range parts: one workgroup per
// (head, slice, part) reads only the part's segment of each row of the slice
// (a row whose valid entries are not an ascending prefix: the whole row), so
// idx and (logit, dp) are read once in all; a part of more than kHistWindow
// keys is handled in windows of that many, one after another.
__global__ __launch_bounds__(kHistThreads) void bwd_fill_parts_kernel(
    const int32_t* __restrict__ idx, const float2* __restrict__ lpd,
    const float4* __restrict__ stats, const int* __restrict__ row_seg,
    const int* __restrict__ bounds, int N, int k, int S, int rows_per_slice, int nh,
    const int* __restrict__ cnt_s, const int* __restrict__ off, BwdEntry* __restrict__ rec) {
  constexpr int R = kGatherRanges;
  extern __shared__ int cur[];
  const int s = static_cast<int>(blockIdx.x) % S, r = static_cast<int>(blockIdx.x) / S;
  const int h = blockIdx.y;
  const size_t hN = static_cast<size_t>(h) * N;
  const long long hk = static_cast<long long>(h) * N * k;
  const int i0 = min(N, s * rows_per_slice), i1 = min(N, i0 + rows_per_slice);
  const int lo = bounds[h * (R + 1) + r], hi = bounds[h * (R + 1) + r + 1];
  const int* before = cnt_s + (static_cast<size_t>(s) * nh + h) * N;
  BwdEntry* rh = rec + hk;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  const int l = lane_id();
  constexpr int kFillWaves = kHistThreads / kWave;
  // A wave takes kFillRows rows at once and walks their part segments as one
  // list, kFillUnroll entries per lane loaded before any is placed: the
  // segment bounds, the idx entries and the (logit, dp) pairs each cost one
  // memory round trip per batch of rows instead of one per row.
  constexpr int kFillRows = 4, kFillUnroll = 4;
  for (int w0 = lo; w0 < hi; w0 += kHistWindow) {
    const int W = min(kHistWindow, hi - w0);
    __syncthreads();      // the previous window's cursors are no longer used
    for (int t = threadIdx.x; t < W; t += kHistThreads) cur[t] = off[hN + w0 + t] + before[w0 + t];
    __syncthreads();
    const unsigned uw0 = static_cast<unsigned>(w0), uW = static_cast<unsigned>(W);
    for (int ib = i0 + w * kFillRows; ib < i1; ib += kFillWaves * kFillRows) {
      int beg[kFillRows], cum[kFillRows + 1];
      float4 st[kFillRows];
      cum[0] = 0;
#pragma unroll
      for (int b = 0; b < kFillRows; ++b) {
        const int i = ib + b;
        int t0 = 0, t1 = 0;
        st[b] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (i < i1) {
          const int* sg = row_seg + (hN + i) * (R + 1);
          const bool sorted = sg[0] >= 0;
          t0 = sorted ? sg[r] : 0;
          t1 = sorted ? sg[r + 1] : k;
          st[b] = stats[hN + i];
        }
        beg[b] = t0;
        cum[b + 1] = cum[b] + (t1 - t0);
      }
      const int tot = cum[kFillRows];
      for (int e0 = 0; e0 < tot; e0 += kWave * kFillUnroll) {
        long long g[kFillUnroll];
        int j[kFillUnroll], bsel[kFillUnroll];
#pragma unroll
        for (int u = 0; u < kFillUnroll; ++u) {
          const int e = e0 + u * kWave + l;
          int b = 0;
#pragma unroll
          for (int c = 1; c < kFillRows; ++c) b += e >= cum[c] ? 1 : 0;
          int t = e, row_beg = 0;
#pragma unroll
          for (int c = 0; c < kFillRows; ++c)
            if (b == c) { t = beg[c] + e - cum[c]; row_beg = ib + c; }
          bsel[u] = b;
          g[u] = (static_cast<long long>(hN) + row_beg) * k + t;
          j[u] = e < tot ? idx[g[u]] : -1;
        }
        float2 ld[kFillUnroll];
#pragma unroll
        for (int u = 0; u < kFillUnroll; ++u) {
          ld[u] = make_float2(-INFINITY, 0.0f);
          if (static_cast<unsigned>(j[u]) - uw0 < uW) ld[u] = lpd[g[u]];
        }
#pragma unroll
        for (int u = 0; u < kFillUnroll; ++u) {
          const unsigned uu = static_cast<unsigned>(j[u]) - uw0;
          if (uu < uW) {
            float4 sb = st[0];
#pragma unroll
            for (int c = 1; c < kFillRows; ++c)
              if (bsel[u] == c) sb = st[c];
            BwdEntry e;
            e.e = static_cast<int>(g[u] - hk);
            e.p = ld[u].x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ld[u].x - sb.x) * sb.y;
            e.dl = e.p != 0.0f ? e.p * (ld[u].y - sb.z) : 0.0f;
            rh[atomicAdd(&cur[uu], 1)] = e;
          }
        }
      }
    }
  }
}

// One workgroup per head: exclusive scan of the counts, i.e. each key's
// first entry within the head's region of the entry list.
__global__ __launch_bounds__(kThreads) void bwd_scan_kernel(const int* __restrict__ cnt, int N,
                                                            int* __restrict__ off) {
  __shared__ int tmp[kThreads / kWave];
  const int h = blockIdx.x;
  const int* c = cnt + static_cast<size_t>(h) * N;
  int* o = off + static_cast<size_t>(h) * N;
  const int w = threadIdx.x / kWave, l = lane_id();
  int running = 0;
  for (int b0 = 0; b0 < N; b0 += kThreads) {
    const int j = b0 + threadIdx.x;
    const int v = j < N ? c[j] : 0;
    const int incl = wave_incl_scan(v);
    if (l == kWave - 1) tmp[w] = incl;
    __syncthreads();
    int before = 0, tot = 0;
    for (int i = 0; i < kThreads / kWave; ++i) {
      before += i < w ? tmp[i] : 0;
      tot += tmp[i];
    }
    if (j < N) o[j] = running + before + incl - v;
    running += tot;
    __syncthreads();
  }
}

// ----------------------------------------------- key-range split passes ---
// The row and key passes can run in kGatherRanges parts, part r on XCD r, so
// that each XCD's L2 serves one part of every head's rows (as the forward's
// split gather does).  Row pass: part r takes the entries whose key lies in
// [bounds[r], bounds[r+1]), cut per head so that each part holds about the
// same number of entries; a row whose valid entries are not an ascending
// prefix is handled by every part scanning the whole row.  Key pass: part r
// takes the entries of rows in slices [r S/8, (r+1) S/8), which the fill
// placed consecutively in each key's segment.  Each part writes a partial
// result per row or key; the merges add the parts in part order.

// Per head: bounds[h][r] = the smallest key j with at least r/8 of the head's
// entries below it (off is each key's exclusive entry count), bounds[h][8] = N.
__global__ void bwd_bounds_kernel(const int* __restrict__ off, const int* __restrict__ cnt, int N,
                                  int* __restrict__ bounds) {
  const int h = blockIdx.x, r = threadIdx.x;
  if (r > kGatherRanges) return;
  const int* o = off + static_cast<size_t>(h) * N;
  const long long total = static_cast<long long>(o[N - 1]) + cnt[static_cast<size_t>(h) * N + N - 1];
  int b;
  if (r == 0) {
    b = 0;
  } else if (r == kGatherRanges) {
    b = N;
  } else {
    const long long target = (total * r + kGatherRanges - 1) / kGatherRanges;
    int lo = 0, hi = N;        // first j with o[j] >= target (N if none)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (o[mid] < target) lo = mid + 1; else hi = mid;
    }
    b = lo;
  }
  bounds[h * (kGatherRanges + 1) + r] = b;
}

// One wave per row: if the row's valid entries (keys 0..N-1) form a prefix
// of it in ascending order, seg[row][r] = the number of them below
// bounds[r] (r = 0..8); else seg[row][0] = -1.
__global__ __launch_bounds__(kThreads) void bwd_row_ranges_kernel(const int32_t* __restrict__ idx,
                                                                  const int* __restrict__ bounds,
                                                                  int N, int k,
                                                                  int* __restrict__ seg) {
  constexpr int R = kGatherRanges;
  const int w = threadIdx.x / kWave, l = lane_id();
  const int q = blockIdx.x * (kThreads / kWave) + w;
  const int h = blockIdx.y;
  if (q >= N) return;
  const size_t row = static_cast<size_t>(h) * N + q;
  const int32_t* ir = idx + row * k;
  const int* b = bounds + h * (R + 1);
  int below[R + 1];
#pragma unroll
  for (int r = 0; r <= R; ++r) below[r] = 0;
  bool ok = true;               // wave-uniform after the ballots
  int last = -1;                // previous chunk's last entry (valid or not)
  constexpr int kChunks = 4;    // 64-entry chunks loaded before any is checked
  for (int c0 = 0; c0 < k; c0 += kChunks * kWave) {
    int jc[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int t = c0 + c * kWave + l;
      jc[c] = t < k ? ir[t] : -1;
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int t = c0 + c * kWave + l;
      const int j = jc[c];
      const bool valid = j >= 0 && j < N;
      int prev = __shfl_up(j, 1, kWave);
      if (l == 0) prev = last;
      const bool prev_valid = prev >= 0 && prev < N;
      // a valid entry right after an invalid one, or below its predecessor
      const bool bad = valid && ((t > 0 && !prev_valid) || (prev_valid && prev > j));
      if (__ballot(bad)) ok = false;
#pragma unroll
      for (int r = 1; r < R; ++r) below[r] += valid && j < b[r] ? 1 : 0;
      below[R] += valid ? 1 : 0;
      last = __shfl(j, kWave - 1, kWave);
    }
  }
  int* out = seg + row * (R + 1);
  if (!ok) {
    if (l == 0) out[0] = -1;
    return;
  }
#pragma unroll
  for (int r = 1; r <= R; ++r) below[r] = wave_sum_i(below[r]);
  if (l == 0) {
    out[0] = 0;
#pragma unroll
    for (int r = 1; r <= R; ++r) out[r] = below[r];
  }
}

// Row parts -> dQ (out_scale times G) and the row's statistics
// (max logit, 1/S, delta); a part record is (m, S, U, -, A[D], B[D]).
// Every load of a row is issued at once (an empty part's record holds stale
// values: its terms are selected away, never multiplied by a zero weight).
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_merge_kernel(const float* __restrict__ part,
                                                                  int N, float out_scale,
                                                                  float* __restrict__ dQ,
                                                                  float4* __restrict__ stats) {
  constexpr int R = kGatherRanges;
  constexpr int PS = 2 * D + 4;
  constexpr int EPL = D / kWave;
  const int w = threadIdx.x / kWave, l = lane_id();
  const int q = blockIdx.x * (kThreads / kWave) + w;
  if (q >= N) return;
  const size_t row = static_cast<size_t>(blockIdx.y) * N + q;
  const float* pr = part + row * R * PS;
  float mr[R], sr[R], ur[R], av[R][EPL], bv[R][EPL];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    mr[r] = pr[r * PS];
    sr[r] = pr[r * PS + 1];
    ur[r] = pr[r * PS + 2];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      av[r][i] = pr[r * PS + 4 + l + kWave * i];
      bv[r][i] = pr[r * PS + 4 + D + l + kWave * i];
    }
  }
  // (keeps the compiler from sinking loads past the reductions below)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    asm volatile("" ::"v"(mr[r]), "v"(sr[r]), "v"(ur[r]));
#pragma unroll
    for (int i = 0; i < EPL; ++i) asm volatile("" ::"v"(av[r][i]), "v"(bv[r][i]));
  }
  float M = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) M = fmaxf(M, mr[r]);
  float c[R];
  float S = 0.0f, U = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float m = mr[r];
    c[r] = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    S = m != -INFINITY ? __builtin_fmaf(c[r], sr[r], S) : S;
    U = m != -INFINITY ? __builtin_fmaf(c[r], ur[r], U) : U;
  }
  const bool none = M == -INFINITY;     // no valid entry in any part
  const float inv = 1.0f / S, delta = U * inv;
  float* dq = dQ + row * D;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    float a = 0.0f, bsum = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      a = c[r] != 0.0f ? __builtin_fmaf(c[r], av[r][i], a) : a;
      bsum = c[r] != 0.0f ? __builtin_fmaf(c[r], bv[r][i], bsum) : bsum;
    }
    dq[l + kWave * i] = none ? 0.0f : out_scale * ((a - delta * bsum) * inv);
  }
  if (l == 0)
    stats[row] = none ? make_float4(-INFINITY, 0.0f, 0.0f, 0.0f) : make_float4(M, inv, delta, 0.0f);
}

// Key parts (dV[D], H[D]) -> dV and dK (out_scale times H), parts in order.
__global__ __launch_bounds__(kThreads) void bwd_keys_merge_kernel(const float* __restrict__ part,
                                                                  int N, int D, float out_scale,
                                                                  float* __restrict__ dK,
                                                                  float* __restrict__ dV) {
  constexpr int R = kGatherRanges;
  const int w = threadIdx.x / kWave, l = lane_id();
  const int j = blockIdx.x * (kThreads / kWave) + w;
  if (j >= N) return;
  const size_t row = static_cast<size_t>(blockIdx.y) * N + j;
  const float* pr = part + row * R * 2 * D;
  for (int e = l; e < D; e += kWave) {
    float v = 0.0f, hsum = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      v += pr[r * 2 * D + e];
      hsum += pr[r * 2 * D + D + e];
    }
    dV[row * D + e] = v;
    dK[row * D + e] = out_scale * hsum;
  }
}

// out[r][d] = pre * out[r][d] + sum_c lo[r][c] P[d][c].  P^T (fp32) and a
// block of lo rows sit in LDS; each thread accumulates a tile of RT rows x 4
// columns.
constexpr int kRptRows = 32;

template <int D, int DP>
__host__ __device__ constexpr size_t rpt_lds_bytes() {
  return static_cast<size_t>(DP * D + kRptRows * DP) * 4;
}

template <typename T, int D, int DP>
__global__ __launch_bounds__(kThreads) void rows_times_pt_kernel(const float* __restrict__ lo,
                                                                 const T* __restrict__ P,
                                                                 long long rows, float pre,
                                                                 float* __restrict__ out) {
  extern __shared__ __align__(16) float rpt_lds[];
  float* pt = rpt_lds;               // pt[c * D + d]
  float* ls = rpt_lds + DP * D;      // ls[r * DP + c]
  for (int e = threadIdx.x; e < D * DP; e += kThreads) {
    const int d = e / DP, c = e % DP;
    pt[c * D + d] = io<T>::to_f32(P[e]);
  }
  constexpr int TPR = D / 4;                    // threads across one row's columns
  constexpr int RT = kRptRows * TPR / kThreads;  // rows per thread
  const int d0 = (threadIdx.x % TPR) * 4;
  const int rr0 = (threadIdx.x / TPR) * RT;
  for (long long rb = blockIdx.x * static_cast<long long>(kRptRows); rb < rows;
       rb += static_cast<long long>(gridDim.x) * kRptRows) {
    const int nr = static_cast<int>(rows - rb < kRptRows ? rows - rb : kRptRows);
    __syncthreads();
    const float4* src = reinterpret_cast<const float4*>(lo + rb * DP);
    for (int e = threadIdx.x; e < kRptRows * DP / 4; e += kThreads)
      reinterpret_cast<float4*>(ls)[e] = e < nr * DP / 4 ? src[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    float acc[RT][4];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
#pragma unroll 4
    for (int c = 0; c < DP; ++c) {
      const float4 p = *reinterpret_cast<const float4*>(pt + c * D + d0);
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const float x = ls[(rr0 + i) * DP + c];
        acc[i][0] = __builtin_fmaf(x, p.x, acc[i][0]);
        acc[i][1] = __builtin_fmaf(x, p.y, acc[i][1]);
        acc[i][2] = __builtin_fmaf(x, p.z, acc[i][2]);
        acc[i][3] = __builtin_fmaf(x, p.w, acc[i][3]);
      }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const long long r = rb + rr0 + i;
      if (r < rows) {
        float4* o = reinterpret_cast<float4*>(out + r * D + d0);
        float4 v = *o;
        v.x = __builtin_fmaf(pre, v.x, acc[i][0]);
        v.y = __builtin_fmaf(pre, v.y, acc[i][1]);
        v.z = __builtin_fmaf(pre, v.z, acc[i][2]);
        v.w = __builtin_fmaf(pre, v.w, acc[i][3]);
        *o = v;
      }
    }
  }
}

// out[r][c] = alpha * sum_d X[r][d] P[d][c] (X fp32 [rows][D], P [D][DP]).
// P (fp32) and a block of X rows sit in LDS; each thread accumulates a tile
// of RT rows x CT columns.
template <int D, int DP>
__host__ __device__ constexpr size_t rp_lds_bytes() {
  return static_cast<size_t>(D * DP + kRptRows * D) * 4;
}

template <typename T, int D, int DP>
__global__ __launch_bounds__(kThreads) void rows_times_p_kernel(const float* __restrict__ X,
                                                                const T* __restrict__ P,
                                                                long long rows, float alpha,
                                                                float* __restrict__ out) {
  extern __shared__ __align__(16) float rp_lds[];
  float* ps = rp_lds;               // ps[d * DP + c]
  float* xs = rp_lds + D * DP;      // xs[r * D + d]
  for (int e = threadIdx.x; e < D * DP; e += kThreads) ps[e] = io<T>::to_f32(P[e]);
  constexpr int CT = DP >= 32 ? 4 : 2;
  constexpr int TPR = DP / CT;                   // threads across one row's columns
  constexpr int RT = kRptRows * TPR / kThreads;  // rows per thread
  static_assert(RT >= 1 && RT * (kThreads / TPR) == kRptRows, "tile cover");
  const int c0 = (threadIdx.x % TPR) * CT;
  const int rr0 = (threadIdx.x / TPR) * RT;
  for (long long rb = blockIdx.x * static_cast<long long>(kRptRows); rb < rows;
       rb += static_cast<long long>(gridDim.x) * kRptRows) {
    const int nr = static_cast<int>(rows - rb < kRptRows ? rows - rb : kRptRows);
    __syncthreads();
    const float4* src = reinterpret_cast<const float4*>(X + rb * D);
    for (int e = threadIdx.x; e < kRptRows * D / 4; e += kThreads)
      reinterpret_cast<float4*>(xs)[e] = e < nr * D / 4 ? src[e] : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    float acc[RT][CT];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
      for (int j = 0; j < CT; ++j) acc[i][j] = 0.0f;
#pragma unroll 4
    for (int d = 0; d < D; ++d) {
      float pv[CT];
#pragma unroll
      for (int j = 0; j < CT; ++j) pv[j] = ps[d * DP + c0 + j];
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const float x = xs[(rr0 + i) * D + d];
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = __builtin_fmaf(x, pv[j], acc[i][j]);
      }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      const long long r = rb + rr0 + i;
      if (r < rows) {
#pragma unroll
        for (int j = 0; j < CT; ++j) out[r * DP + c0 + j] = alpha * acc[i][j];
      }
    }
  }
}

// partial[chunk][d][c] = sum over the chunk's rows r (ascending) of
// X[r][d] lo[r][c]; each thread owns a tile of DT x 4 outputs.
template <typename T, int D, int DP>
__global__ __launch_bounds__(kThreads) void outer_partial_kernel(const T* __restrict__ X,
                                                                 const float* __restrict__ lo,
                                                                 long long rows,
                                                                 float* __restrict__ partial) {
  constexpr int CT = 4, TPC = DP / CT;          // threads across the DP columns
  constexpr int DT = D * DP / kThreads / CT;    // d's per thread
  static_assert(TPC * (D / DT) == kThreads, "tile cover");
  __shared__ __align__(16) float xs[kStageRows * D];
  __shared__ __align__(16) float ls[kStageRows * DP];
  const int c0 = (threadIdx.x % TPC) * CT;
  const int d0 = (threadIdx.x / TPC) * DT;
  float acc[DT][CT];
#pragma unroll
  for (int i = 0; i < DT; ++i)
#pragma unroll
    for (int j = 0; j < CT; ++j) acc[i][j] = 0.0f;
  const long long r0 = blockIdx.x * static_cast<long long>(kOuterRows);
  const long long r1 = r0 + kOuterRows < rows ? r0 + kOuterRows : rows;
  for (long long rb = r0; rb < r1; rb += kStageRows) {
    const int nr = static_cast<int>(r1 - rb < kStageRows ? r1 - rb : kStageRows);
    __syncthreads();
    for (int e = threadIdx.x; e < kStageRows * D; e += kThreads)
      xs[e] = e < nr * D ? io<T>::to_f32(X[rb * D + e]) : 0.0f;
    for (int e = threadIdx.x; e < kStageRows * DP; e += kThreads)
      ls[e] = e < nr * DP ? lo[rb * DP + e] : 0.0f;
    __syncthreads();
    for (int r = 0; r < nr; ++r) {
      const float4 l4 = *reinterpret_cast<const float4*>(ls + r * DP + c0);
#pragma unroll
      for (int i = 0; i < DT; ++i) {
        const float x = xs[r * D + d0 + i];
        acc[i][0] = __builtin_fmaf(x, l4.x, acc[i][0]);
        acc[i][1] = __builtin_fmaf(x, l4.y, acc[i][1]);
        acc[i][2] = __builtin_fmaf(x, l4.z, acc[i][2]);
        acc[i][3] = __builtin_fmaf(x, l4.w, acc[i][3]);
      }
    }
  }
  float* dst = partial + static_cast<size_t>(blockIdx.x) * D * DP;
#pragma unroll
  for (int i = 0; i < DT; ++i)
    *reinterpret_cast<float4*>(dst + (d0 + i) * DP + c0) =
        make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
}

__global__ void outer_reduce_kernel(const float* __restrict__ partial, int nchunks, int n,
                                    float* __restrict__ dP) {
  const int o = blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= n) return;
  float s = 0.0f;
  for (int c = 0; c < nchunks; ++c) s += partial[static_cast<size_t>(c) * n + o];
  dP[o] = s;
}

unsigned grid_for(long long total) {
  long long blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return static_cast<unsigned>(blocks);
}

template <typename T, int D, int DP>
hipError_t rows_pt_t(const float* lo, const void* P, long long rows, float pre, float* out,
                     hipStream_t s) {
  static std::atomic<int> lds_set[kMaxDevices];
  const size_t lds = rpt_lds_bytes<D, DP>();
  const hipError_t e = set_lds_limit_once(
      reinterpret_cast<const void*>(&rows_times_pt_kernel<T, D, DP>), lds, lds_set);
  if (e != hipSuccess) return e;
  long long blocks = (rows + kRptRows - 1) / kRptRows;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((rows_times_pt_kernel<T, D, DP>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), lds, s, lo, static_cast<const T*>(P), rows, pre, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t rows_pt_d(const float* lo, const void* P, long long rows, int dp, float pre, float* out,
                     hipStream_t s) {
  switch (dp) {
    case 16: return rows_pt_t<T, D, 16>(lo, P, rows, pre, out, s);
    case 32: return rows_pt_t<T, D, 32>(lo, P, rows, pre, out, s);
    case 64: return rows_pt_t<T, D, 64>(lo, P, rows, pre, out, s);
    case 128: return rows_pt_t<T, D, 128>(lo, P, rows, pre, out, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D, int DP>
hipError_t rows_p_t(const float* X, const void* P, long long rows, float alpha, float* out,
                    hipStream_t s) {
  static std::atomic<int> lds_set[kMaxDevices];
  const size_t lds = rp_lds_bytes<D, DP>();
  const hipError_t e = set_lds_limit_once(
      reinterpret_cast<const void*>(&rows_times_p_kernel<T, D, DP>), lds, lds_set);
  if (e != hipSuccess) return e;
  long long blocks = (rows + kRptRows - 1) / kRptRows;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL((rows_times_p_kernel<T, D, DP>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), lds, s, X, static_cast<const T*>(P), rows, alpha, out);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t rows_p_d(const float* X, const void* P, long long rows, int dp, float alpha, float* out,
                    hipStream_t s) {
  switch (dp) {
    case 16: return rows_p_t<T, D, 16>(X, P, rows, alpha, out, s);
    case 32: return rows_p_t<T, D, 32>(X, P, rows, alpha, out, s);
    case 64: return rows_p_t<T, D, 64>(X, P, rows, alpha, out, s);
    case 128: return rows_p_t<T, D, 128>(X, P, rows, alpha, out, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t outer_d(const void* X, const float* lo, long long rows, int dp, float* partial,
                   int nchunks, hipStream_t s) {
  switch (dp) {
#define SA_OUT(DPV)                                                                          \
  case DPV:                                                                                  \
    hipLaunchKernelGGL((outer_partial_kernel<T, D, DPV>), dim3(nchunks), dim3(kThreads), 0, s, \
                       static_cast<const T*>(X), lo, rows, partial);                         \
    return hipGetLastError();
    SA_OUT(16)
    SA_OUT(32)
    SA_OUT(64)
    SA_OUT(128)
#undef SA_OUT
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------ backward ---
// Backward of the attention over index sets (page "mhpq.cn/news/1098205",
// §2.3: the forward keeps the hard top-k; in the backward the selected
// positions' gradients flow as usual and the others get none; the scorer is
// reached through the selected positions' attention weights).  With
// p_t = softmax(l)_t, dp_t = dO·V[j_t], delta = sum_t p_t dp_t and
// dl_t = p_t (dp_t - delta):
//   G_i = sum_t dl_t K[j_t],  dQ_i = scale · G_i              (row pass)
//   dV_j = sum over (i, t) with j_t = j of p_t dO_i            (key pass)
//   H_j = sum over the same of dl_t Q_i,  dK_j = scale · H_j   (key pass)
// The scorer's gradients need no further gathers: a kept pair's score
// receives its logit's gradient dl_t (straight-through), so
//   dq_low_i = score_scale · sum_t dl_t k_low[j_t] = score_scale · G_i·Pk,
//   dk_low_j = score_scale · H_j·Pq,
// by linearity (bwd.hip computes them from G and H).  With scorer gradients
// the passes store G and H unscaled (out_scale 1), else scale·G and scale·H.
// The row pass writes (p_t, dl_t) in idx's layout; bwd.hip groups them by
// key, and the key pass gathers the rows of the queries that kept each key,
// as the forward gathers key rows.
constexpr int kBwdChunk = 512;     // key-pass entries staged in LDS at a time

__host__ __device__ constexpr int bwd_row_wave_floats(int k) { return 3 * gather_slog_floats(k); }
__host__ __device__ constexpr int bwd_key_wave_floats() { return 3 * gather_slog_floats(kBwdChunk); }

template <int EPL>
__device__ __forceinline__ void store_f32_row(float* dst, const float (&v)[EPL], float f) {
#pragma unroll
  for (int e = 0; e < EPL; e += 4)
    *reinterpret_cast<float4*>(dst + e) = make_float4(v[e] * f, v[e + 1] * f, v[e + 2] * f, v[e + 3] * f);
}

// Cross-group combination for the row pass: lanes holding the same row
// elements in different row groups (xor partners LPR .. 32).
template <int LPR>
__device__ __forceinline__ float groups_sum(float v) {
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
    v = o == 32 ? sum_xor32(v) : o == 16 ? sum_xor16(v) : v + __shfl_xor(v, o, kWave);
  return v;
}
template <int LPR>
__device__ __forceinline__ float groups_max(float v) {
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
    v = o == 32 ? max_xor32(v) : o == 16 ? max_xor16(v) : fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// K pass of the backward row, one read of each kept K row: the logits
// (base 2, into slog) and, per row group over the entries it loads, the sums
//   S = sum e_t, U = sum e_t dp_t, A = sum e_t dp_t K_t, B = sum e_t K_t,
// with e_t = 2^(l_t - m) for the group's running maximum m (the sums are
// rescaled when m grows).  dp_t comes from sdp.  Then
//   p_t = e_t / S, delta = U / S, sum_t dl_t K_t = (A - delta B) / S
// once the groups are combined at the largest m.
template <typename T, int D>
__device__ __forceinline__ void bwd_logits_online(const T* __restrict__ qrow,
                                                  const T* __restrict__ K,
                                                  const int32_t* __restrict__ row, int n, int N,
                                                  float scale2, float* slog,
                                                  const float* sdp, int& bad, float& m,
                                                  float& S, float& U,
                                                  float (&A)[Vec<T>::kElems],
                                                  float (&B)[Vec<T>::kElems]) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL, RPI = kWave / LPR;
  const int l = lane_id();
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  float qf[EPL];
  Vec<T>::unpack(*reinterpret_cast<const uint4*>(qrow + e0), qf);
  m = -INFINITY;
  S = U = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) A[e] = B[e] = 0.0f;
  for (int tb = 0; tb < n; tb += RPI * kUnroll) {
    const int nu = min(kUnroll, (n - tb + RPI - 1) / RPI);   // loads holding rows (uniform)
    uint4 kv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const int jr = row[t];                       // t < n + RPI: inside the slack
      const int j = t < n ? jr : -1;
      ok[u] = j >= 0 && j < N;
      bad |= (t < n && j >= N) ? 1 : 0;
      kv[u] = *reinterpret_cast<const uint4*>(K + static_cast<size_t>(ok[u] ? j : 0) * D + e0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      float kf[EPL];
      Vec<T>::unpack(kv[u], kf);
      float dot = 0.0f;
      if constexpr (sizeof(T) == 2) {
        bf16x2 kp[4], qp[4];
        const uint4 q4 = *reinterpret_cast<const uint4*>(qrow + e0);
        __builtin_memcpy(kp, &kv[u], 16);
        __builtin_memcpy(qp, &q4, 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) dot = __builtin_amdgcn_fdot2_f32_bf16(kp[i], qp[i], dot, false);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qf[e], kf[e], dot);
      }
      dot = group_sum<LPR>(dot);
      const float lt = ok[u] ? dot * scale2 : -INFINITY;
      if ((l % LPR) == 0 && t < n) slog[t] = lt;
      if (lt > m) {                 // the whole group agrees: lt and m are group values
        const float c = __builtin_amdgcn_exp2f(m - lt);   // m = -inf gives 0
        S *= c;
        U *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          A[e] *= c;
          B[e] *= c;
        }
        m = lt;
      }
      const float ew = ok[u] ? __builtin_amdgcn_exp2f(lt - m) : 0.0f;
      const float ed = ok[u] ? ew * sdp[t] : 0.0f;
      S += ew;
      U += ed;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        A[e] = __builtin_fmaf(ed, kf[e], A[e]);
        B[e] = __builtin_fmaf(ew, kf[e], B[e]);
      }
    }
  }
  // combine the groups at the largest maximum
  const float M = groups_max<LPR>(m);
  const float c = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
  S = groups_sum<LPR>(S * c);
  U = groups_sum<LPR>(U * c);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    A[e] = groups_sum<LPR>(A[e] * c);
    B[e] = groups_sum<LPR>(B[e] * c);
  }
  m = M;
}

// bwd_logits_online for bf16 rows whose entries all hold keys in [0, N)
// (a part's segment of an ascending row): the forward split gather's trusted
// row loads (clamped keys, 32-bit offsets, straight-line blocks of loads,
// the block's dot products reduced together).
template <int D>
__device__ __forceinline__ void bwd_logits_online_trusted(const bf16_t* __restrict__ qrow,
                                                          const bf16_t* __restrict__ Kh,
                                                          const int* __restrict__ row, int n,
                                                          int N, float scale2, float* slog,
                                                          const float* sdp, float& m, float& S,
                                                          float& U, float (&A)[8], float (&B)[8]) {
  constexpr int EPL = 8, LPR = D / EPL, RPI = kWave / LPR, BLK = RPI * kUnroll;
  const int l = lane_id();
  const int g = l / LPR;
  const unsigned lane_off = static_cast<unsigned>((l % LPR) * EPL * 2);
  const char* kb = reinterpret_cast<const char*>(Kh);
  const uint4 q4 = *reinterpret_cast<const uint4*>(qrow + (l % LPR) * EPL);
  bf16x2 qp[4];
  __builtin_memcpy(qp, &q4, 16);
  auto dot_of = [&](const uint4& kv) {
    bf16x2 kp[4];
    __builtin_memcpy(kp, &kv, 16);
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) dot = __builtin_amdgcn_fdot2_f32_bf16(kp[i], qp[i], dot, false);
    return dot;
  };
  m = -INFINITY;
  S = U = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) A[e] = B[e] = 0.0f;
  auto update = [&](float lt, float dp, const uint4& kv) {   // lt finite
    if (lt > m) {
      const float c = __builtin_amdgcn_exp2f(m - lt);
      S *= c;
      U *= c;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        A[e] *= c;
        B[e] *= c;
      }
      m = lt;
    }
    const float ew = __builtin_amdgcn_exp2f(lt - m), ed = ew * dp;
    S += ew;
    U += ed;
    float kf[EPL];
    Vec<bf16_t>::unpack(kv, kf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      A[e] = __builtin_fmaf(ed, kf[e], A[e]);
      B[e] = __builtin_fmaf(ew, kf[e], B[e]);
    }
  };
  int tb = 0;
  for (; tb + BLK <= n; tb += BLK) {
    uint4 kv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      kv[u] = *reinterpret_cast<const uint4*>(kb + row_offset<D>(row, tb + u * RPI + g, N, lane_off));
    float dot[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dot[u] = dot_of(kv[u]);
    group_sum_n<LPR>(dot);
    // the block's largest logit first: one rescale per block, not per row
    float mb = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      dot[u] *= scale2;
      mb = fmaxf(mb, dot[u]);
      if ((l % LPR) == 0) slog[tb + u * RPI + g] = dot[u];
    }
    if (mb > m) {                   // group-uniform
      const float c = __builtin_amdgcn_exp2f(m - mb);   // m = -inf gives 0
      S *= c;
      U *= c;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        A[e] *= c;
        B[e] *= c;
      }
      m = mb;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float ew = __builtin_amdgcn_exp2f(dot[u] - m), ed = ew * sdp[tb + u * RPI + g];
      S += ew;
      U += ed;
      float kf[EPL];
      Vec<bf16_t>::unpack(kv[u], kf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        A[e] = __builtin_fmaf(ed, kf[e], A[e]);
        B[e] = __builtin_fmaf(ew, kf[e], B[e]);
      }
    }
  }
  if (tb < n) {
    const int nu = (n - tb + RPI - 1) / RPI;   // loads holding rows (uniform)
    uint4 kv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      kv[u] = *reinterpret_cast<const uint4*>(kb + row_offset<D>(row, tb + u * RPI + g, N, lane_off));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const float dot = group_sum<LPR>(dot_of(kv[u]));
      if (t < n) {                  // group-uniform: slack entries past the segment are dropped
        const float lt = dot * scale2;
        if ((l % LPR) == 0) slog[t] = lt;
        update(lt, sdp[t], kv[u]);
      }
    }
  }
  const float M = groups_max<LPR>(m);
  const float c = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
  S = groups_sum<LPR>(S * c);
  U = groups_sum<LPR>(U * c);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    A[e] = groups_sum<LPR>(A[e] * c);
    B[e] = groups_sum<LPR>(B[e] * c);
  }
  m = M;
}

// The key pass's two weighted sums over the same trusted bf16 rows list:
// acc1 = sum_t w1_t X1[j_t] and acc2 = sum_t w2_t X2[j_t], the two rows of an
// entry loaded together (kPair entries of each in flight per lane), partial
// sums reduced across the row groups at the end as in weighted_rows.
constexpr int kPair = 4;

template <int D>
__device__ __forceinline__ void weighted_rows2_bf16(const bf16_t* __restrict__ X1,
                                                    const float* __restrict__ w1,
                                                    const bf16_t* __restrict__ X2,
                                                    const float* __restrict__ w2,
                                                    const int* __restrict__ row, int n, int N,
                                                    float (&acc1)[8], float (&acc2)[8]) {
  constexpr int EPL = 8, LPR = D / EPL, RPI = kWave / LPR, BLK = RPI * kPair;
  const int l = lane_id();
  const int g = l / LPR;
  const unsigned lane_off = static_cast<unsigned>((l % LPR) * EPL * 2);
  const char* b1 = reinterpret_cast<const char*>(X1);
  const char* b2 = reinterpret_cast<const char*>(X2);
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc1[e] = acc2[e] = 0.0f;
  auto add = [&](const uint4& v, float w, float (&acc)[8]) {
    float vf[EPL];
    Vec<bf16_t>::unpack(v, vf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, vf[e], acc[e]);
  };
  for (int tb = 0; tb < n; tb += BLK) {
    const int nu = min(kPair, (n - tb + RPI - 1) / RPI);   // loads holding rows (uniform)
    uint4 v1[kPair], v2[kPair];
    float x1[kPair], x2[kPair];
#pragma unroll
    for (int u = 0; u < kPair; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const unsigned o = row_offset<D>(row, t, N, lane_off);
      const bool in = t < n;      // slack entries past the list weigh nothing
      x1[u] = in ? w1[t] : 0.0f;
      x2[u] = in ? w2[t] : 0.0f;
      v1[u] = *reinterpret_cast<const uint4*>(b1 + o);
      v2[u] = *reinterpret_cast<const uint4*>(b2 + o);
    }
#pragma unroll
    for (int u = 0; u < kPair; ++u) {
      if (u >= nu) break;
      add(v1[u], x1[u], acc1);
      add(v2[u], x2[u], acc2);
    }
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc1[e] = o == 32 ? sum_xor32(acc1[e]) : o == 16 ? sum_xor16(acc1[e])
                                                       : acc1[e] + __shfl_xor(acc1[e], o, kWave);
      acc2[e] = o == 32 ? sum_xor32(acc2[e]) : o == 16 ? sum_xor16(acc2[e])
                                                       : acc2[e] + __shfl_xor(acc2[e], o, kWave);
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const int32_t* __restrict__ idx, int k, int N, float scale,
    float out_scale, float* __restrict__ dQ, float2* __restrict__ lpd,
    float4* __restrict__ stats, int* __restrict__ err) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int SL = gather_slog_floats(k);
  float* sl = bwd_lds + w * bwd_row_wave_floats(k);      // logits
  float* sd = sl + SL;                                    // dp_t
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const int h = blockIdx.y;
  const int q = blockIdx.x * kWaves + w;
  if (q >= N) return;
  const size_t hN = static_cast<size_t>(h) * N;
  stage_entries(idx + (hN + q) * k, 0, k, sidx);
  int bad = 0;
  // dp_t = dO·V_t first (V rows), then one pass over the K rows
  logits<T, D>(dO + (hN + q) * D, V + hN * D, sidx, 0, k, N, 1.0f, sd, bad);
  wave_sync();
  float m, S, U, A[EPL], B[EPL];
  bwd_logits_online<T, D>(Q + (hN + q) * D, K + hN * D, sidx, k, N, scale * kLog2e, sl, sd, bad,
                          m, S, U, A, B);
  if (bad) atomicOr(err, 1);
  wave_sync();
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  // (logit, dp_t) in idx's layout and the row's (max, 1/S, delta): the fill
  // forms p_t and dl_t from them (entries that name no key are never read)
  float2* er = lpd + (hN + q) * static_cast<size_t>(k);
  for (int t = l; t < k; t += kWave) er[t] = make_float2(sl[t], sd[t]);
  float acc[EPL];
  if (m == -INFINITY) {    // no valid entry: no gradient from this row
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    if (g == 0) store_f32_row<EPL>(dQ + (hN + q) * D + e0, acc, 1.0f);
    if (l == 0) stats[hN + q] = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
    return;
  }
  const float inv = 1.0f / S;
  const float delta = U * inv;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = (A[e] - delta * B[e]) * inv;
  if (g == 0) store_f32_row<EPL>(dQ + (hN + q) * D + e0, acc, out_scale);
  if (l == 0) stats[hN + q] = make_float4(m, inv, delta, 0.0f);
}

// Row pass, part r of a key-range split (see bwd.hip): the entries of the
// row whose keys lie in [bounds[r], bounds[r+1]) -- one segment of a row
// whose valid entries are an ascending prefix, else the whole row with the
// other keys masked -- give (logit, dp_t) in idx's layout and the part's
// record (m, S, U, -, A[D], B[D]).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const int32_t* __restrict__ idx, const int* __restrict__ seg,
    const int* __restrict__ bounds, int k, int N, float scale, float2* __restrict__ lpd,
    float* __restrict__ part) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL, R = kGatherRanges, PS = 2 * D + 4;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  // consecutive workgroups land on consecutive XCDs: part r runs on XCD r
  const int r = static_cast<int>(blockIdx.x) % R;
  const int q = static_cast<int>(blockIdx.x) / R * kWaves + w;
  const int h = blockIdx.y;
  if (q >= N) return;
  const int SL = gather_slog_floats(k);
  float* sl = bwd_lds + w * bwd_row_wave_floats(k);
  float* sd = sl + SL;
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const size_t hN = static_cast<size_t>(h) * N, row = hN + q;
  const int* sg = seg + row * (R + 1);
  const bool sorted = __builtin_amdgcn_readfirstlane(sg[0]) >= 0;
  const int t0 = sorted ? __builtin_amdgcn_readfirstlane(sg[r]) : 0;
  const int t1 = sorted ? __builtin_amdgcn_readfirstlane(sg[r + 1]) : k;
  float* rec = part + (row * R + r) * PS;
  if (t0 >= t1) {
    if (l == 0) rec[0] = -INFINITY;   // empty part: the merge skips it
    return;
  }
  const int lo = bounds[h * (R + 1) + r], hi = bounds[h * (R + 1) + r + 1];
  const int32_t* ir = idx + row * k;
  const int n = t1 - t0;
  for (int t = l; t < n; t += kWave) {
    const int j = ir[t0 + t];
    sidx[t] = j >= lo && j < hi ? j : -1;
  }
  wave_sync();
  float m, S, U, A[EPL], B[EPL];
  if constexpr (sizeof(T) == 2) {
    if (sorted) {   // the segment's keys all lie in [lo, hi): trusted rows
      logits_bf16_split<D>(dO + row * D, V + hN * D, sidx, n, N, 1.0f, sd);
      wave_sync();
      bwd_logits_online_trusted<D>(Q + row * D, K + hN * D, sidx, n, N, scale * kLog2e, sl, sd, m,
                                   S, U, A, B);
    }
  }
  if (sizeof(T) != 2 || !sorted) {
    int bad = 0;
    logits<T, D>(dO + row * D, V + hN * D, sidx, 0, n, N, 1.0f, sd, bad);
    wave_sync();
    bwd_logits_online<T, D>(Q + row * D, K + hN * D, sidx, n, N, scale * kLog2e, sl, sd, bad, m,
                            S, U, A, B);
  }
  wave_sync();
  float2* er = lpd + row * k + t0;
  for (int t = l; t < n; t += kWave)
    if (sidx[t] >= 0) er[t] = make_float2(sl[t], sd[t]);
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      *reinterpret_cast<float4*>(rec + 4 + e0 + e) = make_float4(A[e], A[e + 1], A[e + 2], A[e + 3]);
      *reinterpret_cast<float4*>(rec + 4 + D + e0 + e) =
          make_float4(B[e], B[e + 1], B[e + 2], B[e + 3]);
    }
  }
  if (l == 0) *reinterpret_cast<float4*>(rec) = make_float4(m, S, U, 0.0f);
}

// Key pass, part r: the key's records from rows of slices [r S/8, (r+1) S/8)
// (consecutive in its segment) give the part's dV[D] and H[D].  kWhich -1
// forms both at once (an entry's dO and Q rows loaded together); 0 forms dV
// from the dO rows and 1 forms H from the Q rows, in two launches, so that
// each XCD's L2 holds one row set of its part at a time instead of both
// (faster for the largest heads, whose part row sets outgrow the L2).
template <typename T, int D, int kWhich>
__global__ __launch_bounds__(kThreads) void bwd_keys_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ dO, const int* __restrict__ seg_off,
    const int* __restrict__ seg_cnt, const int* __restrict__ slice_pre, int S, long long total,
    const BwdEntry* __restrict__ rec, int N, int k, float* __restrict__ part) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL, R = kGatherRanges;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int r = static_cast<int>(blockIdx.x) % R;
  const int j = static_cast<int>(blockIdx.x) / R * kWaves + w;
  const int h = blockIdx.y;
  if (j >= N) return;
  constexpr int SL = gather_slog_floats(kBwdChunk);
  float* sp = bwd_lds + w * bwd_key_wave_floats();
  float* sd = sp + SL;
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const size_t hN = static_cast<size_t>(h) * N, key = hN + j;
  const int s0 = r * (S / R), s1 = (r + 1) * (S / R);
  const int a0 = slice_pre[static_cast<size_t>(s0) * total + key];
  const int a1 = s1 < S ? slice_pre[static_cast<size_t>(s1) * total + key] : seg_cnt[key];
  const size_t o0 = hN * static_cast<size_t>(k) + static_cast<unsigned>(seg_off[key] + a0);
  const int n = a1 - a0;
  const unsigned uk = static_cast<unsigned>(k);
  const T* Qh = Q + hN * D;
  const T* dOh = dO + hN * D;
  float av[EPL], ak[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) av[e] = ak[e] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kBwdChunk) {
    const int m = min(kBwdChunk, n - c0);
    for (int t = l; t < m; t += kWave) {
      const BwdEntry re = rec[o0 + c0 + t];
      sidx[t] = static_cast<int>(static_cast<unsigned>(re.e) / uk);
      sp[t] = re.p;
      sd[t] = re.dl;
    }
    wave_sync();
    // the rows are those of queries that kept the key: all in [0, N)
    float t1[EPL], t2[EPL];
    if constexpr (kWhich < 0 && sizeof(T) == 2) {
      weighted_rows2_bf16<D>(dOh, sp, Qh, sd, sidx, m, N, t1, t2);
    } else if constexpr (sizeof(T) == 2) {
      weighted_rows_bf16_split<D>(kWhich == 0 ? dOh : Qh, sidx, m, N, kWhich == 0 ? sp : sd, t1);
    } else {
      if constexpr (kWhich <= 0) weighted_rows<T, D>(dOh, sidx, 0, m, N, sp, t1);
      if constexpr (kWhich != 0) weighted_rows<T, D>(Qh, sidx, 0, m, N, sd, t2);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      if constexpr (kWhich < 0) {
        av[e] += t1[e];
        ak[e] += t2[e];
      } else if constexpr (kWhich == 0 || sizeof(T) == 2) {
        (kWhich == 0 ? av[e] : ak[e]) += t1[e];
      } else {
        ak[e] += t2[e];
      }
    }
    wave_sync();
  }
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  float* pr = part + (key * R + r) * 2 * D;
  if (g == 0) {
    if constexpr (kWhich <= 0) store_f32_row<EPL>(pr + e0, av, 1.0f);
    if constexpr (kWhich != 0) store_f32_row<EPL>(pr + D + e0, ak, 1.0f);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_keys_kernel(
    const T* __restrict__ Q, const T* __restrict__ dO, const int* __restrict__ seg_off,
    const int* __restrict__ seg_cnt, const BwdEntry* __restrict__ rec, int N, int k,
    float out_scale, float* __restrict__ dK, float* __restrict__ dV) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  constexpr int SL = gather_slog_floats(kBwdChunk);
  float* sp = bwd_lds + w * bwd_key_wave_floats();
  float* sd = sp + SL;
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const int h = blockIdx.y;
  const int j = blockIdx.x * kWaves + w;
  if (j >= N) return;
  const size_t hN = static_cast<size_t>(h) * N;
  const T* Qh = Q + hN * D;
  const T* dOh = dO + hN * D;
  const size_t o0 = hN * static_cast<size_t>(k) + static_cast<unsigned>(seg_off[hN + j]);
  const int n = seg_cnt[hN + j];
  const unsigned uk = static_cast<unsigned>(k);
  float av[EPL], ak[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) av[e] = ak[e] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kBwdChunk) {
    const int m = min(kBwdChunk, n - c0);
    for (int t = l; t < m; t += kWave) {
      const BwdEntry r = rec[o0 + c0 + t];
      sidx[t] = static_cast<int>(static_cast<unsigned>(r.e) / uk);   // e = i*k + t
      sp[t] = r.p;
      sd[t] = r.dl;
    }
    wave_sync();
    // the rows are those of queries that kept the key: all in [0, N)
    if constexpr (sizeof(T) == 2) {
      float t1[EPL], t2[EPL];
      weighted_rows2_bf16<D>(dOh, sp, Qh, sd, sidx, m, N, t1, t2);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        av[e] += t1[e];
        ak[e] += t2[e];
      }
    } else {
      float tmp[EPL];
      weighted_rows<T, D>(dOh, sidx, 0, m, N, sp, tmp);
#pragma unroll
      for (int e = 0; e < EPL; ++e) av[e] += tmp[e];
      weighted_rows<T, D>(Qh, sidx, 0, m, N, sd, tmp);
#pragma unroll
      for (int e = 0; e < EPL; ++e) ak[e] += tmp[e];
    }
    wave_sync();    // the chunk's LDS is read before the next one is staged
  }
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  if (g == 0) {
    store_f32_row<EPL>(dV + (hN + j) * D + e0, av, 1.0f);
    store_f32_row<EPL>(dK + (hN + j) * D + e0, ak, out_scale);
  }
}

template <typename T, int D>
hipError_t bwd_passes_t(const BwdArgs& a, hipStream_t s) {
  static std::atomic<int> lds_rows[kMaxDevices], lds_keys[kMaxDevices];
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_rows_kernel<T, D>),
                                    kWaves * bwd_row_wave_floats(kKMax) * 4, lds_rows);
  if (e != hipSuccess) return e;
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_keys_kernel<T, D>),
                         kWaves * bwd_key_wave_floats() * 4, lds_keys);
  if (e != hipSuccess) return e;
  static std::atomic<int> lds_rs[kMaxDevices], lds_ks[kMaxDevices];
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_rows_split_kernel<T, D>),
                         kWaves * bwd_row_wave_floats(kKMax) * 4, lds_rs);
  if (e != hipSuccess) return e;
  static std::atomic<int> lds_k0[kMaxDevices], lds_k1[kMaxDevices];
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_keys_split_kernel<T, D, -1>),
                         kWaves * bwd_key_wave_floats() * 4, lds_ks);
  if (e != hipSuccess) return e;
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_keys_split_kernel<T, D, 0>),
                         kWaves * bwd_key_wave_floats() * 4, lds_k0);
  if (e != hipSuccess) return e;
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_keys_split_kernel<T, D, 1>),
                         kWaves * bwd_key_wave_floats() * 4, lds_k1);
  if (e != hipSuccess) return e;
  int* err = nullptr;
  e = index_error_flag(&err);
  if (e != hipSuccess) return e;
  const int nb = (a.N + kWaves - 1) / kWaves;
  const dim3 grid(nb, a.nh), grid_split(nb * kGatherRanges, a.nh);
  const float out_scale = a.scorer ? 1.0f : a.scale;
  const size_t lds_r = static_cast<size_t>(kWaves) * bwd_row_wave_floats(a.k) * 4;
  const size_t lds_k = static_cast<size_t>(kWaves) * bwd_key_wave_floats() * 4;
  if (a.pass == 0 && !a.split_rows) {
    hipLaunchKernelGGL((bwd_rows_kernel<T, D>), grid, dim3(kThreads), lds_r, s,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                       static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.idx, a.k, a.N,
                       a.scale, out_scale, a.dQ, a.epd, a.stats, err);
  } else if (a.pass == 0) {
    hipLaunchKernelGGL((bwd_rows_split_kernel<T, D>), grid_split, dim3(kThreads), lds_r, s,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                       static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.idx,
                       a.row_seg, a.bounds, a.k, a.N, a.scale, a.epd, a.part);
  } else if (!a.split_keys) {
    hipLaunchKernelGGL((bwd_keys_kernel<T, D>), grid, dim3(kThreads), lds_k, s,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.dO), a.seg_off,
                       a.seg_cnt, a.rec, a.N, a.k, out_scale, a.dK, a.dV);
  } else {
    const long long args_total = static_cast<long long>(a.nh) * a.N;
    auto keys_split = [&](auto which) {
      hipLaunchKernelGGL((bwd_keys_split_kernel<T, D, decltype(which)::value>), grid_split,
                         dim3(kThreads), lds_k, s, static_cast<const T*>(a.Q),
                         static_cast<const T*>(a.dO), a.seg_off, a.seg_cnt, a.slice_pre,
                         a.slices, args_total, a.rec, a.N, a.k, a.part);
      return hipGetLastError();
    };
    if (a.keys_which == 0) return keys_split(std::integral_constant<int, 0>{});
    if (a.keys_which == 1) return keys_split(std::integral_constant<int, 1>{});
    return keys_split(std::integral_constant<int, -1>{});
  }
  return hipGetLastError();
}

}  // namespace

int bwd_slices(int N, int k) {
  const long long e = static_cast<long long>(N) * k;
  return static_cast<int>(std::min<long long>(16, std::max<long long>(1, e >> 20)));
}

namespace {
struct HistGrid {
  dim3 grid;
  int S, rows_per_slice;
  size_t lds;
};
HistGrid hist_grid(int nh, int N, int S) {
  HistGrid g;
  g.S = S;
  g.rows_per_slice = (N + g.S - 1) / g.S;
  const int nwin = (N + kHistWindow - 1) / kHistWindow;
  g.grid = dim3(g.S * nwin, nh);
  g.lds = static_cast<size_t>(std::min(N, kHistWindow)) * 4;
  return g;
}
}  // namespace

hipError_t launch_bwd_hist(const int32_t* idx, int nh, int N, int k, int S, int* cnt_s,
                           hipStream_t s) {
  static std::atomic<int> lds_set[kMaxDevices];
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_hist_kernel),
                                    kHistWindow * 4, lds_set);
  if (e != hipSuccess) return e;
  const HistGrid g = hist_grid(nh, N, S);
  hipLaunchKernelGGL(bwd_hist_kernel, g.grid, dim3(kHistThreads), g.lds, s, idx, N, k, g.S,
                     g.rows_per_slice, nh, cnt_s);
  return hipGetLastError();
}

hipError_t launch_bwd_slice_prefix(int* cnt_s, int S, long long total, int* cnt, hipStream_t s) {
  hipLaunchKernelGGL(bwd_slice_prefix_kernel, dim3(grid_for(total)), dim3(kThreads), 0, s, cnt_s,
                     S, total, cnt);
  return hipGetLastError();
}

hipError_t launch_bwd_scan(const int* cnt, int nh, int N, int* off, hipStream_t s) {
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(nh), dim3(kThreads), 0, s, cnt, N, off);
  return hipGetLastError();
}

hipError_t launch_bwd_fill(const int32_t* idx, const float2* lpd, const float4* stats, int nh,
                           int N, int k, int S, const int* cnt_s, const int* off, BwdEntry* rec,
                           hipStream_t s) {
  static std::atomic<int> lds_set[kMaxDevices];
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_fill_kernel),
                                    kHistWindow * 4, lds_set);
  if (e != hipSuccess) return e;
  const HistGrid g = hist_grid(nh, N, S);
  hipLaunchKernelGGL(bwd_fill_kernel, g.grid, dim3(kHistThreads), g.lds, s, idx, lpd, stats, N, k,
                     g.S, g.rows_per_slice, nh, cnt_s, off, rec);
  return hipGetLastError();
}

hipError_t launch_bwd_fill_parts(const int32_t* idx, const float2* lpd, const float4* stats,
                                 const int* row_seg, const int* bounds, int nh, int N, int k,
                                 int S, const int* cnt_s, const int* off, BwdEntry* rec,
                                 hipStream_t s) {
  static std::atomic<int> lds_set[kMaxDevices];
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_fill_parts_kernel),
                                    kHistWindow * 4, lds_set);
  if (e != hipSuccess) return e;
  const int rps = (N + S - 1) / S;
  hipLaunchKernelGGL(bwd_fill_parts_kernel, dim3(S * kGatherRanges, nh), dim3(kHistThreads),
                     static_cast<size_t>(kHistWindow) * 4, s, idx, lpd, stats, row_seg, bounds,
                     N, k, S, rps, nh, cnt_s, off, rec);
  return hipGetLastError();
}

hipError_t launch_bwd_bounds(const int* off, const int* cnt, int nh, int N, int* bounds,
                             hipStream_t s) {
  hipLaunchKernelGGL(bwd_bounds_kernel, dim3(nh), dim3(kWave), 0, s, off, cnt, N, bounds);
  return hipGetLastError();
}

hipError_t launch_bwd_row_ranges(const int32_t* idx, const int* bounds, int nh, int N, int k,
                                 int* seg, hipStream_t s) {
  const dim3 grid((N + kThreads / kWave - 1) / (kThreads / kWave), nh);
  hipLaunchKernelGGL(bwd_row_ranges_kernel, grid, dim3(kThreads), 0, s, idx, bounds, N, k, seg);
  return hipGetLastError();
}

hipError_t launch_bwd_rows_merge(const float* part, int nh, int N, int D, float out_scale,
                                 float* dQ, float4* stats, hipStream_t s) {
  const dim3 grid((N + kThreads / kWave - 1) / (kThreads / kWave), nh);
  if (D == 128)
    hipLaunchKernelGGL(bwd_rows_merge_kernel<128>, grid, dim3(kThreads), 0, s, part, N, out_scale,
                       dQ, stats);
  else if (D == 64)
    hipLaunchKernelGGL(bwd_rows_merge_kernel<64>, grid, dim3(kThreads), 0, s, part, N, out_scale,
                       dQ, stats);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_keys_merge(const float* part, int nh, int N, int D, float out_scale,
                                 float* dK, float* dV, hipStream_t s) {
  const dim3 grid((N + kThreads / kWave - 1) / (kThreads / kWave), nh);
  hipLaunchKernelGGL(bwd_keys_merge_kernel, grid, dim3(kThreads), 0, s, part, N, D, out_scale, dK,
                     dV);
  return hipGetLastError();
}

hipError_t launch_rows_times_pt(const float* lo, const void* P, int dtype, long long rows, int D,
                                int dp, float pre, float* out, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return rows_pt_d<float, 64>(lo, P, rows, dp, pre, out, s);
    if (D == 128) return rows_pt_d<float, 128>(lo, P, rows, dp, pre, out, s);
  } else {
    if (D == 64) return rows_pt_d<bf16_t, 64>(lo, P, rows, dp, pre, out, s);
    if (D == 128) return rows_pt_d<bf16_t, 128>(lo, P, rows, dp, pre, out, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rows_times_p(const float* X, const void* P, int dtype, long long rows, int D,
                               int dp, float alpha, float* out, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return rows_p_d<float, 64>(X, P, rows, dp, alpha, out, s);
    if (D == 128) return rows_p_d<float, 128>(X, P, rows, dp, alpha, out, s);
  } else {
    if (D == 64) return rows_p_d<bf16_t, 64>(X, P, rows, dp, alpha, out, s);
    if (D == 128) return rows_p_d<bf16_t, 128>(X, P, rows, dp, alpha, out, s);
  }
  return hipErrorInvalidValue;
}

int outer_sum_chunks(long long rows) {
  return static_cast<int>((rows + kOuterRows - 1) / kOuterRows);
}

hipError_t launch_outer_sum(const void* X, int dtype, const float* lo, long long rows, int D,
                            int dp, float* partial, int nchunks, float* dP, hipStream_t s) {
  hipError_t e = hipErrorInvalidValue;
  if (dtype == 0) {
    if (D == 64) e = outer_d<float, 64>(X, lo, rows, dp, partial, nchunks, s);
    if (D == 128) e = outer_d<float, 128>(X, lo, rows, dp, partial, nchunks, s);
  } else {
    if (D == 64) e = outer_d<bf16_t, 64>(X, lo, rows, dp, partial, nchunks, s);
    if (D == 128) e = outer_d<bf16_t, 128>(X, lo, rows, dp, partial, nchunks, s);
  }
  if (e != hipSuccess) return e;
  const int n = D * dp;
  hipLaunchKernelGGL(outer_reduce_kernel, dim3((n + kThreads - 1) / kThreads), dim3(kThreads), 0,
                     s, partial, nchunks, n, dP);
  return hipGetLastError();
}

// Heads of more than 2^23 row elements (N > 65536 at D = 128) take dV and H
// in two launches (128K: 87 -> 78 ms for the pair), smaller ones in one (32K:
// 10.2 against 12.5 ms, 64K causal: 36.3 against 39.2 ms).
bool bwd_keys_two_launches(int N, int D) {
  return static_cast<long long>(N) * D > (1ll << 23);
}

hipError_t launch_bwd_pass(const BwdArgs& a, hipStream_t s) {
  if (a.dtype == 0) {
    if (a.D == 64) return bwd_passes_t<float, 64>(a, s);
    if (a.D == 128) return bwd_passes_t<float, 128>(a, s);
  } else {
    if (a.D == 64) return bwd_passes_t<bf16_t, 64>(a, s);
    if (a.D == 128) return bwd_passes_t<bf16_t, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
