// Exact re-rank of the filter's candidates, and the exact fallback.
//
// The selection rule (page "mhpq.cn/news/1098205", §3.2: torch.topk over the
// scores, masked keys excluded first, all keys kept when fewer than k are
// valid) is applied to the exact fp32 score s of exact_score().  Ties go to
// the lower key index; rows are written in ascending key order, then -1.
//
// Re-rank, one wavefront per query.  Each candidate carries its bf16 MFMA
// score s~; with the per-query margin m every exact score lies in
// [l, u] = [s~ - m, s~ + m] (rounded outwards).  Let lo be the k-th largest l
// and hi the (k+1)-th largest u (or tau if larger).  Then
//   u < lo   -> the key is certainly out (its exact score is below the k-th),
//   l > hi   -> certainly in (at most k-1 other keys can reach its score),
// and only the remaining "uncertain" keys are re-scored exactly, in fp32,
// and ranked by (s descending, key ascending) to fill the rest of the row.
// The candidate list of each query half is already in ascending key order
// (the filter streams keys in order), so the output row is a merge.
#include <float.h>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;   // fallback workgroup

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// K-th largest (1-based) of the keys key(i), i in [0, n) with ok(i), by an
// MSB-first radix select with 8-bit digits over a wave-private histogram.
// Requires 1 <= K <= number of admitted keys.
template <typename KeyT, typename KeyFn>
__device__ KeyT wave_kth_largest(int n, int K, int* hist, KeyFn key_of) {
  const int l = lane_id();
  KeyT prefix = 0, pmask = 0;
  constexpr int kBits = 8 * sizeof(KeyT);
  for (int shift = kBits - 8; shift >= 0; shift -= 8) {
    for (int b = l; b < 256; b += kWave) hist[b] = 0;
    wave_sync();
    for (int i = l; i < n; i += kWave) {
      KeyT key;
      if (key_of(i, key) && (key & pmask) == prefix)
        atomicAdd(&hist[static_cast<int>((key >> shift) & 255)], 1);
    }
    wave_sync();
    // lane L owns bins 255-4L .. 252-4L (descending)
    int c[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = hist[255 - 4 * l - t];
    const int s = c[0] + c[1] + c[2] + c[3];
    const int incl = wave_incl_scan(s);
    const unsigned long long crossing = __ballot(incl >= K);
    const int F = crossing ? __builtin_ctzll(crossing) : 0;
    int digit = 0, above = 0;
    if (l == F) {
      int cum = incl - s;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (cum + c[t] >= K) { digit = 255 - 4 * l - t; break; }
        cum += c[t];
      }
      above = cum;
    }
    digit = __shfl(digit, F, kWave);
    above = __shfl(above, F, kWave);
    K -= above;
    prefix |= static_cast<KeyT>(digit) << shift;
    pmask |= static_cast<KeyT>(255) << shift;
    wave_sync();
  }
  return prefix;
}

// First position in the ascending list a[0..n) whose value is >= x.
__device__ __forceinline__ int lower_bound(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

template <int DP>
__global__ __launch_bounds__(kThreads) void finalize_kernel(
    const uint2* __restrict__ cand, const int* __restrict__ cnt, const float* __restrict__ tau,
    const float2* __restrict__ qstat, const uint32_t* __restrict__ kstat,
    const float* __restrict__ q32, const float* __restrict__ k32, int N, int Npad, int k,
    int causal, int capH, float scale, int32_t* __restrict__ idx, int* __restrict__ fblist,
    WsHeader* __restrict__ hdr) {
  extern __shared__ unsigned char smem[];
  const int wpb = blockDim.x / kWave;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const int cap = 2 * capH;
  // per-wave LDS: keys, scores, class, histogram, q row
  unsigned char* base = smem + static_cast<size_t>(w) * (cap * 9 + 256 * 4 + DP * 4);
  int* cj = reinterpret_cast<int*>(base);
  float* cs = reinterpret_cast<float*>(base + cap * 4);
  int* hist = reinterpret_cast<int*>(base + cap * 8);
  float* qrow = reinterpret_cast<float*>(base + cap * 8 + 1024);
  unsigned char* cls = base + cap * 8 + 1024 + DP * 4;

  const int h = blockIdx.y;
  const int q = blockIdx.x * wpb + w;
  if (q >= N) return;
  const size_t hq = static_cast<size_t>(h) * Npad;
  int32_t* out = idx + (static_cast<size_t>(h) * N + q) * k;
  const int n_valid = causal ? q + 1 : N;
  const int k_i = min(k, n_valid);

  if (n_valid <= k) {  // every valid key is kept
    for (int t = l; t < k; t += kWave) out[t] = t < n_valid ? t : -1;
    if (l == 0) atomicAdd(&hdr->queries, 1ull);
    return;
  }
  const int c0 = cnt[(hq + q) * 2], c1 = cnt[(hq + q) * 2 + 1];
  const float tq = tau[hq + q];
  if (c0 > capH || c1 > capH) {
    if (l == 0) {
      const unsigned slot = atomicAdd(&hdr->fb_count, 1u);
      fblist[slot] = static_cast<int>(hq + q);
      atomicAdd(&hdr->overflow_queries, 1ull);
      atomicAdd(&hdr->queries, 1ull);
    }
    return;
  }
  const int c = c0 + c1;
  const uint2* list0 = cand + (hq + q) * 2 * static_cast<size_t>(capH);
  const uint2* list1 = list0 + capH;
  for (int i = l; i < c; i += kWave) {
    const uint2 e = i < c0 ? list0[i] : list1[i - c0];
    cj[i] = static_cast<int>(e.x);
    cs[i] = __uint_as_float(e.y) * scale;
  }
  for (int t = l; t < DP; t += kWave) qrow[t] = q32[(hq + q) * DP + t];
  wave_sync();

  const float2 st = qstat[hq + q];
  const float m = score_margin(st.x, st.y, __uint_as_float(kstat[2 * h]),
                               __uint_as_float(kstat[2 * h + 1]), scale);
  auto lower = [&](float s) { return (s - m) - (fabsf(s) + m) * (1.0f / 4194304.0f); };
  auto upper = [&](float s) { return (s + m) + (fabsf(s) + m) * (1.0f / 4194304.0f); };

  // the threshold is proven to lie below the k-th best exact score only if
  // k candidates have a lower bound >= tau
  int ok_cnt = 0;
  for (int i = l; i < c; i += kWave) ok_cnt += lower(cs[i]) >= tq ? 1 : 0;
  ok_cnt = wave_sum_i(ok_cnt);
  if (ok_cnt < k_i) {
    if (l == 0) {
      const unsigned slot = atomicAdd(&hdr->fb_count, 1u);
      fblist[slot] = static_cast<int>(hq + q);
      atomicAdd(&hdr->queries, 1ull);
    }
    return;
  }

  const uint32_t lo_key = wave_kth_largest<uint32_t>(c, k_i, hist, [&](int i, uint32_t& key) {
    key = order_key(lower(cs[i]));
    return true;
  });
  const float lo = key_to_float(lo_key);
  float hi = tq;
  if (c >= k_i + 1) {
    const uint32_t hi_key = wave_kth_largest<uint32_t>(c, k_i + 1, hist, [&](int i, uint32_t& key) {
      key = order_key(upper(cs[i]));
      return true;
    });
    hi = fmaxf(hi, key_to_float(hi_key));
  }

  // classify; re-score the uncertain band exactly
  int n_in = 0, n_unc = 0;
  for (int i = l; i < c; i += kWave) {
    const float s = cs[i];
    unsigned char k_cls;
    if (lower(s) > hi) {
      k_cls = 1;
      ++n_in;
    } else if (upper(s) < lo) {
      k_cls = 0;
    } else {
      k_cls = 2;
      ++n_unc;
      cs[i] = exact_score<DP>(qrow, k32 + (hq + cj[i]) * DP, scale);
    }
    cls[i] = k_cls;
  }
  n_in = wave_sum_i(n_in);
  n_unc = wave_sum_i(n_unc);
  wave_sync();
  const int need = k_i - n_in;
  if (need > n_unc) {
    // cannot happen when the margins hold; resolve the query exactly anyway
    if (l == 0) {
      const unsigned slot = atomicAdd(&hdr->fb_count, 1u);
      fblist[slot] = static_cast<int>(hq + q);
      atomicAdd(&hdr->queries, 1ull);
    }
    return;
  }
  unsigned long long kth = ~0ull;
  if (need > 0) {
    kth = wave_kth_largest<unsigned long long>(c, need, hist, [&](int i, unsigned long long& key) {
      if (cls[i] != 2) return false;
      key = (static_cast<unsigned long long>(order_key(cs[i])) << 32) |
            static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(cj[i]));
      return true;
    });
  }
  // Compact the kept keys of each half, in key order, into `sel` (the score
  // array, reused): half 0 fills sel[0, n0), half 1 fills sel[n0, n0 + n1).
  // A write never passes the chunk being read, and the wave syncs between
  // reading a chunk's scores and overwriting them.
  int* sel = reinterpret_cast<int*>(cs);
  int run = 0, n0 = 0;
  for (int i0 = 0; i0 < c; i0 += kWave) {
    const int i = i0 + l;
    int take = 0, key = 0;
    if (i < c) {
      key = cj[i];
      if (cls[i] == 1) {
        take = 1;
      } else if (cls[i] == 2 && need > 0) {
        const unsigned long long k64 =
            (static_cast<unsigned long long>(order_key(cs[i])) << 32) |
            static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(key));
        take = k64 >= kth ? 1 : 0;
      }
    }
    const int incl = wave_incl_scan(take);
    const int first_half = (i < c0 && take) ? 1 : 0;
    n0 += wave_sum_i(first_half);
    wave_sync();
    if (take) sel[run + incl - 1] = key;
    run += __shfl(incl, kWave - 1, kWave);
    wave_sync();
  }
  const int n1 = run - n0;
  // merge the two ascending lists into the output row
  for (int p = l; p < n0; p += kWave) out[p + lower_bound(sel + n0, n1, sel[p])] = sel[p];
  for (int p = l; p < n1; p += kWave) out[p + lower_bound(sel, n0, sel[n0 + p])] = sel[n0 + p];
  for (int t = run + l; t < k; t += kWave) out[t] = -1;
  if (l == 0) {
    atomicAdd(&hdr->rescored, static_cast<unsigned long long>(n_unc));
    atomicAdd(&hdr->queries, 1ull);
  }
}

// ------------------------------------------------------------ fallback ---
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int w = threadIdx.x / kWave, l = lane_id();
  const int incl = wave_incl_scan(v);
  if (l == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < kWavesPerBlock; ++i) {
    const int t = tmp[i];
    if (i < w) off += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + incl - v;
}

// Exact selection for queued queries: score every valid key exactly into a
// per-workgroup scratch row, find the k-th largest score by radix select,
// and write keys above it plus the lowest-index ties, in ascending order.
// Persistent: each workgroup takes queued queries until the queue is empty.
template <int DP>
__global__ __launch_bounds__(kThreads) void fallback_kernel(
    const float* __restrict__ q32, const float* __restrict__ k32, const int* __restrict__ fblist,
    int N, int Npad, int k, int causal, float scale, float* __restrict__ scratch,
    int32_t* __restrict__ idx, WsHeader* __restrict__ hdr) {
  __shared__ float qrow[DP];
  __shared__ int hist[256];
  __shared__ int tmp[kWavesPerBlock];
  __shared__ int s_item, s_digit, s_above;
  const int tid = threadIdx.x;
  const unsigned n_items = hdr->fb_count;
  float* row = scratch + static_cast<size_t>(blockIdx.x) * Npad;
  for (;;) {
    __syncthreads();
    if (tid == 0) s_item = static_cast<int>(atomicAdd(&hdr->fb_next, 1u));
    __syncthreads();
    const int item = s_item;
    if (item >= static_cast<int>(n_items)) break;
    const int entry = fblist[item];
    const int h = entry / Npad, q = entry % Npad;
    const size_t hq = static_cast<size_t>(h) * Npad;
    const int n_valid = causal ? q + 1 : N;
    const int k_i = min(k, n_valid);
    if (tid < DP) qrow[tid] = q32[(hq + q) * DP + tid];
    __syncthreads();
    for (int j = tid; j < n_valid; j += kThreads)
      row[j] = exact_score<DP>(qrow, k32 + (hq + j) * DP, scale);
    __syncthreads();
    // k_i-th largest order key
    uint32_t prefix = 0, pmask = 0;
    int K = k_i;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < n_valid; j += kThreads) {
        const uint32_t key = order_key(row[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      const int cval = hist[255 - tid];   // thread t owns bin 255 - t
      int total;
      const int excl = block_excl_scan(cval, tmp, total);
      if (excl < K && excl + cval >= K) {
        s_digit = 255 - tid;
        s_above = excl;
      }
      __syncthreads();
      K -= s_above;
      prefix |= static_cast<uint32_t>(s_digit) << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    // keys strictly above the k-th score, then ties in ascending key order
    int gt = 0;
    for (int j = tid; j < n_valid; j += kThreads) gt += order_key(row[j]) > prefix ? 1 : 0;
    int gt_total;
    block_excl_scan(gt, tmp, gt_total);
    const int ties_needed = k_i - gt_total;
    int32_t* out = idx + (hq / Npad * static_cast<size_t>(N) + q) * k;
    int run_take = 0, run_eq = 0;
    for (int j0 = 0; j0 < n_valid; j0 += kThreads) {
      const int j = j0 + tid;
      const uint32_t key = j < n_valid ? order_key(row[j]) : 0u;
      const int is_eq = (j < n_valid && key == prefix) ? 1 : 0;
      int eq_total;
      const int eq_before = run_eq + block_excl_scan(is_eq, tmp, eq_total);
      const int take = (j < n_valid && (key > prefix || (is_eq && eq_before < ties_needed))) ? 1 : 0;
      int take_total;
      const int pos = run_take + block_excl_scan(take, tmp, take_total);
      if (take) out[pos] = j;
      run_take += take_total;
      run_eq += eq_total;
    }
    for (int t = k_i + tid; t < k; t += kThreads) out[t] = -1;
    if (tid == 0) atomicAdd(&hdr->fallback_queries, 1ull);
  }
}

template <int DP>
hipError_t finalize_t(const Plan& p, const Bufs& b, int nh, float scale, int32_t* idx,
                      hipStream_t s) {
  // as many waves (queries) per workgroup as the per-wave LDS allows
  const size_t per_wave = static_cast<size_t>(2 * p.capH) * 9 + 1024 + DP * 4;
  int wpb = static_cast<int>((160 * 1024) / per_wave);
  wpb = wpb < 1 ? 1 : (wpb > 4 ? 4 : wpb);
  const dim3 grid((p.N + wpb - 1) / wpb, nh);
  const size_t lds = static_cast<size_t>(wpb) * per_wave;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&finalize_kernel<DP>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((finalize_kernel<DP>), grid, dim3(wpb * kWave), lds, s, b.cand, b.cnt, b.tau,
                     b.qstat, b.kstat, b.qlo32, b.klo32, p.N, p.Npad, p.k, p.causal, p.capH,
                     scale, idx, b.fblist, b.hdr);
  return hipGetLastError();
}

template <int DP>
hipError_t fallback_t(const Plan& p, const Bufs& b, float scale, int32_t* idx, hipStream_t s) {
  hipLaunchKernelGGL((fallback_kernel<DP>), dim3(kFallbackBlocks), dim3(kThreads), 0, s,
                     b.qlo32, b.klo32, b.fblist, p.N, p.Npad, p.k, p.causal, scale,
                     b.fbscratch, idx, b.hdr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_finalize(const Plan& p, const Bufs& b, int nh, float score_scale,
                           int32_t* idx_chunk, hipStream_t s) {
  switch (p.dp) {
    case 16: return finalize_t<16>(p, b, nh, score_scale, idx_chunk, s);
    case 32: return finalize_t<32>(p, b, nh, score_scale, idx_chunk, s);
    case 64: return finalize_t<64>(p, b, nh, score_scale, idx_chunk, s);
    case 128: return finalize_t<128>(p, b, nh, score_scale, idx_chunk, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fallback(const Plan& p, const Bufs& b, int nh, float score_scale,
                           int32_t* idx_chunk, hipStream_t s) {
  (void)nh;
  switch (p.dp) {
    case 16: return fallback_t<16>(p, b, score_scale, idx_chunk, s);
    case 32: return fallback_t<32>(p, b, score_scale, idx_chunk, s);
    case 64: return fallback_t<64>(p, b, score_scale, idx_chunk, s);
    case 128: return fallback_t<128>(p, b, score_scale, idx_chunk, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
