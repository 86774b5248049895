// Decode: one new query per (b, h) against the keys cached so far (page
// "mhpq.cn/news/1098205", §3.4: at inference the selection runs per
// generated token over the KV cache, and the keys' selection counts can
// decide which cache entries to keep; page "Attention机制优化：原理、挑战与
// 工程实践", §4.3: a preallocated cache updated in place).
//
// The scorer's key projections live in a caller-owned k_low cache, filled by
// the same projection kernel as the prefill (so a key's k_low is bit for bit
// the prefill's).  A step then
//   1. projects the query (same kernel again),
//   2. scores every cached key exactly (exact_score's arithmetic: the lanes
//      of a group hold four coordinates each and add their partials in the
//      fixed butterfly order), a memory-bound pass over the k_low cache,
//   3. selects the top-k of those scores per head (radix select on the
//      order keys, ties to the lower key index, written ascending),
//   4. runs the gather attention over the selected K and V cache rows.
// With the cache holding keys 0..len-1 of a sequence, the step's index row
// is exactly the causal prefill's row len-1.
//
// A step has one query per head, so each stage is spread over many
// workgroups per head: the scores in slices of the cache, each slice adding
// its keys' leading 11-bit order-key bins to the head's histogram; the
// keys at or above the bin that holds the head's k-th largest score are
// collected per slice; one workgroup per head finishes the select over
// those few keys; the attention runs in eight parts of the index row.
#include <algorithm>
#include <mutex>

#include "rows.h"

namespace sa {

// Device-resident workspace of sparse_attn_decode_noalloc, for callers that
// cannot allocate (code under graph capture, tight serving loops).  Each GPU
// the library runs on holds its own copy until the process ends; host code
// reaches it only through the address hipGetSymbolAddress reports for the
// current device (the array's name is not a device address on the host).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

// The current device's copy of `scratch`, looked up once per device.
hipError_t decode_scratch(void** out) {
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(mu);
    p = ptrs[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      ptrs[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kScoreUnroll = 16;  // key loads in flight per lane
constexpr int kSelThreads = 1024; // the final select: one big workgroup per head
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelLoads = 8;      // score loads in flight per thread in the fallback
constexpr int kSelTopBits = 11;   // first digit: sign, exponent, 2 mantissa bits
static_assert((1 << kSelTopBits) == kDecodeHistBins, "histogram bins");
constexpr int kSelCap = 8192;     // collected keys the final select keeps in LDS
constexpr int kSelMaxSlices = 4096;
// final select LDS: keys and indices (kSelCap each), the second digits'
// histogram, the slices' prefix counts
constexpr size_t kSelLds = (2 * static_cast<size_t>(kSelCap) + 2048 + kSelMaxSlices + 1) * 4;

__global__ void decode_clear_kernel(uint32_t* __restrict__ hist, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    hist[i] = 0u;
}

// Workgroup (slice, head): scores of keys [slice * kDecodeSliceKeys, ...)
// and their leading-bin counts (an LDS histogram, then one global add per
// non-empty bin).
template <int DP>
__global__ __launch_bounds__(kThreads) void decode_score_kernel(
    const float* __restrict__ qlo, int q_stride, const float* __restrict__ klow, int Ncap,
    int len, float scale, float* __restrict__ scores, uint32_t* __restrict__ hist) {
  constexpr int G = DP / 4;           // lanes per key, four coordinates each
  constexpr int KPI = kWave / G;      // keys per pass of a wave
  constexpr int PER_WAVE = KPI * kScoreUnroll;
  static_assert(kDecodeSliceKeys % (kWaves * PER_WAVE) == 0, "slice of whole passes");
  __shared__ uint32_t lh[kDecodeHistBins];
  for (int b = threadIdx.x; b < kDecodeHistBins; b += kThreads) lh[b] = 0u;
  __syncthreads();
  const int h = blockIdx.y;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const int g = l % G, grp = l / G;
  const float4 qv = reinterpret_cast<const float4*>(qlo + static_cast<size_t>(h) * q_stride * DP)[g];
  const float* kh = klow + static_cast<size_t>(h) * Ncap * DP;
  float* out = scores + static_cast<size_t>(h) * Ncap;
  const int js = blockIdx.x * kDecodeSliceKeys;
  const int je = min(len, js + kDecodeSliceKeys);
  for (int j0 = js + w * PER_WAVE; j0 < je; j0 += kWaves * PER_WAVE) {
    float4 kv[kScoreUnroll];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int j = j0 + u * KPI + grp;
      kv[u] = j < je ? reinterpret_cast<const float4*>(kh + static_cast<size_t>(j) * DP)[g]
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const float p = group_sum<G>(group_partial<DP>(qv, kv[u]));
      const int j = j0 + u * KPI + grp;
      if (g == 0 && j < je) {
        const float v = p * scale;
        out[j] = v;
        atomicAdd(&lh[order_key(v) >> (32 - kSelTopBits)], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* hh = hist + static_cast<size_t>(h) * kDecodeHistBins;
  for (int b = threadIdx.x; b < kDecodeHistBins; b += kThreads) {
    const uint32_t c = lh[b];
    if (c != 0u) atomicAdd(&hh[b], c);
  }
}

// Exclusive scan of one int per thread over a workgroup of NW waves.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int w = threadIdx.x / kWave, l = lane_id();
  const int incl = wave_incl_scan(v);
  if (l == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < NW; ++i) {
    const int t = tmp[i];
    if (i < w) off += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + incl - v;
}

// The bin holding the K-th largest key, bins nb-1 .. 0 in descending key
// order with counts cnt(b), nb = BPT * (threads of the workgroup): thread t
// owns bins nb-1-BPT*t down to nb-BPT-BPT*t.  *s_digit = the bin, *s_above =
// keys in higher bins (1 <= K <= the total count).
template <int NW, int BPT, typename Cnt>
__device__ __forceinline__ void pick_bin(int nb, int K, Cnt cnt, int* tmp, int* s_digit,
                                         int* s_above) {
  const int top = nb - 1 - BPT * static_cast<int>(threadIdx.x);
  int c[BPT];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    c[i] = top - i >= 0 ? cnt(top - i) : 0;
    mine += c[i];
  }
  int total;
  const int excl = block_excl_scan<NW>(mine, tmp, total);
  if (excl < K && excl + mine >= K) {
    int run = excl;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (run < K && run + c[i] >= K) {
        *s_digit = top - i;
        *s_above = run;
      }
      run += c[i];
    }
  }
  __syncthreads();
}

// Workgroup (slice, head): the slice's keys whose leading bin is at or above
// the bin of the head's k_i-th largest score, in index order, as (order key,
// index) pairs; the slice's full count goes to ccount (entries past
// kDecodeCandCap are dropped, and the final select then works over the
// scores instead).  Slice 0 also records the bin and the keys above it.
__global__ __launch_bounds__(kThreads) void decode_collect_kernel(
    const float* __restrict__ scores, int Ncap, int len, int k, const uint32_t* __restrict__ hist,
    uint2* __restrict__ cand, int* __restrict__ ccount, int2* __restrict__ selinfo) {
  __shared__ int tmp[kWaves];
  __shared__ int wcnt[kWaves];
  __shared__ int s_digit, s_above;
  const int h = blockIdx.y, s = blockIdx.x, nsl = gridDim.x;
  const int tid = threadIdx.x, wv = tid / kWave, lane = lane_id();
  const int k_i = min(k, len);
  const uint32_t* hh = hist + static_cast<size_t>(h) * kDecodeHistBins;
  pick_bin<kWaves, kDecodeHistBins / kThreads>(
      kDecodeHistBins, k_i, [&](int b) { return static_cast<int>(hh[b]); }, tmp, &s_digit,
      &s_above);
  const uint32_t B1 = static_cast<uint32_t>(s_digit);
  const float* row = scores + static_cast<size_t>(h) * Ncap;
  const int js = s * kDecodeSliceKeys, je = min(len, js + kDecodeSliceKeys);
  constexpr int kTiles = kDecodeSliceKeys / kThreads;
  float v[kTiles];
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    const int j = js + u * kThreads + tid;
    v[u] = j < je ? row[j] : 0.0f;
  }
  uint2* out = cand + (static_cast<size_t>(h) * nsl + s) * kDecodeCandCap;
  const unsigned long long below = (1ull << lane) - 1ull;
  int run = 0;
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    const int j = js + u * kThreads + tid;
    const uint32_t key = order_key(v[u]);
    const bool take = j < je && (key >> (32 - kSelTopBits)) >= B1;
    const unsigned long long ms = __ballot(take);
    if (lane == 0) wcnt[wv] = __popcll(ms);
    __syncthreads();
    int pos = run, tile = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int c = wcnt[i];
      pos += i < wv ? c : 0;
      tile += c;
    }
    pos += __popcll(ms & below);
    if (take && pos < kDecodeCandCap) out[pos] = make_uint2(key, static_cast<uint32_t>(j));
    run += tile;
    __syncthreads();    // wcnt is rewritten by the next tile
  }
  if (tid == 0) {
    ccount[static_cast<size_t>(h) * nsl + s] = run;
    if (s == 0) selinfo[h] = make_int2(s_digit, s_above);
  }
}

// Writes, in ascending key order, the keys of `key(e)` (e = 0 .. n-1, in
// index order, index `at(e)`) above T and the first `ties` equal to T: one
// coalesced pass in tiles of kSelThreads, each key's rank among the ties and
// its output position from ballots within the wave and the earlier waves'
// counts.
template <typename KeyAt, typename IdxAt>
__device__ __forceinline__ void write_selected(int n, uint32_t T, int ties, KeyAt key, IdxAt at,
                                               int32_t* out, int32_t* cnt,
                                               int (*wcnt)[2]) {
  const int tid = threadIdx.x, wv = tid / kWave, lane = lane_id();
  const unsigned long long below = (1ull << lane) - 1ull;
  int run_sel = 0, run_eq = 0;
  for (int b0 = 0; b0 < n; b0 += kSelThreads) {
    const int e = b0 + tid;
    const uint32_t x = e < n ? key(e) : 0u;
    const bool eq = e < n && x == T;
    const bool gt = e < n && x > T;
    const unsigned long long me = __ballot(eq);
    if (lane == 0) wcnt[wv][0] = __popcll(me);
    __syncthreads();
    int eq_before = run_eq, eq_tile = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      const int c = wcnt[i][0];
      eq_before += i < wv ? c : 0;
      eq_tile += c;
    }
    const bool sel = gt || (eq && eq_before + static_cast<int>(__popcll(me & below)) < ties);
    const unsigned long long ms = __ballot(sel);
    if (lane == 0) wcnt[wv][1] = __popcll(ms);
    __syncthreads();
    int pos = run_sel, sel_tile = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      const int c = wcnt[i][1];
      pos += i < wv ? c : 0;
      sel_tile += c;
    }
    if (sel) {
      const int j = at(e);
      out[pos + __popcll(ms & below)] = j;
      if (cnt != nullptr) atomicAdd(&cnt[j], 1);
    }
    run_eq += eq_tile;
    run_sel += sel_tile;
    __syncthreads();    // wcnt is rewritten by the next tile
  }
}

// One workgroup of 1024 threads per head finishes the select of the top k_i
// of the head's len scores (ties to the lower key index) and writes them
// ascending, then -1.  Normally over the collected keys: the slices' pairs,
// in slice order (so in index order), into LDS; the two remaining digits of
// the order key (11 and 10 bits) below the first one the collect step fixed,
// then the output.  If a slice overflowed or more than kSelCap keys were
// collected, a radix select with four 8-bit digits over the scores in memory
// instead.
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(
    const float* __restrict__ scores, int len, int k, const uint2* __restrict__ cand,
    const int* __restrict__ ccount, const int2* __restrict__ selinfo, int32_t* __restrict__ idx,
    int32_t* __restrict__ counts, int Ncap) {
  extern __shared__ __align__(16) uint32_t sel_lds[];
  __shared__ int tmp[kSelWaves];
  __shared__ int wcnt[kSelWaves][2];
  __shared__ int s_digit, s_above, s_over;
  const int tid = threadIdx.x;
  const int wv = tid / kWave;
  const int h = blockIdx.x;
  const float* row = scores + static_cast<size_t>(h) * Ncap;
  int32_t* out = idx + static_cast<size_t>(h) * k;
  int32_t* cnt = counts != nullptr ? counts + static_cast<size_t>(h) * Ncap : nullptr;
  const int k_i = min(k, len);
  const int nsl = decode_slices(len);
  uint32_t* lkey = sel_lds;
  int* lidx = reinterpret_cast<int*>(sel_lds + kSelCap);
  uint32_t* h2 = sel_lds + 2 * kSelCap;
  int* pre = reinterpret_cast<int*>(h2 + 2048);     // [nsl + 1] prefix counts
  // ---- the slices' counts: prefix sums, overflow
  if (tid == 0) s_over = nsl > kSelMaxSlices ? 1 : 0;
  __syncthreads();
  int M = 0;
  if (s_over == 0) {
    const int* cc = ccount + static_cast<size_t>(h) * nsl;
    int run = 0;
    for (int b0 = 0; b0 < nsl; b0 += kSelThreads) {
      const int sl = b0 + tid;
      const int c = sl < nsl ? cc[sl] : 0;
      if (c > kDecodeCandCap) s_over = 1;
      int tot;
      const int ex = block_excl_scan<kSelWaves>(c, tmp, tot);
      if (sl < nsl) pre[sl] = run + ex;
      run += tot;
    }
    if (tid == 0) pre[nsl] = run;
    M = run;
    __syncthreads();
  }
  const bool fast = s_over == 0 && M <= kSelCap;
  int K;
  uint32_t prefix, pmask;
  if (fast) {
    const int2 si = selinfo[h];
    K = k_i - si.y;                  // keys still to take from the first bin
    const uint2* hc = cand + static_cast<size_t>(h) * nsl * kDecodeCandCap;
    for (int e = tid; e < M; e += kSelThreads) {
      int lo = 0, hi = nsl - 1;      // the slice holding collected key e
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= e) lo = mid; else hi = mid - 1;
      }
      const uint2 c = hc[static_cast<size_t>(lo) * kDecodeCandCap + (e - pre[lo])];
      lkey[e] = c.x;
      lidx[e] = static_cast<int>(c.y);
    }
    __syncthreads();
    // ---- the two remaining digits (11 and 10 bits) over the kept keys
    prefix = static_cast<uint32_t>(si.x) << (32 - kSelTopBits);
    pmask = ~0u << (32 - kSelTopBits);
    for (int pass = 0; pass < 2; ++pass) {
      const int bits = pass == 0 ? 11 : 10, shift = pass == 0 ? 10 : 0, nb = 1 << bits;
      for (int b = tid; b < nb; b += kSelThreads) h2[b] = 0;
      __syncthreads();
      for (int e = tid; e < M; e += kSelThreads) {
        const uint32_t key = lkey[e];
        if ((key & pmask) == prefix) atomicAdd(&h2[(key >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      pick_bin<kSelWaves, 2>(nb, K, [&](int b) { return static_cast<int>(h2[b]); }, tmp,
                             &s_digit, &s_above);
      K -= s_above;
      prefix |= static_cast<uint32_t>(s_digit) << shift;
      pmask |= static_cast<uint32_t>(nb - 1) << shift;
      __syncthreads();
    }
    write_selected(M, prefix, K, [&](int e) { return lkey[e]; }, [&](int e) { return lidx[e]; },
                   out, cnt, wcnt);
  } else {
    // ---- four 8-bit digits over the scores (one LDS histogram per wave)
    int (*h8)[256] = reinterpret_cast<int (*)[256]>(sel_lds);
    prefix = 0;
    pmask = 0;
    K = k_i;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < kSelWaves * 256; b += kSelThreads) (&h8[0][0])[b] = 0;
      __syncthreads();
      for (int j0 = tid; j0 < len; j0 += kSelThreads * kSelLoads) {
        float v[kSelLoads];
#pragma unroll
        for (int u = 0; u < kSelLoads; ++u) {
          const int j = j0 + u * kSelThreads;
          v[u] = j < len ? row[j] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kSelLoads; ++u) {
          const int j = j0 + u * kSelThreads;
          const uint32_t key = order_key(v[u]);
          if (j < len && (key & pmask) == prefix) atomicAdd(&h8[wv][(key >> shift) & 255], 1);
        }
      }
      __syncthreads();
      pick_bin<kSelWaves, 1>(256, K, [&](int b) {
        int c = 0;
        for (int w = 0; w < kSelWaves; ++w) c += h8[w][b];
        return c;
      }, tmp, &s_digit, &s_above);
      K -= s_above;
      prefix |= static_cast<uint32_t>(s_digit) << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    write_selected(len, prefix, K, [&](int e) { return order_key(row[e]); },
                   [&](int e) { return e; }, out, cnt, wcnt);
  }
  for (int t = k_i + tid; t < k; t += kSelThreads) out[t] = -1;
}

// One wave per (head, part): the attention partial of entries
// [r k_i / R, (r + 1) k_i / R) of the head's index row (all keys < len), as
// the forward's split gather writes it: (max, sum, -, -, unnormalised acc).
template <typename T, int D, bool kTrusted>
__global__ __launch_bounds__(kThreads) void decode_gather_part_kernel(
    const T* __restrict__ q, const T* __restrict__ Kc, const T* __restrict__ Vc,
    const int32_t* __restrict__ idx, int k, int k_i, int nh, int Ncap, float scale,
    float* __restrict__ part) {
  constexpr int EPL = Vec<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int R = kGatherRanges;
  constexpr int SL = gather_slog_floats(kKMax / R + 16);
  __shared__ float slog_all[kWaves * 2 * SL];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int gid = static_cast<int>(blockIdx.x) * kWaves + w;
  const int h = gid / R, r = gid % R;
  if (h >= nh) return;
  float* slog = slog_all + w * 2 * SL;
  int* sidx = reinterpret_cast<int*>(slog + SL);
  const int s0 = r * k_i / R, s1 = (r + 1) * k_i / R;
  float* rec = part + (static_cast<size_t>(h) * R + r) * (D + 4);
  if (s0 >= s1) {
    if (l == 0) rec[0] = -INFINITY;   // empty: the merge skips it
    return;
  }
  const T* Kh = Kc + static_cast<size_t>(h) * Ncap * D;
  const T* Vh = Vc + static_cast<size_t>(h) * Ncap * D;
  const T* qrow = q + static_cast<size_t>(h) * D;
  stage_entries(idx + static_cast<size_t>(h) * k, s0, s1, sidx);
  if constexpr (kTrusted) {
    logits_bf16_split<D>(qrow, Kh, sidx, s1 - s0, Ncap, scale * kLog2e, slog);
  } else {
    int bad = 0;
    logits<T, D>(qrow, Kh, sidx, s0, s1, Ncap, scale * kLog2e, slog, bad);
  }
  wave_sync();
  float sum;
  const float mx = softmax_weights(slog, s1 - s0, sum);
  wave_sync();
  float acc[EPL];
  if constexpr (kTrusted)
    weighted_rows_bf16_split<D>(Vh, sidx, s1 - s0, Ncap, slog, acc);
  else
    weighted_rows<T, D>(Vh, sidx, s0, s1, Ncap, slog, acc);
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  if (g == 0) {
    float4* dst = reinterpret_cast<float4*>(rec + 4 + e0);
#pragma unroll
    for (int e = 0; e < EPL; e += 4) dst[e / 4] = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
  if (l == 0) {
    rec[0] = mx;
    rec[1] = sum;
  }
}

// One wave per head: O = sum_r 2^(m_r - M) acc_r / sum_r 2^(m_r - M) l_r.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_gather_merge_kernel(
    const float* __restrict__ part, int nh, T* __restrict__ O) {
  constexpr int R = kGatherRanges;
  constexpr int EPM = D / kWave;
  const int w = threadIdx.x / kWave, l = lane_id();
  const int h = blockIdx.x * kWaves + w;
  if (h >= nh) return;
  const float* recs = part + static_cast<size_t>(h) * R * (D + 4);
  float m = -INFINITY, lsum = 0.0f;
  if (l < R) {
    m = recs[static_cast<size_t>(l) * (D + 4)];
    if (m != -INFINITY) lsum = recs[static_cast<size_t>(l) * (D + 4) + 1];
  }
  const float M = wave_max(m);
  T* out = O + static_cast<size_t>(h) * D + l * EPM;
  float acc[EPM];
#pragma unroll
  for (int e = 0; e < EPM; ++e) acc[e] = 0.0f;
  if (M != -INFINITY) {
    const float wr = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    const float L = wave_sum(wr * lsum);
    for (int r = 0; r < R; ++r) {
      const float wv = __shfl(wr, r, kWave);
      if (wv != 0.0f) {
        const float* a = recs + static_cast<size_t>(r) * (D + 4) + 4 + l * EPM;
#pragma unroll
        for (int e = 0; e < EPM; ++e) acc[e] = __builtin_fmaf(wv, a[e], acc[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < EPM; ++e) acc[e] /= L;
  }
#pragma unroll
  for (int e = 0; e < EPM; ++e) out[e] = io<T>::from_f32(acc[e]);
}

template <int DP>
hipError_t scores_t(const float* qlo, int q_stride, const float* klow, int Ncap, int len, int nh,
                    float scale, float* scores, uint32_t* hist, hipStream_t s) {
  const dim3 grid(decode_slices(len), nh);
  hipLaunchKernelGGL((decode_score_kernel<DP>), grid, dim3(kThreads), 0, s, qlo, q_stride, klow,
                     Ncap, len, scale, scores, hist);
  return hipGetLastError();
}

template <typename T, int D, bool kTrusted>
hipError_t gather_part_t(const void* q, const void* Kc, const void* Vc, const int32_t* idx, int k,
                         int len, int nh, int Ncap, float scale, float* part, hipStream_t s) {
  const int waves = nh * kGatherRanges;
  hipLaunchKernelGGL((decode_gather_part_kernel<T, D, kTrusted>),
                     dim3((waves + kWaves - 1) / kWaves), dim3(kThreads), 0, s,
                     static_cast<const T*>(q), static_cast<const T*>(Kc),
                     static_cast<const T*>(Vc), idx, k, std::min(k, len), nh, Ncap, scale, part);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t gather_merge_t(const float* part, int nh, void* O, hipStream_t s) {
  hipLaunchKernelGGL((decode_gather_merge_kernel<T, D>), dim3((nh + kWaves - 1) / kWaves),
                     dim3(kThreads), 0, s, part, nh, static_cast<T*>(O));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_clear(uint32_t* hist, int nh, hipStream_t s) {
  const int n = nh * kDecodeHistBins;
  const int blocks = std::min((n + 255) / 256, 1024);
  hipLaunchKernelGGL(decode_clear_kernel, dim3(blocks), dim3(256), 0, s, hist, n);
  return hipGetLastError();
}

hipError_t launch_decode_scores(const float* qlo, int q_stride, const float* klow, int Ncap,
                                int len, int nh, int dp, float scale, float* scores,
                                uint32_t* hist, hipStream_t s) {
  switch (dp) {
    case 16: return scores_t<16>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, hist, s);
    case 32: return scores_t<32>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, hist, s);
    case 64: return scores_t<64>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, hist, s);
    case 128: return scores_t<128>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, hist, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_collect(const float* scores, int Ncap, int len, int nh, int k,
                                 const uint32_t* hist, uint2* cand, int* ccount, int2* selinfo,
                                 hipStream_t s) {
  hipLaunchKernelGGL(decode_collect_kernel, dim3(decode_slices(len), nh), dim3(kThreads), 0, s,
                     scores, Ncap, len, k, hist, cand, ccount, selinfo);
  return hipGetLastError();
}

hipError_t launch_decode_select(const float* scores, int len, int nh, int k, const uint2* cand,
                                const int* ccount, const int2* selinfo, int32_t* idx,
                                int32_t* counts, int Ncap, hipStream_t s) {
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&decode_select_kernel),
                                          static_cast<int>(kSelLds), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_select_kernel, dim3(nh), dim3(kSelThreads), kSelLds, s, scores, len,
                     k, cand, ccount, selinfo, idx, counts, Ncap);
  return hipGetLastError();
}

hipError_t launch_decode_gather_part(const void* q, const void* Kc, const void* Vc,
                                     const int32_t* idx, int k, int len, int nh, int Ncap, int D,
                                     float softmax_scale, int dtype, float* part, hipStream_t s) {
  // bf16 rows are read as trusted (every entry below k_i is a key < len) when
  // a head's cache rows fit 32-bit byte offsets
  const bool trusted = static_cast<long long>(Ncap) * D * 2 < (1ll << 32);
  if (dtype == 0) {
    if (D == 64) return gather_part_t<float, 64, false>(q, Kc, Vc, idx, k, len, nh, Ncap, softmax_scale, part, s);
    if (D == 128) return gather_part_t<float, 128, false>(q, Kc, Vc, idx, k, len, nh, Ncap, softmax_scale, part, s);
  } else if (trusted) {
    if (D == 64) return gather_part_t<bf16_t, 64, true>(q, Kc, Vc, idx, k, len, nh, Ncap, softmax_scale, part, s);
    if (D == 128) return gather_part_t<bf16_t, 128, true>(q, Kc, Vc, idx, k, len, nh, Ncap, softmax_scale, part, s);
  } else {
    if (D == 64) return gather_part_t<bf16_t, 64, false>(q, Kc, Vc, idx, k, len, nh, Ncap, softmax_scale, part, s);
    if (D == 128) return gather_part_t<bf16_t, 128, false>(q, Kc, Vc, idx, k, len, nh, Ncap, softmax_scale, part, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_gather_merge(const float* part, int nh, int D, int dtype, void* O,
                                      hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return gather_merge_t<float, 64>(part, nh, O, s);
    if (D == 128) return gather_merge_t<float, 128>(part, nh, O, s);
  } else {
    if (D == 64) return gather_merge_t<bf16_t, 64>(part, nh, O, s);
    if (D == 128) return gather_merge_t<bf16_t, 128>(part, nh, O, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
