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
#include <mutex>

#include "sa_internal.h"

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
constexpr int kScoreUnroll = 8;   // key loads in flight per lane
constexpr int kSelThreads = 1024; // the select kernel: one big workgroup per head
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelLoads = 8;      // score loads in flight per thread in the select

template <int DP>
__global__ __launch_bounds__(kThreads) void decode_score_kernel(
    const float* __restrict__ qlo, int q_stride, const float* __restrict__ klow, int Ncap,
    int len, float scale, float* __restrict__ scores) {
  constexpr int G = DP / 4;           // lanes per key, four coordinates each
  constexpr int KPI = kWave / G;      // keys per pass of a wave
  const int h = blockIdx.y;
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const int g = l % G, grp = l / G;
  const float4 qv = reinterpret_cast<const float4*>(qlo + static_cast<size_t>(h) * q_stride * DP)[g];
  const float* kh = klow + static_cast<size_t>(h) * Ncap * DP;
  float* out = scores + static_cast<size_t>(h) * Ncap;
  const int per_block = KPI * kWaves * kScoreUnroll;
  const int j0 = blockIdx.x * per_block + w * KPI * kScoreUnroll;
  float4 kv[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    const int j = j0 + u * KPI + grp;
    kv[u] = j < len ? reinterpret_cast<const float4*>(kh + static_cast<size_t>(j) * DP)[g]
                    : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    const float p = group_sum<G>(group_partial<DP>(qv, kv[u]));
    const int j = j0 + u * KPI + grp;
    if (g == 0 && j < len) out[j] = p * scale;
  }
}

__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int w = threadIdx.x / kWave, l = lane_id();
  const int incl = wave_incl_scan(v);
  if (l == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < kSelWaves; ++i) {
    const int t = tmp[i];
    if (i < w) off += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + incl - v;
}

constexpr int kSelTopBits = 11;                   // first digit: sign, exponent, 2 mantissa bits
constexpr int kSelTopBins = 1 << kSelTopBits;
constexpr int kSelCap = 8192;                     // keys kept in LDS after the first digit
constexpr size_t kSelLds = static_cast<size_t>(kSelWaves) * kSelTopBins * 4;   // 128 KB

// The bin holding the K-th largest key, bins nb-1 .. 0 in descending key
// order with counts cnt(b) (nb <= 2 * kSelThreads; thread t owns bins
// nb-1-2t and nb-2-2t): *s_digit = the bin, *s_above = keys in higher bins.
template <typename Cnt>
__device__ __forceinline__ void pick_bin(int nb, int K, Cnt cnt, int* tmp, int* s_digit,
                                         int* s_above) {
  const int bh = nb - 1 - 2 * static_cast<int>(threadIdx.x), bl = bh - 1;
  const int ch = bh >= 0 ? cnt(bh) : 0;
  const int cl = bl >= 0 ? cnt(bl) : 0;
  int total;
  const int excl = block_excl_scan(ch + cl, tmp, total);
  if (bh >= 0 && excl < K && excl + ch >= K) {
    *s_digit = bh;
    *s_above = excl;
  }
  if (bl >= 0 && excl + ch < K && excl + ch + cl >= K) {
    *s_digit = bl;
    *s_above = excl + ch;
  }
  __syncthreads();
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
    const bool sel = gt || (eq && eq_before + __popcll(me & below) < ties);
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

// One workgroup of 1024 threads per head selects the top k_i of the head's
// len scores (ties to the lower key index) and writes them ascending, then
// -1.  A radix select on the 32-bit order keys: the first digit (11 bits)
// from one pass over the scores, with one LDS histogram per wave so the
// LDS atomics of different waves never meet; a second pass keeps the keys
// at or above the k_i-th key's bin, in index order, in LDS (about 2 % of the
// keys at 128K), and the two remaining digits and the output run there.  If
// that bin holds too many keys, the select runs over the scores in memory
// with four 8-bit digits instead.
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(
    const float* __restrict__ scores, int len, int k, int32_t* __restrict__ idx,
    int32_t* __restrict__ counts, int Ncap) {
  extern __shared__ __align__(16) uint32_t sel_lds[];
  __shared__ int tmp[kSelWaves];
  __shared__ int wcnt[kSelWaves][2];
  __shared__ int s_digit, s_above;
  const int tid = threadIdx.x;
  const int wv = tid / kWave, lane = lane_id();
  const int h = blockIdx.x;
  const float* row = scores + static_cast<size_t>(h) * Ncap;
  int32_t* out = idx + static_cast<size_t>(h) * k;
  int32_t* cnt = counts != nullptr ? counts + static_cast<size_t>(h) * Ncap : nullptr;
  const int k_i = min(k, len);
  // ---- first digit over the scores
  uint32_t* hist = sel_lds;          // [kSelWaves][kSelTopBins]
  for (int b = tid; b < kSelWaves * kSelTopBins; b += kSelThreads) hist[b] = 0;
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
      if (j < len) atomicAdd(&hist[wv * kSelTopBins + (order_key(v[u]) >> (32 - kSelTopBits))], 1u);
    }
  }
  __syncthreads();
  pick_bin(kSelTopBins, k_i, [&](int b) {
    int c = 0;
    for (int w = 0; w < kSelWaves; ++w) c += static_cast<int>(hist[w * kSelTopBins + b]);
    return c;
  }, tmp, &s_digit, &s_above);
  const uint32_t B1 = static_cast<uint32_t>(s_digit);
  int K = k_i - s_above;             // keys still to take from bin B1
  // ---- the keys of bins >= B1, in index order
  uint32_t* lkey = sel_lds;
  int* lidx = reinterpret_cast<int*>(sel_lds + kSelCap);
  const unsigned long long below = (1ull << lane) - 1ull;
  int run = 0;
  for (int b0 = 0; b0 < len; b0 += kSelThreads) {
    const int j = b0 + tid;
    const uint32_t key = j < len ? order_key(row[j]) : 0u;
    const bool take = j < len && (key >> (32 - kSelTopBits)) >= B1;
    const unsigned long long ms = __ballot(take);
    if (lane == 0) wcnt[wv][0] = __popcll(ms);
    __syncthreads();
    int pos = run, tile = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      const int c = wcnt[i][0];
      pos += i < wv ? c : 0;
      tile += c;
    }
    pos += __popcll(ms & below);
    if (take && pos < kSelCap) {
      lkey[pos] = key;
      lidx[pos] = j;
    }
    run += tile;
    __syncthreads();
  }
  const int M = run;
  uint32_t prefix, pmask;
  if (M <= kSelCap) {
    // ---- the two remaining digits (11 and 10 bits) over the kept keys
    prefix = B1 << (32 - kSelTopBits);
    pmask = ~0u << (32 - kSelTopBits);
    uint32_t* h2 = sel_lds + 2 * kSelCap;
    for (int pass = 0; pass < 2; ++pass) {
      const int bits = pass == 0 ? 11 : 10, shift = pass == 0 ? 10 : 0, nb = 1 << bits;
      for (int b = tid; b < nb; b += kSelThreads) h2[b] = 0;
      __syncthreads();
      for (int e = tid; e < M; e += kSelThreads) {
        const uint32_t key = lkey[e];
        if ((key & pmask) == prefix) atomicAdd(&h2[(key >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      pick_bin(nb, K, [&](int b) { return static_cast<int>(h2[b]); }, tmp, &s_digit, &s_above);
      K -= s_above;
      prefix |= static_cast<uint32_t>(s_digit) << shift;
      pmask |= static_cast<uint32_t>(nb - 1) << shift;
      __syncthreads();
    }
    write_selected(M, prefix, K, [&](int e) { return lkey[e]; }, [&](int e) { return lidx[e]; },
                   out, cnt, wcnt);
  } else {
    // ---- too many keys in the bin: four 8-bit digits over the scores
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
      pick_bin(256, K, [&](int b) {
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

template <int DP>
hipError_t scores_t(const float* qlo, int q_stride, const float* klow, int Ncap, int len, int nh,
                    float scale, float* scores, hipStream_t s) {
  constexpr int KPI = kWave / (DP / 4);
  const int per_block = KPI * kWaves * kScoreUnroll;
  const dim3 grid((len + per_block - 1) / per_block, nh);
  hipLaunchKernelGGL((decode_score_kernel<DP>), grid, dim3(kThreads), 0, s, qlo, q_stride, klow,
                     Ncap, len, scale, scores);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_scores(const float* qlo, int q_stride, const float* klow, int Ncap,
                                int len, int nh, int dp, float scale, float* scores,
                                hipStream_t s) {
  switch (dp) {
    case 16: return scores_t<16>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, s);
    case 32: return scores_t<32>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, s);
    case 64: return scores_t<64>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, s);
    case 128: return scores_t<128>(qlo, q_stride, klow, Ncap, len, nh, scale, scores, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_select(const float* scores, int len, int nh, int k, int32_t* idx,
                                int32_t* counts, int Ncap, hipStream_t s) {
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&decode_select_kernel),
                                          kSelLds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_select_kernel, dim3(nh), dim3(kSelThreads), kSelLds, s, scores, len, k,
                     idx, counts, Ncap);
  return hipGetLastError();
}

}  // namespace sa
