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

// One workgroup of 1024 threads per head: the k_i-th largest order key by a
// radix select (four 8-bit digits; each wave counts into its own LDS
// histogram, so the LDS atomics of different waves never meet), then the
// keys above it and the lowest-index ties, in ascending key order.
__global__ __launch_bounds__(kSelThreads) void decode_select_kernel(
    const float* __restrict__ scores, int len, int k, int32_t* __restrict__ idx,
    int32_t* __restrict__ counts, int Ncap) {
  __shared__ int hist[kSelWaves][256];
  __shared__ int tmp[kSelWaves];
  __shared__ int wcnt[kSelWaves][2];
  __shared__ int s_digit, s_above;
  const int tid = threadIdx.x;
  const int wv = tid / kWave;
  const int h = blockIdx.x;
  const float* row = scores + static_cast<size_t>(h) * Ncap;
  const int k_i = min(k, len);
  uint32_t prefix = 0, pmask = 0;
  int K = k_i;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < kSelWaves * 256; b += kSelThreads) (&hist[0][0])[b] = 0;
    __syncthreads();
    // kSelLoads scores in flight per thread before their histogram updates
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
        if (j < len && (key & pmask) == prefix) atomicAdd(&hist[wv][(key >> shift) & 255], 1);
      }
    }
    __syncthreads();
    // thread t < 256 owns bin 255 - t (the sum of the waves' counts)
    int cval = 0;
    if (tid < 256) {
      for (int v = 0; v < kSelWaves; ++v) cval += hist[v][255 - tid];
    }
    int total;
    const int excl = block_excl_scan(cval, tmp, total);
    if (tid < 256 && excl < K && excl + cval >= K) {
      s_digit = 255 - tid;
      s_above = excl;
    }
    __syncthreads();
    K -= s_above;
    prefix |= static_cast<uint32_t>(s_digit) << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // K is now the number of ties with the k_i-th key that are kept (the
  // lowest indices).  One coalesced pass in tiles of kSelThreads keys: each
  // key's rank among the ties and its output position come from ballots
  // within the wave and the earlier waves' counts.
  const int ties_needed = K;
  int32_t* out = idx + static_cast<size_t>(h) * k;
  int32_t* cnt = counts != nullptr ? counts + static_cast<size_t>(h) * Ncap : nullptr;
  const int lane = lane_id();
  const unsigned long long below = (1ull << lane) - 1ull;
  int run_sel = 0, run_eq = 0;
  for (int b0 = 0; b0 < len; b0 += kSelThreads) {
    const int j = b0 + tid;
    const uint32_t key = j < len ? order_key(row[j]) : 0u;
    const bool eq = j < len && key == prefix;
    const bool gt = j < len && key > prefix;
    const unsigned long long me = __ballot(eq);
    if (lane == 0) wcnt[wv][0] = __popcll(me);
    __syncthreads();
    int eq_before = run_eq, eq_tile = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      const int c = wcnt[i][0];
      eq_before += i < wv ? c : 0;
      eq_tile += c;
    }
    const bool sel = gt || (eq && eq_before + __popcll(me & below) < ties_needed);
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
      out[pos + __popcll(ms & below)] = j;
      if (cnt != nullptr) atomicAdd(&cnt[j], 1);
    }
    run_eq += eq_tile;
    run_sel += sel_tile;
    __syncthreads();    // wcnt is rewritten by the next tile
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
  hipLaunchKernelGGL(decode_select_kernel, dim3(nh), dim3(kSelThreads), 0, s, scores, len, k, idx,
                     counts, Ncap);
  return hipGetLastError();
}

}  // namespace sa
