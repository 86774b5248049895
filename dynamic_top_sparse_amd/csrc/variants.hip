// Index variants that feed the same gather attention:
//  - a dilated window wrapped around the sequence (page
//    "Attention机制优化：原理、挑战与工程实践", §3.3: offsets t·dilation for
//    t < window, taken modulo the sequence length);
//  - a band whose radius is chosen per batch sample (page
//    "nxmr.cn/news/163144", §6 adaptive attention: the window size is a
//    per-sample value the model computes);
//  - boundary smoothing of the top-k (page "mhpq.cn/news/1098205", §4.2:
//    when the k-th and (k+1)-th scores are closer than a threshold, both
//    keys are kept).
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

// Grid-stride over every entry of idx [heads][N][k].
__global__ void dilated_kernel(long long total, int N, int window, int dilation,
                               int32_t* __restrict__ idx, int k) {
  for (long long e = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(e % k);
    const int i = static_cast<int>((e / k) % N);
    // (i + t * dilation) mod N without overflow: both terms reduced first
    const long long off = (static_cast<long long>(t) * dilation) % N;
    const int j = static_cast<int>((i + off) % N);
    idx[e] = t < window ? j : -1;
  }
}

__global__ void band_batch_kernel(long long total, int H, int N, const int32_t* __restrict__ radii,
                                  int32_t* __restrict__ idx, int k) {
  for (long long e = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(e % k);
    const long long row = e / k;
    const int i = static_cast<int>(row % N);
    const int b = static_cast<int>(row / N / H);
    const int w = max(0, radii[b]);            // a negative radius is taken as 0
    const int lo = max(0, i - w);
    const int hi = static_cast<int>(min(static_cast<long long>(N) - 1, static_cast<long long>(i) + w));
    const int j = lo + t;
    idx[e] = j <= hi ? j : -1;
  }
}

unsigned grid_for(long long total) {
  long long blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return static_cast<unsigned>(blocks);
}

// Boundary smoothing of top-(k+1) rows, one wavefront per query.  A row
// with k+1 keys holds the best k+1 by (s descending, key ascending), where s
// is the selection's exact fp32 score (exact_score()).  The two worst of
// them by that order are the k-th and the (k+1)-th; the (k+1)-th stays when
// s_k - s_(k+1) < gap, the difference taken in double precision (exact for
// two fp32 values), else it is removed and the row closes up.
constexpr int kSmoothWaves = kThreads / kWave;

__device__ __forceinline__ unsigned long long smooth_rank(float s, int j) {
  return (static_cast<unsigned long long>(order_key(s)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(j));
}

__device__ __forceinline__ unsigned long long wave_min64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long u = __shfl_xor(v, o, kWave);
    v = u < v ? u : v;
  }
  return v;
}

template <int DP>
__global__ __launch_bounds__(kThreads) void smooth_kernel(const float* __restrict__ q32,
                                                          const float* __restrict__ k32, int N,
                                                          int Npad, int k1, int causal,
                                                          float scale, double gap,
                                                          int32_t* __restrict__ idx) {
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  const int q = blockIdx.x * kSmoothWaves + w;
  const int h = blockIdx.y;
  if (q >= N) return;
  const int n_valid = causal ? q + 1 : N;
  if (n_valid < k1) return;          // at most k keys: nothing to smooth
  const size_t hq = static_cast<size_t>(h) * Npad;
  int32_t* row = idx + (static_cast<size_t>(h) * N + q) * k1;
  const float* qrow = q32 + (hq + q) * DP;
  // Exact scores of the row's keys, G lanes per key holding four
  // coordinates each (group_sum adds their partials in exact_score's fixed
  // order, so the values are those of the dump); lane 0 of each group keeps
  // the two smallest rank keys it has seen (worst first).
  constexpr int G = DP / 4, KPI = kWave / G, U = 8;
  const int g = l % G, grp = l / G;
  const float4 qv = reinterpret_cast<const float4*>(qrow)[g];
  unsigned long long m1 = ~0ull, m2 = ~0ull;
  for (int t0 = 0; t0 < k1; t0 += KPI * U) {
    float4 kv[U];
    int jj[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * KPI + grp;
      jj[u] = t < k1 ? row[t] : -1;
      kv[u] = jj[u] >= 0 ? reinterpret_cast<const float4*>(k32 + (hq + jj[u]) * DP)[g]
                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = group_sum<G>(group_partial<DP>(qv, kv[u]));
      if (g == 0 && jj[u] >= 0) {
        const unsigned long long r = smooth_rank(p * scale, jj[u]);
        if (r < m1) {
          m2 = m1;
          m1 = r;
        } else if (r < m2) {
          m2 = r;
        }
      }
    }
  }
  const unsigned long long w1 = wave_min64(m1);
  // second smallest overall: the smallest of every lane's best that is not
  // w1, and of the lane holding w1's runner-up
  const unsigned long long w2 = wave_min64(m1 == w1 ? m2 : m1);
  const float s_next = key_to_float(static_cast<uint32_t>(w1 >> 32));
  const float s_kth = key_to_float(static_cast<uint32_t>(w2 >> 32));
  if (static_cast<double>(s_kth) - static_cast<double>(s_next) < gap) return;
  const int drop = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(w1 & 0xFFFFFFFFull));
  // close the row up over the dropped key: entries are ascending, so those
  // after it move one place left; each chunk is read before it is written
  // and a write never reaches the next chunk
  for (int t0 = 0; t0 < k1; t0 += kWave) {
    const int t = t0 + l;
    const int j = t < k1 ? row[t] : -1;
    const bool after = t < k1 && j > drop;
    __builtin_amdgcn_wave_barrier();
    if (after) row[t - 1] = j;
  }
  if (l == 0) row[k1 - 1] = -1;
}

template <int DP>
hipError_t smooth_t(const Plan& p, const Bufs& b, int nh, float scale, float gap, int32_t* idx,
                    hipStream_t s) {
  const dim3 grid((p.N + kSmoothWaves - 1) / kSmoothWaves, nh);
  hipLaunchKernelGGL((smooth_kernel<DP>), grid, dim3(kThreads), 0, s, b.qlo32, b.klo32, p.N,
                     p.Npad, p.k, p.causal, scale, static_cast<double>(gap), idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dilated(int nheads, int N, int window, int dilation, int32_t* idx, int k,
                          hipStream_t s) {
  const long long total = static_cast<long long>(nheads) * N * k;
  hipLaunchKernelGGL(dilated_kernel, dim3(grid_for(total)), dim3(kThreads), 0, s, total, N,
                     window, dilation, idx, k);
  return hipGetLastError();
}

hipError_t launch_band_batch(int B, int H, int N, const int32_t* radii, int32_t* idx, int k,
                             hipStream_t s) {
  const long long total = static_cast<long long>(B) * H * N * k;
  hipLaunchKernelGGL(band_batch_kernel, dim3(grid_for(total)), dim3(kThreads), 0, s, total, H, N,
                     radii, idx, k);
  return hipGetLastError();
}

hipError_t launch_smooth(const Plan& p, const Bufs& b, int nh, float score_scale, float gap,
                         int32_t* idx_chunk, hipStream_t s) {
  switch (p.dp) {
    case 16: return smooth_t<16>(p, b, nh, score_scale, gap, idx_chunk, s);
    case 32: return smooth_t<32>(p, b, nh, score_scale, gap, idx_chunk, s);
    case 64: return smooth_t<64>(p, b, nh, score_scale, gap, idx_chunk, s);
    case 128: return smooth_t<128>(p, b, nh, score_scale, gap, idx_chunk, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
