// Attention over per-query index sets, and band index sets.
//
// Gather-attention (page "mhpq.cn/news/1098205", §3.2: gather the selected K
// and V rows, matmul·scale, softmax, matmul; §1.2: softmax(QKᵀ/√d_k)V): for
// query i with index row idx_i,
//   logit_t = softmax_scale · q_i·K[idx_t],  w = softmax(logit) (max-subtracted),
//   O_i = Σ_t w_t V[idx_t],
// over the entries idx_t >= 0.  Logits, softmax and accumulation are fp32
// (page "Attention机制优化：原理、挑战与工程实践", §4.2: keep fp32 before the
// softmax).  Nothing is materialised: one wavefront per query streams the
// selected rows with 16-byte loads (a bf16 row of 128 is 16 lanes x 16 B, so
// one load instruction fetches 4 whole rows) and keeps its logits in LDS.
// The work is HBM/cache-bandwidth bound (~1 flop per byte), so the kernel is
// written for memory-level parallelism: several row loads in flight per
// lane, no MFMA.
//
// Band indices (page "Attention机制改进：稀疏注意力应用", create_local_mask:
// i-w <= j <= i+w; page "nxmr.cn/news/163144", §2.2): row i lists keys
// max(0, i-w_left) .. min(N-1, i+w_right), clipped at the ends, then -1.
#include "sa_internal.h"

namespace sa {

__device__ int g_index_error_flag = 0;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;   // row loads in flight per lane

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void unpack(uint4 v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <> struct Vec<bf16_t> {
  static constexpr int kElems = 8;
  __device__ __forceinline__ static void unpack(uint4 v, float (&f)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static uint4 pack(const float (&f)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, int k, int N, float scale, T* __restrict__ O) {
  constexpr int EPL = Vec<T>::kElems;                     // elements per lane
  constexpr int LPR = D / EPL;                            // lanes per row
  constexpr int RPI = kWave / LPR;                        // rows per load instruction
  extern __shared__ int smem[];
  const int w = threadIdx.x / kWave;
  const int l = lane_id();
  int* sidx = smem + static_cast<size_t>(w) * 2 * k;
  float* slog = reinterpret_cast<float*>(sidx + k);
  const int h = blockIdx.y;
  const int q = blockIdx.x * kWaves + w;
  if (q >= N) return;
  const size_t hN = static_cast<size_t>(h) * N;
  const T* Kh = K + hN * D;
  const T* Vh = V + hN * D;
  const int32_t* row = idx + (hN + q) * k;
  for (int t = l; t < k; t += kWave) sidx[t] = row[t];

  const int g = l / LPR;           // row group of this lane
  const int e0 = (l % LPR) * EPL;  // first element of this lane's slice
  float qv[EPL];
  Vec<T>::unpack(*reinterpret_cast<const uint4*>(Q + (hN + q) * D + e0), qv);
  wave_sync();

  int bad = 0;
  // logits
  for (int t0 = 0; t0 < k; t0 += RPI * kUnroll) {
    uint4 kv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * RPI + g;
      const int j = t < k ? sidx[t] : -1;
      ok[u] = j >= 0 && j < N;
      bad |= (t < k && j >= N) ? 1 : 0;
      kv[u] = ok[u] ? *reinterpret_cast<const uint4*>(Kh + static_cast<size_t>(j) * D + e0)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[EPL];
      Vec<T>::unpack(kv[u], kf);
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qv[e], kf[e], dot);
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
      const int t = t0 + u * RPI + g;
      if ((l % LPR) == 0 && t < k) slog[t] = ok[u] ? dot * scale : -INFINITY;
    }
  }
  wave_sync();
  float mx = -INFINITY;
  for (int t = l; t < k; t += kWave) mx = fmaxf(mx, slog[t]);
  mx = wave_max(mx);
  T* out = O + (hN + q) * D;
  if (bad) atomicOr(&g_index_error_flag, 1);
  if (mx == -INFINITY) {  // no valid entry: zero output
    float z[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) z[e] = 0.0f;
    if (g == 0) *reinterpret_cast<uint4*>(out + e0) = Vec<T>::pack(z);
    return;
  }
  float sum = 0.0f;
  for (int t = l; t < k; t += kWave) {
    const float x = slog[t];
    const float p = x == -INFINITY ? 0.0f : expf(x - mx);
    slog[t] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  wave_sync();

  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int t0 = 0; t0 < k; t0 += RPI * kUnroll) {
    uint4 vv[kUnroll];
    float wt[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = t0 + u * RPI + g;
      const int j = t < k ? sidx[t] : -1;
      const bool ok = j >= 0 && j < N;
      wt[u] = ok ? slog[t] : 0.0f;
      vv[u] = ok ? *reinterpret_cast<const uint4*>(Vh + static_cast<size_t>(j) * D + e0)
                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float vf[EPL];
      Vec<T>::unpack(vv[u], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(wt[u], vf[e], acc[e]);
    }
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += __shfl_xor(acc[e], o, kWave);
  }
  if (g == 0) {
    float r[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) r[e] = acc[e] / sum;
    *reinterpret_cast<uint4*>(out + e0) = Vec<T>::pack(r);
  }
}

__global__ void band_kernel(long long total, int N, int w_left, int w_right,
                            int32_t* __restrict__ idx, int k) {
  for (long long e = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int t = static_cast<int>(e % k);
    const int i = static_cast<int>((e / k) % N);
    const int lo = max(0, i - w_left);
    const int hi = min(N - 1, i + w_right);
    const int j = lo + t;
    idx[e] = j <= hi ? j : -1;
  }
}

template <typename T, int D>
hipError_t gather_t(const void* Q, const void* K, const void* V, const int32_t* idx, int k,
                    int nheads, int N, float scale, void* O, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kWaves) * 2 * k * sizeof(int);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gather_kernel<T, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(kWaves) * 2 * kKMax * 4);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid((N + kWaves - 1) / kWaves, nheads);
  hipLaunchKernelGGL((gather_kernel<T, D>), grid, dim3(kThreads), lds, s,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     idx, k, N, scale, static_cast<T*>(O));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const void* Q, const void* K, const void* V, const int32_t* idx, int k,
                         int nheads, int N, int D, float softmax_scale, int dtype, void* O,
                         hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return gather_t<float, 64>(Q, K, V, idx, k, nheads, N, softmax_scale, O, s);
    if (D == 128) return gather_t<float, 128>(Q, K, V, idx, k, nheads, N, softmax_scale, O, s);
  } else {
    if (D == 64) return gather_t<bf16_t, 64>(Q, K, V, idx, k, nheads, N, softmax_scale, O, s);
    if (D == 128) return gather_t<bf16_t, 128>(Q, K, V, idx, k, nheads, N, softmax_scale, O, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_band(int nheads, int N, int w_left, int w_right, int32_t* idx, int k,
                       hipStream_t s) {
  const long long total = static_cast<long long>(nheads) * N * k;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(band_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, total, N,
                     w_left, w_right, idx, k);
  return hipGetLastError();
}

hipError_t read_and_clear_device_flag(int* value, hipStream_t s) {
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  int v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_index_error_flag), sizeof(int), 0,
                          hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *value = v;
  if (v != 0) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_index_error_flag), &zero, sizeof(int), 0,
                          hipMemcpyHostToDevice);
  }
  return e;
}

}  // namespace sa
