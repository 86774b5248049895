// Scorer projection: q_low = Q·Pq and k_low = K·Pk for every row of a head
// chunk (page "mhpq.cn/news/1098205", §2.2: the scorer's q_proj / k_proj map
// each head's d_model-wide vectors to d_proj dimensions).
//
// Per row it writes the fp32 projection (accumulated with FMAs in ascending
// order of the model dimension, the fixed order every exact score relies
// on), its bf16 rounding for the MFMA filter, and two norms that bound the
// filter's error: ||x_low|| and ||x_low - bf16(x_low)||, both rounded up.
// Key rows also feed a per-head maximum of those norms and every 16th key
// row is copied to the threshold sample.  Rows N..Npad-1 are zero padding.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kRows = 64;       // rows per workgroup
constexpr int kThreads = 256;

// Round-up factor for norms computed in fp32 (covers the rounding of the
// sum of squares and of the square root).
constexpr float kNormUp = 1.0f + 1.0f / 65536.0f;

template <typename T, int D, int DP>
__global__ __launch_bounds__(kThreads) void project_kernel(
    const T* __restrict__ X, const T* __restrict__ P, int N, int Npad, int is_key,
    float* __restrict__ lo32, bf16_t* __restrict__ lo16, float2* __restrict__ stat,
    bf16_t* __restrict__ samp, uint32_t* __restrict__ kstat) {
  constexpr int kXFloats = kRows * (D + 1);
  constexpr int kLoFloats = 2 * kRows * (DP + 1);
  __shared__ float sP[D * DP];
  // the staged input rows are dead once accumulated, so the projected rows
  // and their bf16 residuals reuse that space
  __shared__ float sXLo[kXFloats > kLoFloats ? kXFloats : kLoFloats];
  __shared__ float sMax[2][kRows];
  float* sX = sXLo;
  float* sLo = sXLo;
  float* sRes = sXLo + kRows * (DP + 1);

  const int tid = threadIdx.x;
  const int h = blockIdx.y;                 // head within the chunk
  const int row0 = blockIdx.x * kRows;
  const T* Xh = X + static_cast<size_t>(h) * N * D;

  for (int e = tid; e < D * DP; e += kThreads) sP[e] = io<T>::to_f32(P[e]);
  for (int e = tid; e < kRows * D; e += kThreads) {
    const int r = e / D, d = e % D;
    const int row = row0 + r;
    sX[r * (D + 1) + d] = (row < N) ? io<T>::to_f32(Xh[static_cast<size_t>(row) * D + d]) : 0.0f;
  }
  __syncthreads();

  constexpr int kGroups = kThreads / DP;    // row groups
  constexpr int kRowsPerThread = kRows / kGroups;
  const int c = tid % DP;
  const int g = tid / DP;
  float acc[kRowsPerThread];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) acc[i] = 0.0f;
  for (int d = 0; d < D; ++d) {
    const float pv = sP[d * DP + c];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i)
      acc[i] = __builtin_fmaf(sX[(g + i * kGroups) * (D + 1) + d], pv, acc[i]);
  }
  const size_t base = static_cast<size_t>(h) * Npad;
  __syncthreads();  // every thread is done reading sX
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = g + i * kGroups;
    const int row = row0 + r;
    const float v = (row < N) ? acc[i] : 0.0f;
    const bf16_t vb = f32_to_bf16(v);
    lo32[(base + row) * DP + c] = v;
    lo16[(base + row) * DP + c] = vb;
    if (samp != nullptr && (row % kSampleStride) == 0)
      samp[(static_cast<size_t>(h) * (Npad / kSampleStride) + row / kSampleStride) * DP + c] = vb;
    sLo[r * (DP + 1) + c] = v;
    sRes[r * (DP + 1) + c] = v - bf16_to_f32(vb);
  }
  __syncthreads();
  if (tid < kRows) {
    float s2 = 0.0f, r2 = 0.0f;
    for (int cc = 0; cc < DP; ++cc) {
      const float a = sLo[tid * (DP + 1) + cc];
      const float b = sRes[tid * (DP + 1) + cc];
      s2 = __builtin_fmaf(a, a, s2);
      r2 = __builtin_fmaf(b, b, r2);
    }
    const float n = __builtin_sqrtf(s2) * kNormUp;
    const float rn = __builtin_sqrtf(r2) * kNormUp;
    if (stat != nullptr) stat[base + row0 + tid] = make_float2(n, rn);
    sMax[0][tid] = n;
    sMax[1][tid] = rn;
  }
  if (is_key) {
    __syncthreads();
    if (tid < 2) {
      float m = 0.0f;
      for (int r = 0; r < kRows; ++r) m = fmaxf(m, sMax[tid][r]);
      // non-negative floats order like their bit patterns
      atomicMax(&kstat[2 * h + tid], __float_as_uint(m));
    }
  }
}

__global__ void init_chunk_kernel(WsHeader* hdr, uint32_t* kstat, int nh, int first_chunk) {
  const int t = threadIdx.x;
  if (t == 0) {
    if (first_chunk) {
      hdr->fallback_queries = 0;
      hdr->overflow_queries = 0;
      hdr->candidates = 0;
      hdr->rescored = 0;
      hdr->queries = 0;
    }
    hdr->fb_count = 0;
    hdr->fb_next = 0;
  }
  for (int i = t; i < 2 * nh; i += blockDim.x) kstat[i] = 0u;
}

template <typename T, int D, int DP>
hipError_t project_t(const Plan& p, const Bufs& b, const void* Q, const void* K,
                     const void* Pq, const void* Pk, int h0, int nh, hipStream_t s) {
  const dim3 grid(p.Npad / kRows, nh, 1);
  const T* Qh = static_cast<const T*>(Q) + static_cast<size_t>(h0) * p.N * D;
  const T* Kh = static_cast<const T*>(K) + static_cast<size_t>(h0) * p.N * D;
  hipLaunchKernelGGL((project_kernel<T, D, DP>), grid, dim3(kThreads), 0, s, Qh,
                     static_cast<const T*>(Pq), p.N, p.Npad, 0, b.qlo32, b.qlo16, b.qstat,
                     static_cast<bf16_t*>(nullptr), b.kstat);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((project_kernel<T, D, DP>), grid, dim3(kThreads), 0, s, Kh,
                     static_cast<const T*>(Pk), p.N, p.Npad, 1, b.klo32, b.klo16,
                     static_cast<float2*>(nullptr), b.ksamp, b.kstat);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t project_d(const Plan& p, const Bufs& b, const void* Q, const void* K,
                     const void* Pq, const void* Pk, int h0, int nh, hipStream_t s) {
  switch (p.dp) {
    case 16: return project_t<T, D, 16>(p, b, Q, K, Pq, Pk, h0, nh, s);
    case 32: return project_t<T, D, 32>(p, b, Q, K, Pq, Pk, h0, nh, s);
    case 64: return project_t<T, D, 64>(p, b, Q, K, Pq, Pk, h0, nh, s);
    case 128: return project_t<T, D, 128>(p, b, Q, K, Pq, Pk, h0, nh, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_init_chunk(const Plan& p, const Bufs& b, int first_chunk, hipStream_t s) {
  hipLaunchKernelGGL(init_chunk_kernel, dim3(1), dim3(256), 0, s, b.hdr, b.kstat, p.hc,
                     first_chunk);
  return hipGetLastError();
}

hipError_t launch_project(const Plan& p, const Bufs& b, const void* Q, const void* K,
                          const void* Pq, const void* Pk, int h0, int nh, hipStream_t s) {
  if (p.dtype == 0) {
    if (p.D == 64) return project_d<float, 64>(p, b, Q, K, Pq, Pk, h0, nh, s);
    if (p.D == 128) return project_d<float, 128>(p, b, Q, K, Pq, Pk, h0, nh, s);
  } else {
    if (p.D == 64) return project_d<bf16_t, 64>(p, b, Q, K, Pq, Pk, h0, nh, s);
    if (p.D == 128) return project_d<bf16_t, 128>(p, b, Q, K, Pq, Pk, h0, nh, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
