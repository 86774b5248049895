// Helpers of the backward (page "mhpq.cn/news/1098205", §2.3, gradients of
// the top-k attention): the key segments of the entry list (how many rows
// kept each key, then where each key's entries start), and the scorer's
// projection gradients.
//
// Scorer: with q_low = Q·Pq and k_low = K·Pk, the straight-through gradient
// reaches dq_low and dk_low (the two passes in gather.hip); then
//   dQ += dq_low·Pqᵀ, dK += dk_low·Pkᵀ   (rows_times_pt),
//   dPq = sum over every row of Qᵀ·dq_low, dPk likewise  (outer_sum: fixed
//   row chunks, then the chunks' partial sums added in chunk order, so the
//   result does not depend on scheduling).
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kOuterRows = 4096;    // rows per outer-sum chunk
constexpr int kStageRows = 32;      // rows staged in LDS at a time

__global__ void fill_zero_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < n16;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void bwd_count_kernel(const int32_t* __restrict__ idx, long long total, int N, int k,
                                 int* __restrict__ cnt) {
  for (long long e = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<long long>(gridDim.x) * blockDim.x) {
    const int j = idx[e];
    const long long h = e / (static_cast<long long>(N) * k);
    if (j >= 0 && j < N) atomicAdd(&cnt[h * N + j], 1);
  }
}

// One workgroup per head: exclusive scan of the counts, i.e. each key's
// first entry within the head's region of the entry list.
__global__ __launch_bounds__(kThreads) void bwd_scan_kernel(const int* __restrict__ cnt, int N,
                                                            int* __restrict__ off,
                                                            int* __restrict__ cursor) {
  __shared__ int tmp[kThreads / kWave];
  const int h = blockIdx.x;
  const int* c = cnt + static_cast<size_t>(h) * N;
  int* o = off + static_cast<size_t>(h) * N;
  int* cu = cursor + static_cast<size_t>(h) * N;
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
    if (j < N) {
      const int x = running + before + incl - v;
      o[j] = x;
      cu[j] = x;
    }
    running += tot;
    __syncthreads();
  }
}

// out[r][d] += sum_c lo[r][c] P[d][c]; P staged transposed in LDS (fp32).
template <typename T, int D, int DP>
__global__ __launch_bounds__(kThreads) void rows_times_pt_kernel(const float* __restrict__ lo,
                                                                 const T* __restrict__ P,
                                                                 long long rows,
                                                                 float* __restrict__ out) {
  __shared__ float pt[DP * D];    // pt[c * D + d]
  for (int e = threadIdx.x; e < D * DP; e += kThreads) {
    const int d = e / DP, c = e % DP;
    pt[c * D + d] = io<T>::to_f32(P[e]);
  }
  __syncthreads();
  constexpr int RPB = kThreads / D;       // rows per pass of a workgroup
  const int d = threadIdx.x % D;
  for (long long r = blockIdx.x * static_cast<long long>(RPB) + threadIdx.x / D; r < rows;
       r += static_cast<long long>(gridDim.x) * RPB) {
    const float* lr = lo + r * DP;
    float acc = 0.0f;
#pragma unroll 8
    for (int c = 0; c < DP; ++c) acc = __builtin_fmaf(lr[c], pt[c * D + d], acc);
    out[r * D + d] += acc;
  }
}

// partial[chunk][d][c] = sum over the chunk's rows r (ascending) of
// X[r][d] lo[r][c]; each thread owns D*DP/256 of the outputs.
template <typename T, int D, int DP>
__global__ __launch_bounds__(kThreads) void outer_partial_kernel(const T* __restrict__ X,
                                                                 const float* __restrict__ lo,
                                                                 long long rows,
                                                                 float* __restrict__ partial) {
  constexpr int U = D * DP / kThreads;
  __shared__ float xs[kStageRows * D];
  __shared__ float ls[kStageRows * DP];
  float acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.0f;
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
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int o = threadIdx.x + u * kThreads;
        acc[u] = __builtin_fmaf(xs[r * D + o / DP], ls[r * DP + o % DP], acc[u]);
      }
    }
  }
  float* dst = partial + static_cast<size_t>(blockIdx.x) * D * DP;
#pragma unroll
  for (int u = 0; u < U; ++u) dst[threadIdx.x + u * kThreads] = acc[u];
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

template <typename T, int D>
hipError_t rows_pt_d(const float* lo, const void* P, long long rows, int dp, float* out,
                     hipStream_t s) {
  const unsigned grid = grid_for(rows * D);
  switch (dp) {
#define SA_RPT(DPV)                                                                          \
  case DPV:                                                                                  \
    hipLaunchKernelGGL((rows_times_pt_kernel<T, D, DPV>), dim3(grid), dim3(kThreads), 0, s, lo, \
                       static_cast<const T*>(P), rows, out);                                 \
    return hipGetLastError();
    SA_RPT(16)
    SA_RPT(32)
    SA_RPT(64)
    SA_RPT(128)
#undef SA_RPT
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

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;    // callers pass multiples of 16 bytes
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(static_cast<long long>(n16))), dim3(kThreads),
                     0, s, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

hipError_t launch_bwd_count(const int32_t* idx, int nh, int N, int k, int* cnt, hipStream_t s) {
  const long long total = static_cast<long long>(nh) * N * k;
  hipLaunchKernelGGL(bwd_count_kernel, dim3(grid_for(total)), dim3(kThreads), 0, s, idx, total, N,
                     k, cnt);
  return hipGetLastError();
}

hipError_t launch_bwd_scan(const int* cnt, int nh, int N, int* off, int* cursor,
                           hipStream_t s) {
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(nh), dim3(kThreads), 0, s, cnt, N, off, cursor);
  return hipGetLastError();
}

hipError_t launch_rows_times_pt(const float* lo, const void* P, int dtype, long long rows, int D,
                                int dp, float* out, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return rows_pt_d<float, 64>(lo, P, rows, dp, out, s);
    if (D == 128) return rows_pt_d<float, 128>(lo, P, rows, dp, out, s);
  } else {
    if (D == 64) return rows_pt_d<bf16_t, 64>(lo, P, rows, dp, out, s);
    if (D == 128) return rows_pt_d<bf16_t, 128>(lo, P, rows, dp, out, s);
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

}  // namespace sa
