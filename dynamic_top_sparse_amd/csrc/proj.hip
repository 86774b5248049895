// Scorer projection: q_low = Q·Pq and k_low = K·Pk for every row of a head
// chunk (page "mhpq.cn/news/1098205", §2.2: the scorer's q_proj / k_proj map
// each head's vectors to d_proj dimensions).
//
// Per row it writes the fp32 projection (bf16 rows: products on the bf16
// MFMA, exact in fp32, summed in fp32; fp32 rows: FMAs in ascending order of
// the model dimension) -- the values every exact score is computed from --
// and, for the filter, a 16-bit copy scaled by a power of two (one
// exponent per query row, one per key head), plus the norms that bound the
// filter's error: ||x_low|| and ||x_low - x~|| (x~ the 16-bit row back in
// true units), both rounded up.  Keys need their head's exponent before they
// can be rounded, so they take two kernels: the projection (fp32 rows, the
// head's max |k| and max ||k||) and the pack (16-bit rows, residual norms,
// and every 16th row copied to the threshold sample).  Rows N..Npad-1 are
// zero padding.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kRows = 64;       // rows per workgroup
constexpr int kThreads = 256;

// Round-up factor for norms computed in fp32 (covers the rounding of the
// sum of squares and of the square root).
constexpr float kNormUp = 1.0f + 1.0f / 65536.0f;

template <typename T, int D, int DP, typename F>
__global__ __launch_bounds__(kThreads) void project_kernel(
    const T* __restrict__ X, const T* __restrict__ P, int N, int Npad, int is_key,
    float* __restrict__ lo32, uint16_t* __restrict__ lo16, float4* __restrict__ qstat,
    uint32_t* __restrict__ kstat, int pad_rows) {
  // pad_rows: rows N .. (block end) are written as zeros (the selection's
  // buffers hold Npad rows); otherwise only rows < N are written (a cache
  // being appended to).  kstat may be null for keys.
  constexpr int kXFloats = kRows * (D + 1);
  constexpr int kLoFloats = 2 * kRows * (DP + 1);
  // bf16 rows: 32x32 output tiles on the bf16 MFMA (the products are exact in
  // fp32, the sums fp32); fp32 rows: FMAs in ascending order of d.
  constexpr bool kMfma = sizeof(T) == 2 && DP % 32 == 0;
  constexpr int kPtRow = D + 8;             // padded row of the transposed copy
  // P as fp32 for the FMA path; for the MFMA path P transposed, bf16
  // (sPt[c * kPtRow + d]), so a lane's 8 consecutive k are one 16-byte read
  __shared__ float sP[kMfma ? 1 : D * DP];
  __shared__ uint16_t sPt[kMfma ? DP * kPtRow : 8];
  // the staged input rows are dead once accumulated, so the projected rows
  // and their rounding residuals reuse that space
  __shared__ float sXLo[kXFloats > kLoFloats ? kXFloats : kLoFloats];
  __shared__ int sE[kRows];
  __shared__ float sMax[2][kRows];
  float* sX = sXLo;
  float* sLo = sXLo;
  float* sRes = sXLo + kRows * (DP + 1);

  const int tid = threadIdx.x;
  const int h = blockIdx.y;                 // head within the chunk
  const int row0 = blockIdx.x * kRows;
  const T* Xh = X + static_cast<size_t>(h) * N * D;

  if constexpr (kMfma) {
    // 8 consecutive columns of one row of P per 16-byte load
    for (int e = tid; e < D * DP / 8; e += kThreads) {
      const int d = e / (DP / 8), c0 = (e % (DP / 8)) * 8;
      const uint4 u = *reinterpret_cast<const uint4*>(P + static_cast<size_t>(d) * DP + c0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        sPt[(c0 + i) * kPtRow + d] = static_cast<uint16_t>(w[i / 2] >> (16 * (i & 1)));
    }
  } else {
    for (int e = tid; e < D * DP; e += kThreads) sP[e] = io<T>::to_f32(P[e]);
  }
  constexpr int kGroups = kThreads / DP;    // row groups
  constexpr int kRowsPerThread = kRows / kGroups;
  const int c = tid % DP;
  const int g = tid / DP;
  const size_t base = static_cast<size_t>(h) * Npad;
  if constexpr (kMfma) {
    __syncthreads();
    const int w = tid >> 6, l = tid & 63;
    constexpr int CT = DP / 32;              // column tiles
    for (int t = w; t < (kRows / 32) * CT; t += kThreads / 64) {
      const int rt = t / CT, ct = t % CT;
      const int arow = row0 + 32 * rt + (l & 31);
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const int k0 = 16 * ks + 8 * (l >> 5);
        uint4 ua = make_uint4(0, 0, 0, 0);
        if (arow < N) ua = *reinterpret_cast<const uint4*>(Xh + static_cast<size_t>(arow) * D + k0);
        bf16x8 va, vb;
        __builtin_memcpy(&va, &ua, 16);
        const uint4 ub = *reinterpret_cast<const uint4*>(&sPt[(32 * ct + (l & 31)) * kPtRow + k0]);
        __builtin_memcpy(&vb, &ub, 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, acc, 0, 0, 0);
      }
      // lane l, register r: row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 32 * rt + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        const int cc = 32 * ct + (l & 31);
        const float v = (row0 + rr < N) ? acc[r] : 0.0f;
        if (pad_rows || row0 + rr < N) lo32[(base + row0 + rr) * DP + cc] = v;
        sLo[rr * (DP + 1) + cc] = v;
      }
    }
  } else {
    for (int e = tid; e < kRows * D; e += kThreads) {
      const int r = e / D, d = e % D;
      const int row = row0 + r;
      sX[r * (D + 1) + d] = (row < N) ? io<T>::to_f32(Xh[static_cast<size_t>(row) * D + d]) : 0.0f;
    }
    __syncthreads();
    float acc[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) acc[i] = 0.0f;
    for (int d = 0; d < D; ++d) {
      const float pv = sP[d * DP + c];
#pragma unroll
      for (int i = 0; i < kRowsPerThread; ++i)
        acc[i] = __builtin_fmaf(sX[(g + i * kGroups) * (D + 1) + d], pv, acc[i]);
    }
    __syncthreads();  // every thread is done reading sX
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int r = g + i * kGroups;
      const int row = row0 + r;
      const float v = (row < N) ? acc[i] : 0.0f;
      if (pad_rows || row < N) lo32[(base + row) * DP + c] = v;
      sLo[r * (DP + 1) + c] = v;
    }
  }
  __syncthreads();
  if (tid < kRows) {
    float mx = 0.0f, s2 = 0.0f;
    for (int cc = 0; cc < DP; ++cc) {
      const float a = sLo[tid * (DP + 1) + cc];
      mx = fmaxf(mx, fabsf(a));
      s2 = __builtin_fmaf(a, a, s2);
    }
    sE[tid] = scale_exponent(mx);
    sMax[0][tid] = __builtin_sqrtf(s2) * kNormUp;
    sMax[1][tid] = mx;
  }
  __syncthreads();
  if (!is_key && lo16 == nullptr) return;   // fp32 rows and norms only
  if (is_key) {
    if (tid < 2 && kstat != nullptr) {
      float m = 0.0f;
      for (int r = 0; r < kRows; ++r) m = fmaxf(m, sMax[tid][r]);
      // non-negative floats order like their bit patterns
      atomicMax(&kstat[kKeyStatWords * h + (tid == 0 ? 0 : 2)], __float_as_uint(m));
    }
    return;
  }
  // queries: 16-bit rows with the row's own exponent, and residuals
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = g + i * kGroups;
    const int row = row0 + r;
    const int e = sE[r];
    const float v = sLo[r * (DP + 1) + c];
    const uint16_t u = F::round(__builtin_ldexpf(v, e));
    if (pad_rows || row < N) lo16[(base + row) * DP + c] = u;
    sRes[r * (DP + 1) + c] = v - __builtin_ldexpf(F::back(u), -e);
  }
  __syncthreads();
  if (tid < kRows && (pad_rows || row0 + tid < N)) {
    float r2 = 0.0f;
    for (int cc = 0; cc < DP; ++cc) {
      const float b = sRes[tid * (DP + 1) + cc];
      r2 = __builtin_fmaf(b, b, r2);
    }
    qstat[base + row0 + tid] =
        make_float4(sMax[0][tid], __builtin_sqrtf(r2) * kNormUp, __builtin_ldexpf(1.0f, -sE[tid]), 0.0f);
  }
}

// Keys: 16-bit rows with the head's exponent, the threshold sample, and the
// head's largest residual norm.
template <int DP, typename F>
__global__ __launch_bounds__(kThreads) void pack_keys_kernel(
    const float* __restrict__ k32, int Npad, int sstride, uint32_t* __restrict__ kstat,
    uint16_t* __restrict__ k16, uint16_t* __restrict__ samp) {
  __shared__ float sRes[kRows * (DP + 1)];
  __shared__ float sMax[kRows];
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int row0 = blockIdx.x * kRows;
  const int E = scale_exponent(__uint_as_float(kstat[kKeyStatWords * h + 2]));
  const size_t base = static_cast<size_t>(h) * Npad;
  constexpr int kGroups = kThreads / DP;
  constexpr int kRowsPerThread = kRows / kGroups;
  const int c = tid % DP;
  const int g = tid / DP;
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int r = g + i * kGroups;
    const int row = row0 + r;
    const float v = k32[(base + row) * DP + c];
    const uint16_t u = F::round(__builtin_ldexpf(v, E));
    k16[(base + row) * DP + c] = u;
    if ((row % sstride) == 0)
      samp[(static_cast<size_t>(h) * (Npad / sstride) + row / sstride) * DP + c] = u;
    sRes[r * (DP + 1) + c] = v - __builtin_ldexpf(F::back(u), -E);
  }
  __syncthreads();
  if (tid < kRows) {
    float r2 = 0.0f;
    for (int cc = 0; cc < DP; ++cc) {
      const float b = sRes[tid * (DP + 1) + cc];
      r2 = __builtin_fmaf(b, b, r2);
    }
    sMax[tid] = __builtin_sqrtf(r2) * kNormUp;
  }
  __syncthreads();
  if (tid == 0) {
    float m = 0.0f;
    for (int r = 0; r < kRows; ++r) m = fmaxf(m, sMax[r]);
    atomicMax(&kstat[kKeyStatWords * h + 1], __float_as_uint(m));
  }
}

__global__ void init_chunk_kernel(WsHeader* hdr, uint32_t* kstat, int* rcount, int nh,
                                  int first_chunk) {
  const int t = threadIdx.x;
  if (t == 0) {
    if (first_chunk) {
      hdr->fallback_queries = 0;
      hdr->overflow_queries = 0;
      hdr->candidates = 0;
      hdr->rescored = 0;
      hdr->queries = 0;
      hdr->retried = 0;
      hdr->margin_violations = 0;
      hdr->wide_queries = 0;
    }
    hdr->fb_count = 0;
    hdr->fb_next = 0;
  }
  for (int i = t; i < kKeyStatWords * nh; i += blockDim.x) kstat[i] = 0u;
  for (int i = t; i < nh; i += blockDim.x) rcount[i] = 0;
}

template <typename T, int D, int DP, typename F>
hipError_t project_t(const Plan& p, const Bufs& b, const void* Q, const void* K,
                     const void* Pq, const void* Pk, int h0, int nh, hipStream_t s) {
  const dim3 grid(p.Npad / kRows, nh, 1);
  const T* Qh = static_cast<const T*>(Q) + static_cast<size_t>(h0) * p.N * D;
  const T* Kh = static_cast<const T*>(K) + static_cast<size_t>(h0) * p.N * D;
  hipLaunchKernelGGL((project_kernel<T, D, DP, F>), grid, dim3(kThreads), 0, s, Qh,
                     static_cast<const T*>(Pq), p.N, p.Npad, 0, b.qlo32, b.qlo16, b.qstat,
                     b.kstat, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((project_kernel<T, D, DP, F>), grid, dim3(kThreads), 0, s, Kh,
                     static_cast<const T*>(Pk), p.N, p.Npad, 1, b.klo32,
                     static_cast<uint16_t*>(nullptr), static_cast<float4*>(nullptr), b.kstat, 1);
  return hipGetLastError();
}

template <typename T, int D, typename F>
hipError_t project_d(const Plan& p, const Bufs& b, const void* Q, const void* K,
                     const void* Pq, const void* Pk, int h0, int nh, hipStream_t s) {
  switch (p.dp) {
    case 16: return project_t<T, D, 16, F>(p, b, Q, K, Pq, Pk, h0, nh, s);
    case 32: return project_t<T, D, 32, F>(p, b, Q, K, Pq, Pk, h0, nh, s);
    case 64: return project_t<T, D, 64, F>(p, b, Q, K, Pq, Pk, h0, nh, s);
    case 128: return project_t<T, D, 128, F>(p, b, Q, K, Pq, Pk, h0, nh, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename F>
hipError_t project_tf(const Plan& p, const Bufs& b, const void* Q, const void* K,
                      const void* Pq, const void* Pk, int h0, int nh, hipStream_t s) {
  if (p.D == 64) return project_d<T, 64, F>(p, b, Q, K, Pq, Pk, h0, nh, s);
  if (p.D == 128) return project_d<T, 128, F>(p, b, Q, K, Pq, Pk, h0, nh, s);
  return hipErrorInvalidValue;
}

template <typename F>
hipError_t pack_f(const Plan& p, const Bufs& b, int nh, hipStream_t s) {
  const dim3 grid(p.Npad / kRows, nh, 1);
  switch (p.dp) {
#define SA_PACK(DPV)                                                                          \
  case DPV:                                                                                   \
    hipLaunchKernelGGL((pack_keys_kernel<DPV, F>), grid, dim3(kThreads), 0, s, b.klo32, p.Npad, \
                       p.sstride, b.kstat, b.klo16, b.ksamp);                                 \
    return hipGetLastError();
    SA_PACK(16)
    SA_PACK(32)
    SA_PACK(64)
    SA_PACK(128)
#undef SA_PACK
  }
  return hipErrorInvalidValue;
}

template <typename T, int D, int DP>
hipError_t project_rows_t(const void* X, const void* P, int nh, int rows, int out_stride,
                          int is_key, float* lo32, uint16_t* lo16, float4* qstat,
                          hipStream_t s) {
  const dim3 grid((rows + kRows - 1) / kRows, nh, 1);
  hipLaunchKernelGGL((project_kernel<T, D, DP, FiltF16>), grid, dim3(kThreads), 0, s,
                     static_cast<const T*>(X), static_cast<const T*>(P), rows, out_stride, is_key,
                     lo32, lo16, qstat, static_cast<uint32_t*>(nullptr), 0);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t project_rows_d(const void* X, const void* P, int nh, int rows, int out_stride, int dp,
                          int is_key, float* lo32, uint16_t* lo16, float4* qstat, hipStream_t s) {
  switch (dp) {
    case 16: return project_rows_t<T, D, 16>(X, P, nh, rows, out_stride, is_key, lo32, lo16, qstat, s);
    case 32: return project_rows_t<T, D, 32>(X, P, nh, rows, out_stride, is_key, lo32, lo16, qstat, s);
    case 64: return project_rows_t<T, D, 64>(X, P, nh, rows, out_stride, is_key, lo32, lo16, qstat, s);
    case 128: return project_rows_t<T, D, 128>(X, P, nh, rows, out_stride, is_key, lo32, lo16, qstat, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_project_rows(const void* X, const void* P, int nh, int rows, int out_stride,
                               int D, int dp, int dtype, int is_key, float* lo32, uint16_t* lo16,
                               float4* qstat, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return project_rows_d<float, 64>(X, P, nh, rows, out_stride, dp, is_key, lo32, lo16, qstat, s);
    if (D == 128) return project_rows_d<float, 128>(X, P, nh, rows, out_stride, dp, is_key, lo32, lo16, qstat, s);
  } else {
    if (D == 64) return project_rows_d<bf16_t, 64>(X, P, nh, rows, out_stride, dp, is_key, lo32, lo16, qstat, s);
    if (D == 128) return project_rows_d<bf16_t, 128>(X, P, nh, rows, out_stride, dp, is_key, lo32, lo16, qstat, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_init_chunk(const Plan& p, const Bufs& b, int first_chunk, hipStream_t s) {
  hipLaunchKernelGGL(init_chunk_kernel, dim3(1), dim3(256), 0, s, b.hdr, b.kstat, b.rcount, p.hc,
                     first_chunk);
  return hipGetLastError();
}

hipError_t launch_project(const Plan& p, const Bufs& b, const void* Q, const void* K,
                          const void* Pq, const void* Pk, int h0, int nh, hipStream_t s) {
  if (p.dtype == 0) {
    return p.filt ? project_tf<float, FiltBf16>(p, b, Q, K, Pq, Pk, h0, nh, s)
                  : project_tf<float, FiltF16>(p, b, Q, K, Pq, Pk, h0, nh, s);
  }
  return p.filt ? project_tf<bf16_t, FiltBf16>(p, b, Q, K, Pq, Pk, h0, nh, s)
                : project_tf<bf16_t, FiltF16>(p, b, Q, K, Pq, Pk, h0, nh, s);
}

hipError_t launch_pack_keys(const Plan& p, const Bufs& b, int nh, hipStream_t s) {
  return p.filt ? pack_f<FiltBf16>(p, b, nh, s) : pack_f<FiltF16>(p, b, nh, s);
}

}  // namespace sa
