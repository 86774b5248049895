// The exact fp32 scores that decide the selection, written out for chosen
// query rows (page "mhpq.cn/news/1098205", §2.2: the scorer's output
// d_proj^-1/2 · q_low·k_lowᵀ; its FAQ in §4.4 suggests comparing top-k
// indices across runs, which needs the scores themselves).  Each value comes
// from exact_score(), the same function the re-rank and the fallback use, so
// the top-k of these values is exactly the index set the library returns.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;

template <int DP>
__global__ __launch_bounds__(kThreads) void dump_kernel(
    const float* __restrict__ q32, const float* __restrict__ k32, int N, int Npad, int causal,
    float scale, int row_begin, int row_count, float* __restrict__ S) {
  __shared__ float qrow[DP];
  const int h = blockIdx.y;
  const int r = blockIdx.x;
  const int i = row_begin + r;
  const size_t hq = static_cast<size_t>(h) * Npad;
  if (threadIdx.x < DP) qrow[threadIdx.x] = q32[(hq + i) * DP + threadIdx.x];
  __syncthreads();
  float* out = S + (static_cast<size_t>(h) * row_count + r) * N;
  for (int j = threadIdx.x; j < N; j += kThreads)
    out[j] = (causal && j > i) ? -INFINITY : exact_score<DP>(qrow, k32 + (hq + j) * DP, scale);
}

template <int DP>
hipError_t dump_t(const Plan& p, const Bufs& b, int nh, float scale, int row_begin,
                  int row_count, float* S, hipStream_t s) {
  hipLaunchKernelGGL((dump_kernel<DP>), dim3(row_count, nh), dim3(kThreads), 0, s, b.qlo32,
                     b.klo32, p.N, p.Npad, p.causal, scale, row_begin, row_count, S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dump(const Plan& p, const Bufs& b, int nh, float score_scale, int row_begin,
                       int row_count, float* S_chunk, hipStream_t s) {
  switch (p.dp) {
    case 16: return dump_t<16>(p, b, nh, score_scale, row_begin, row_count, S_chunk, s);
    case 32: return dump_t<32>(p, b, nh, score_scale, row_begin, row_count, S_chunk, s);
    case 64: return dump_t<64>(p, b, nh, score_scale, row_begin, row_count, S_chunk, s);
    case 128: return dump_t<128>(p, b, nh, score_scale, row_begin, row_count, S_chunk, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
