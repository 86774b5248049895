// Block-granular selection: keys are cut into blocks of `block` consecutive
// rows, each block is scored as a whole, each query keeps its kb best blocks
// and attends to every valid key in them (block-sparse attention: the SSA
// page's _block_sparsify works on blocks of the mask; page
// "mhpq.cn/news/1098205", §2.1, block-sparse attention computes only some
// block pairs).  A block is scored with its mean key,
//   kbar_J = fl(sum of the block's k_low rows, in key order) / n_J,
// so its score exact_score(q_low_i, kbar_J) is (up to rounding) the mean of
// its keys' scores.  Causally a query keeps its own block (its keys up to
// the query) and picks kb - 1 more among the blocks that end before it.
//
// The score pass is plain fp32 FMA work (one query per lane, the block
// means staged in LDS and read by every lane at once): with block rows of 64
// there are 64x fewer scores than key pairs, so it is short next to the
// gather that follows.
#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kBlocksPerStage = 64;   // block means staged in LDS at a time
constexpr int kBlockKbMax = 32;       // most blocks a query keeps

template <int DP>
__global__ __launch_bounds__(kThreads) void block_means_kernel(const float* __restrict__ k32,
                                                               int N, int block, int NB,
                                                               float* __restrict__ kbar) {
  const int h = blockIdx.y;
  const int J = blockIdx.x;
  const int c = threadIdx.x;
  if (c >= DP) return;
  const int j0 = J * block, j1 = min(N, j0 + block);
  const float* src = k32 + static_cast<size_t>(h) * N * DP;
  float s = 0.0f;
  for (int j = j0; j < j1; ++j) s += src[static_cast<size_t>(j) * DP + c];
  kbar[(static_cast<size_t>(h) * NB + J) * DP + c] = s / static_cast<float>(j1 - j0);
}

__device__ __forceinline__ unsigned long long block_rank(float s, int J) {
  return (static_cast<unsigned long long>(order_key(s)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(J));
}

// One query per thread: its top-kb blocks by (score descending, block
// ascending), kept in registers as a list sorted best first.
template <int DP, int KB>
__global__ __launch_bounds__(kThreads) void block_select_kernel(
    const float* __restrict__ q32, const float* __restrict__ kbar, int N, int block, int NB,
    int kb, int causal, float scale, int32_t* __restrict__ sel) {
  __shared__ float4 sk[kBlocksPerStage * DP / 4];
  const int h = blockIdx.y;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const bool live = i < N;
  float q[DP];
  {
    const float4* qr = reinterpret_cast<const float4*>(q32 + (static_cast<size_t>(h) * N + (live ? i : 0)) * DP);
#pragma unroll
    for (int c = 0; c < DP / 4; ++c) {
      const float4 v = qr[c];
      q[4 * c] = v.x; q[4 * c + 1] = v.y; q[4 * c + 2] = v.z; q[4 * c + 3] = v.w;
    }
  }
  const int own = i / block;
  // candidate blocks: all, or (causal) those before the query's own block
  const int ncand = causal ? own : NB;
  const int want = causal ? min(kb - 1, ncand) : min(kb, ncand);
  // (KB >= kb: the list's register length, the smallest of 4, 8, 16, 32)
  unsigned long long best[KB];
#pragma unroll
  for (int t = 0; t < KB; ++t) best[t] = 0ull;   // below every real rank
  unsigned long long last = 0ull;                         // best[want - 1]
  // blocks the workgroup must score: the largest candidate count among its queries
  const int i_last = min(N, static_cast<int>(blockIdx.x) * kThreads + kThreads) - 1;
  const int nscan = causal ? i_last / block : NB;
  const float4* kh = reinterpret_cast<const float4*>(kbar + static_cast<size_t>(h) * NB * DP);
  for (int J0 = 0; J0 < nscan; J0 += kBlocksPerStage) {
    const int nst = min(kBlocksPerStage, nscan - J0);
    __syncthreads();
    for (int e = threadIdx.x; e < nst * DP / 4; e += kThreads) sk[e] = kh[static_cast<size_t>(J0) * DP / 4 + e];
    __syncthreads();
    for (int u = 0; u < nst; ++u) {
      const int J = J0 + u;
      const float* kr = reinterpret_cast<const float*>(sk + u * DP / 4);
      const float s = exact_score<DP>(q, kr, scale);
      const unsigned long long r = block_rank(s, J);
      // insert when it beats the last kept entry (and is a candidate)
      if (live && J < ncand && want > 0 && r > last) {
        unsigned long long x = r;
#pragma unroll
        for (int t = 0; t < KB; ++t) {
          if (t < want && x > best[t]) {
            const unsigned long long y = best[t];
            best[t] = x;
            x = y;
          }
          if (t == want - 1) last = best[t];
        }
      }
    }
  }
  if (!live) return;
  // kept blocks by rank (best first), then (causal) the query's own block;
  // the expand kernel puts them in key order
  int32_t* out = sel + (static_cast<size_t>(h) * N + i) * kb;
#pragma unroll
  for (int t = 0; t < KB; ++t) {
    if (t < kb) {
      int v = -1;
      if (t < want) v = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best[t] & 0xFFFFFFFFull));
      else if (causal && t == want) v = own;
      out[t] = v;
    }
  }
}

// One wavefront per query: the keys of its kept blocks, ascending (valid
// keys only: causally j <= i), then -1 up to kb * block entries.  Lane t
// holds kept block t; its place in key order is the number of kept blocks
// with a smaller id (ids are distinct), its output offset the key count of
// those blocks.
__global__ __launch_bounds__(kThreads) void block_expand_kernel(const int32_t* __restrict__ sel,
                                                                int N, int block, int kb,
                                                                int causal,
                                                                int32_t* __restrict__ idx) {
  const int w = threadIdx.x / kWave, l = lane_id();
  const int i = blockIdx.x * (kThreads / kWave) + w;
  const int h = blockIdx.y;
  if (i >= N) return;
  const int32_t* s = sel + (static_cast<size_t>(h) * N + i) * kb;
  const int width = kb * block;
  int32_t* out = idx + (static_cast<size_t>(h) * N + i) * width;
  const int J = l < kb ? s[l] : -1;
  int j0 = 0, len = 0;
  if (J >= 0) {
    j0 = J * block;
    int j1 = min(N, j0 + block);
    if (causal) j1 = min(j1, i + 1);
    len = max(0, j1 - j0);
  }
  int start = 0;
  for (int u = 0; u < kb; ++u) {
    const int Ju = __shfl(J, u, kWave);
    const int lu = __shfl(len, u, kWave);
    if (Ju >= 0 && J >= 0 && Ju < J) start += lu;
  }
  int total = 0;
  for (int u = 0; u < kb; ++u) {
    const int Ju = __shfl(J, u, kWave);          // wave-uniform from here on
    if (Ju < 0) continue;
    const int su = __shfl(start, u, kWave);
    const int lu = __shfl(len, u, kWave);
    const int b0 = __shfl(j0, u, kWave);
    for (int e = l; e < lu; e += kWave) out[su + e] = b0 + e;
    total += lu;
  }
  for (int t = total + l; t < width; t += kWave) out[t] = -1;
}

template <int DP>
__global__ __launch_bounds__(kThreads) void block_dump_kernel(const float* __restrict__ q32,
                                                              const float* __restrict__ kbar,
                                                              int N, int NB, float scale,
                                                              int row_begin, int row_count,
                                                              float* __restrict__ S) {
  __shared__ float qrow[DP];
  const int h = blockIdx.y, r = blockIdx.x;
  const int i = row_begin + r;
  if (threadIdx.x < DP) qrow[threadIdx.x] = q32[(static_cast<size_t>(h) * N + i) * DP + threadIdx.x];
  __syncthreads();
  float* out = S + (static_cast<size_t>(h) * row_count + r) * NB;
  for (int J = threadIdx.x; J < NB; J += kThreads)
    out[J] = exact_score<DP>(qrow, kbar + (static_cast<size_t>(h) * NB + J) * DP, scale);
}

template <int DP>
hipError_t means_sel_t(const float* q32, const float* k32, int nh, int N, int block, int kb,
                       int causal, float scale, float* kbar, int32_t* sel, hipStream_t s) {
  const int NB = (N + block - 1) / block;
  hipLaunchKernelGGL((block_means_kernel<DP>), dim3(NB, nh), dim3(DP), 0, s, k32, N, block, NB,
                     kbar);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || sel == nullptr) return e;
  const dim3 grid((N + kThreads - 1) / kThreads, nh);
  if (kb <= 4)
    hipLaunchKernelGGL((block_select_kernel<DP, 4>), grid, dim3(kThreads), 0, s, q32, kbar, N,
                       block, NB, kb, causal, scale, sel);
  else if (kb <= 8)
    hipLaunchKernelGGL((block_select_kernel<DP, 8>), grid, dim3(kThreads), 0, s, q32, kbar, N,
                       block, NB, kb, causal, scale, sel);
  else if (kb <= 16)
    hipLaunchKernelGGL((block_select_kernel<DP, 16>), grid, dim3(kThreads), 0, s, q32, kbar, N,
                       block, NB, kb, causal, scale, sel);
  else
    hipLaunchKernelGGL((block_select_kernel<DP, kBlockKbMax>), grid, dim3(kThreads), 0, s, q32,
                       kbar, N, block, NB, kb, causal, scale, sel);
  return hipGetLastError();
}

template <int DP>
hipError_t bdump_t(const float* q32, const float* kbar, int nh, int N, int NB, float scale,
                   int row_begin, int row_count, float* S, hipStream_t s) {
  hipLaunchKernelGGL((block_dump_kernel<DP>), dim3(row_count, nh), dim3(kThreads), 0, s, q32,
                     kbar, N, NB, scale, row_begin, row_count, S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_select(const float* q32, const float* k32, int nh, int N, int dp,
                               int block, int kb, int causal, float scale, float* kbar,
                               int32_t* sel, hipStream_t s) {
  switch (dp) {
    case 16: return means_sel_t<16>(q32, k32, nh, N, block, kb, causal, scale, kbar, sel, s);
    case 32: return means_sel_t<32>(q32, k32, nh, N, block, kb, causal, scale, kbar, sel, s);
    case 64: return means_sel_t<64>(q32, k32, nh, N, block, kb, causal, scale, kbar, sel, s);
    case 128: return means_sel_t<128>(q32, k32, nh, N, block, kb, causal, scale, kbar, sel, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_block_expand(const int32_t* sel, int nh, int N, int block, int kb, int causal,
                               int32_t* idx, hipStream_t s) {
  const dim3 grid((N + kThreads / kWave - 1) / (kThreads / kWave), nh);
  hipLaunchKernelGGL(block_expand_kernel, grid, dim3(kThreads), 0, s, sel, N, block, kb, causal,
                     idx);
  return hipGetLastError();
}

hipError_t launch_block_dump(const float* q32, const float* kbar, int nh, int N, int NB, int dp,
                             float scale, int row_begin, int row_count, float* S, hipStream_t s) {
  switch (dp) {
    case 16: return bdump_t<16>(q32, kbar, nh, N, NB, scale, row_begin, row_count, S, s);
    case 32: return bdump_t<32>(q32, kbar, nh, N, NB, scale, row_begin, row_count, S, s);
    case 64: return bdump_t<64>(q32, kbar, nh, N, NB, scale, row_begin, row_count, S, s);
    case 128: return bdump_t<128>(q32, kbar, nh, N, NB, scale, row_begin, row_count, S, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
