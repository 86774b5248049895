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
#include "rows.h"

namespace sa {

__device__ int g_index_error_flag = 0;

// The current device's copy of the flag, for kernels of other sources.
hipError_t index_error_flag(int** out) {
  static std::atomic<int*> ptrs[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int* p = ptrs[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    void* v = nullptr;
    e = hipGetSymbolAddress(&v, HIP_SYMBOL(g_index_error_flag));
    if (e != hipSuccess) return e;
    p = static_cast<int*>(v);
    ptrs[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

// One wave attends query row `row` (Q, idx, O rows at row; the head's K and
// V rows at Kh, Vh, N of them).
template <typename T, int D>
__device__ __forceinline__ void gather_row(const T* __restrict__ Q, const T* __restrict__ Kh,
                                           const T* __restrict__ Vh,
                                           const int32_t* __restrict__ idx, int k, int N,
                                           float scale, T* __restrict__ O, size_t row,
                                           float* slog, int* sidx) {
  constexpr int EPL = Vec<T>::kElems;
  constexpr int LPR = D / EPL;
  const int l = lane_id();
  stage_entries(idx + row * k, 0, k, sidx);
  const int32_t* rw = sidx;
  int bad = 0;
  logits<T, D>(Q + row * D, Kh, rw, 0, k, N, scale * kLog2e, slog, bad);
  if (bad) atomicOr(&g_index_error_flag, 1);
  wave_sync();
  float sum;
  const float mx = softmax_weights(slog, k, sum);
  T* out = O + row * D;
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  float acc[EPL];
  if (mx == -INFINITY) {  // no valid entry: zero output
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    if (g == 0) *reinterpret_cast<uint4*>(out + e0) = Vec<T>::pack(acc);
    return;
  }
  wave_sync();
  weighted_rows<T, D>(Vh, rw, 0, k, N, slog, acc);
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] /= sum;
    *reinterpret_cast<uint4*>(out + e0) = Vec<T>::pack(acc);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, int k, int Nq, int Nk, float scale, T* __restrict__ O) {
  // Nq query rows (and idx, O rows) and Nk key rows per head: equal in the
  // forward, one query against a key cache when decoding
  extern __shared__ float slog_all[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform, scalar
  float* slog = slog_all + w * gather_wave_floats(k);
  int* sidx = reinterpret_cast<int*>(slog + gather_slog_floats(k));
  const int h = blockIdx.y;
  const int q = blockIdx.x * kWaves + w;
  if (q >= Nq) return;
  gather_row<T, D>(Q, K + static_cast<size_t>(h) * Nk * D, V + static_cast<size_t>(h) * Nk * D,
                   idx, k, Nk, scale, O, static_cast<size_t>(h) * Nq + q, slog, sidx);
}

// The rows listed in `list` (flat row numbers h*N + q, count at *count),
// each attended as gather_kernel does: the rows the key-range path of
// sparse_attn_gather_ws cannot take.  A fixed grid of waves walks the list.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void gather_list_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, int k, int N, float scale, const int* __restrict__ list,
    const int* __restrict__ count, T* __restrict__ O) {
  extern __shared__ float slog_all[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  float* slog = slog_all + w * gather_wave_floats(k);
  int* sidx = reinterpret_cast<int*>(slog + gather_slog_floats(k));
  const int n = *count;
  for (int i = blockIdx.x * kWaves + w; i < n; i += gridDim.x * kWaves) {
    const size_t row = static_cast<size_t>(static_cast<unsigned>(list[i]));
    const size_t h = row / static_cast<unsigned>(N);
    gather_row<T, D>(Q, K + h * N * D, V + h * N * D, idx, k, N, scale, O, row, slog, sidx);
    wave_sync();    // this row's LDS reads are done before the next row is staged
  }
}

// Row check of sparse_attn_gather_ws, one wave per row.  A row whose valid
// entries (0 <= j < N) form an ascending prefix (repeats allowed), followed
// by negative entries only, gets seg[row][r] = its valid entries below the
// start of key range r (r = 0..8; seg[row][8] = all of them), the form the
// key-range kernels take.  Any other row (out of order, an entry >= N, a
// valid entry after a negative one) gets -1 throughout, so the range kernels
// leave it empty, and joins the list of rows the single-pass kernel takes.
__global__ __launch_bounds__(kThreads) void gather_row_check_kernel(
    const int32_t* __restrict__ idx, int k, int N, long long rows, GatherRanges gr,
    int* __restrict__ seg, int* __restrict__ list, int* __restrict__ count) {
  constexpr int R = kGatherRanges;
  const int w = threadIdx.x / kWave, l = lane_id();
  const long long row = static_cast<long long>(blockIdx.x) * (kThreads / kWave) + w;
  if (row >= rows) return;
  const int32_t* ir = idx + row * k;
  int below[R + 1];
#pragma unroll
  for (int r = 0; r <= R; ++r) below[r] = 0;
  bool ok = true;               // wave-uniform after the ballots
  int last = -1;                // previous chunk's last entry
  constexpr int kChunks = 4;    // 64-entry chunks loaded before any is checked
  for (int c0 = 0; c0 < k; c0 += kChunks * kWave) {
    int jc[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int t = c0 + c * kWave + l;
      jc[c] = t < k ? ir[t] : -1;
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int t = c0 + c * kWave + l;
      const int j = jc[c];
      const bool valid = j >= 0 && j < N;
      int prev = __shfl_up(j, 1, kWave);
      if (l == 0) prev = last;
      const bool prev_valid = prev >= 0 && prev < N;
      const bool bad = j >= N || (valid && ((t > 0 && !prev_valid) || (prev_valid && prev > j)));
      if (__ballot(bad)) ok = false;
#pragma unroll
      for (int r = 1; r < R; ++r) below[r] += valid && j < gr.b[r] ? 1 : 0;
      below[R] += valid ? 1 : 0;
      last = __shfl(j, kWave - 1, kWave);
    }
  }
  int* out = seg + row * (R + 1);
  if (!ok) {
    if (l <= R) out[l] = -1;
    if (l == 0) list[atomicAdd(count, 1)] = static_cast<int>(row);
    return;
  }
#pragma unroll
  for (int r = 1; r <= R; ++r) below[r] = wave_sum_i(below[r]);
  if (l == 0) {
    out[0] = 0;
#pragma unroll
    for (int r = 1; r <= R; ++r) out[r] = below[r];
  }
}

__global__ void gather_zero_kernel(int* __restrict__ x) { *x = 0; }

// --------------------------------------------------------- split gather ---
// The fused forward's idx rows are ascending, so the keys of a row that fall
// in one key range form one contiguous segment of it.  A head's K and V rows
// (64 MB at N = 128K, D = 128, bf16) are far larger than one XCD's 4 MB L2,
// and a row is read by about k queries, so the gather splits the keys into
// kGatherRanges ranges and orders its workgroups so that each XCD serves one
// range at a time (workgroups are handed to the 8 XCDs in turn): an XCD's
// working set is then one range.  Eight ranges (8 MB of K and V each at the
// headline size) measured faster than sixteen: every (query, range) pays a
// fixed cost, and halving their number outweighs the lower L2 hit rate.
// Causal rows read low keys far more often than high ones, so there the
// ranges are cut for equal expected work instead of equal width (see
// gather_ranges); the kernel itself only reads the rows' range starts.  Each
// (query, range) writes an online-softmax partial (max m, sum l of 2^(x-m),
// unnormalised sum of 2^(x-m) V) and a merge combines the partials of a query.

template <typename T, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void gather_part_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, const int* __restrict__ seg, int k, int N, int QB,
    float scale, float* __restrict__ part) {
  constexpr int EPL = Vec<T>::kElems;
  constexpr int LPR = D / EPL;
  constexpr int R = kGatherRanges;
  extern __shared__ float slog_all[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform, scalar
  const int l = lane_id();
  // workgroup i -> (range, query block); consecutive workgroups land on
  // consecutive XCDs, so XCD x serves ranges x, x + 8, ... one after another
  const int i = static_cast<int>(blockIdx.x);
  const int x = i % kXcds, rest = i / kXcds;
  const int qb = rest % QB, r = rest / QB * kXcds + x;
  const int q = qb * kWaves + w;
  if (q >= N) return;
  float* slog = slog_all + w * gather_wave_floats(k);
  int* sidx = reinterpret_cast<int*>(slog + gather_slog_floats(k));
  // the segment bounds are the wave's own (every lane reads the same words):
  // kept in scalar registers, every loop bound and trip count below is
  // uniform and needs no lane mask
  const int s0 = __builtin_amdgcn_readfirstlane(seg[static_cast<size_t>(q) * (R + 1) + r]);
  const int s1 = __builtin_amdgcn_readfirstlane(seg[static_cast<size_t>(q) * (R + 1) + r + 1]);
  float* rec = part + (static_cast<size_t>(q) * R + r) * (D + 4);
  if (s0 >= s1) {
    if (l == 0) rec[0] = -INFINITY;   // empty: the merge skips it
    return;
  }
  stage_entries(idx + static_cast<size_t>(q) * k, s0, s1, sidx);
  const int32_t* row = sidx;
  if constexpr (sizeof(T) == 2) {
    logits_bf16_split<D>(Q + static_cast<size_t>(q) * D, K, row, s1 - s0, N, scale * kLog2e, slog);
  } else {
    int bad = 0;
    logits<T, D>(Q + static_cast<size_t>(q) * D, K, row, s0, s1, N, scale * kLog2e, slog, bad);
    if (bad) atomicOr(&g_index_error_flag, 1);
  }
  wave_sync();
  float sum;
  const float mx = softmax_weights(slog, s1 - s0, sum);
  if (mx == -INFINITY) {
    if (l == 0) rec[0] = -INFINITY;
    return;
  }
  wave_sync();
  float acc[EPL];
  if constexpr (sizeof(T) == 2)
    weighted_rows_bf16_split<D>(V, row, s1 - s0, N, slog, acc);
  else
    weighted_rows<T, D>(V, row, s0, s1, N, slog, acc);
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

// O_q = sum_r 2^(m_r - M) acc_r / sum_r 2^(m_r - M) l_r, M = max_r m_r (base-2
// logits, as in the partials).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void gather_merge_kernel(const float* __restrict__ part,
                                                                int N, T* __restrict__ O) {
  constexpr int R = kGatherRanges;
  constexpr int EPM = D / kWave;     // output elements per lane
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform, scalar
  const int l = lane_id();
  // Last query block first: the partial kernel wrote the partials in query
  // order, so the most recent ones, still in the memory-side cache, are read
  // before they are pushed out.
  const int q = (gridDim.x - 1 - blockIdx.x) * kWaves + w;
  if (q >= N) return;
  const float* recs = part + static_cast<size_t>(q) * R * (D + 4);
  // Every load is issued at once: the maxima with their sums and the
  // partial rows (an empty range's row and sum hold stale values, so they
  // are selected away, never multiplied by its weight 0).
  const int lr = l < R ? l : 0;
  const float m0 = recs[static_cast<size_t>(lr) * (D + 4)];
  const float s0 = recs[static_cast<size_t>(lr) * (D + 4) + 1];
  float a[R][EPM];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float* src = recs + static_cast<size_t>(r) * (D + 4) + 4 + l * EPM;
#pragma unroll
    for (int e = 0; e < EPM; ++e) a[r][e] = src[e];
  }
  // (the compiler would otherwise sink loads past the reductions, or into
  // the branch it makes of the first range's select: a second round trip)
  asm volatile("" ::"v"(m0), "v"(s0));
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < EPM; ++e) asm volatile("" ::"v"(a[r][e]));
  const float m = l < R ? m0 : -INFINITY;
  const float lsum = m != -INFINITY ? s0 : 0.0f;
  const float M = wave_max(m);
  T* out = O + static_cast<size_t>(q) * D + l * EPM;
  float acc[EPM];
#pragma unroll
  for (int e = 0; e < EPM; ++e) acc[e] = 0.0f;
  const float wr = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
  const float L = wave_sum(wr * lsum);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float wv = __shfl(wr, r, kWave);
#pragma unroll
    for (int e = 0; e < EPM; ++e) acc[e] = wv != 0.0f ? __builtin_fmaf(wv, a[r][e], acc[e]) : acc[e];
  }
  // no valid entry in any range (M = -inf, L = 0): a zero row
  const bool none = M == -INFINITY;
#pragma unroll
  for (int e = 0; e < EPM; ++e) out[e] = io<T>::from_f32(none ? 0.0f : acc[e] / L);
}

template <typename T, int D>
hipError_t gather_split_t(const void* Q, const void* K, const void* V, const int32_t* idx,
                          int k, int N, float scale, const int* seg, float* part,
                          void* O, sa_profile* prof, hipStream_t s) {
  const int QB = (N + kWaves - 1) / kWaves;
  const size_t lds_part = static_cast<size_t>(kWaves) * gather_wave_floats(k) * sizeof(float);
  static std::atomic<int> lds_set[kMaxDevices];
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&gather_part_kernel<T, D>),
                                    static_cast<int>(kWaves) * gather_wave_floats(kKMax) * 4,
                                    lds_set);
  if (e != hipSuccess) return e;
  int t = prof_begin(prof, "gather", s);
  hipLaunchKernelGGL((gather_part_kernel<T, D>), dim3(QB * kGatherRanges), dim3(kThreads), lds_part, s,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     idx, seg, k, N, QB, scale, part);
  e = hipGetLastError();
  prof_end(prof, t, s);
  if (e != hipSuccess) return e;
  t = prof_begin(prof, "gather_merge", s);
  hipLaunchKernelGGL((gather_merge_kernel<T, D>), dim3(QB), dim3(kThreads), 0, s, part, N,
                     static_cast<T*>(O));
  e = hipGetLastError();
  prof_end(prof, t, s);
  return e;
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
                    int nheads, int N, int Nk, float scale, void* O, hipStream_t s) {
  const size_t lds = static_cast<size_t>(kWaves) * gather_wave_floats(k) * sizeof(float);
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&gather_kernel<T, D>),
                                          static_cast<int>(kWaves) * gather_wave_floats(kKMax) * 4,
                                          lds_set);
  if (e != hipSuccess) return e;
  const dim3 grid((N + kWaves - 1) / kWaves, nheads);
  hipLaunchKernelGGL((gather_kernel<T, D>), grid, dim3(kThreads), lds, s,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     idx, k, N, Nk, scale, static_cast<T*>(O));
  return hipGetLastError();
}

template <typename T, int D>
hipError_t gather_list_t(const void* Q, const void* K, const void* V, const int32_t* idx, int k,
                         int N, float scale, const int* list, const int* count, void* O,
                         hipStream_t s) {
  const size_t lds = static_cast<size_t>(kWaves) * gather_wave_floats(k) * sizeof(float);
  static std::atomic<int> lds_set[kMaxDevices];
  const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&gather_list_kernel<T, D>),
                                          static_cast<int>(kWaves) * gather_wave_floats(kKMax) * 4,
                                          lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gather_list_kernel<T, D>), dim3(1024), dim3(kThreads), lds, s,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     idx, k, N, scale, list, count, static_cast<T*>(O));
  return hipGetLastError();
}

}  // namespace


hipError_t launch_gather(const void* Q, const void* K, const void* V, const int32_t* idx, int k,
                         int nheads, int N, int D, float softmax_scale, int dtype, void* O,
                         hipStream_t s) {
  return launch_gather_rows(Q, K, V, idx, k, nheads, N, N, D, softmax_scale, dtype, O, s);
}

hipError_t launch_gather_rows(const void* Q, const void* K, const void* V, const int32_t* idx,
                              int k, int nheads, int Nq, int Nk, int D, float softmax_scale,
                              int dtype, void* O, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return gather_t<float, 64>(Q, K, V, idx, k, nheads, Nq, Nk, softmax_scale, O, s);
    if (D == 128) return gather_t<float, 128>(Q, K, V, idx, k, nheads, Nq, Nk, softmax_scale, O, s);
  } else {
    if (D == 64) return gather_t<bf16_t, 64>(Q, K, V, idx, k, nheads, Nq, Nk, softmax_scale, O, s);
    if (D == 128) return gather_t<bf16_t, 128>(Q, K, V, idx, k, nheads, Nq, Nk, softmax_scale, O, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_split(const void* Q, const void* K, const void* V, const int32_t* idx,
                               int k, int N, int D, float softmax_scale, int dtype, const int* seg,
                               float* part, void* O, sa_profile* prof, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return gather_split_t<float, 64>(Q, K, V, idx, k, N, softmax_scale, seg, part, O, prof, s);
    if (D == 128) return gather_split_t<float, 128>(Q, K, V, idx, k, N, softmax_scale, seg, part, O, prof, s);
  } else {
    if (D == 64) return gather_split_t<bf16_t, 64>(Q, K, V, idx, k, N, softmax_scale, seg, part, O, prof, s);
    if (D == 128) return gather_split_t<bf16_t, 128>(Q, K, V, idx, k, N, softmax_scale, seg, part, O, prof, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gather_check(const int32_t* idx, int k, int nheads, int N, int* seg,
                               int* list, int* count, hipStream_t s) {
  hipLaunchKernelGGL(gather_zero_kernel, dim3(1), dim3(1), 0, s, count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long rows = static_cast<long long>(nheads) * N;
  const long long blocks = (rows + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(gather_row_check_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                     0, s, idx, k, N, rows, gather_ranges(N, 0), seg, list, count);
  return hipGetLastError();
}

hipError_t launch_gather_list(const void* Q, const void* K, const void* V, const int32_t* idx,
                              int k, int N, int D, float softmax_scale, int dtype, const int* list,
                              const int* count, void* O, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return gather_list_t<float, 64>(Q, K, V, idx, k, N, softmax_scale, list, count, O, s);
    if (D == 128) return gather_list_t<float, 128>(Q, K, V, idx, k, N, softmax_scale, list, count, O, s);
  } else {
    if (D == 64) return gather_list_t<bf16_t, 64>(Q, K, V, idx, k, N, softmax_scale, list, count, O, s);
    if (D == 128) return gather_list_t<bf16_t, 128>(Q, K, V, idx, k, N, softmax_scale, list, count, O, s);
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
