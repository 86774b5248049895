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
constexpr int kUnroll = 7;   // row loads in flight per lane (7 keeps the partial kernel at 8 waves per SIMD)
constexpr int kXcds = 8;     // XCDs of the chip: workgroups are dealt to them in turn

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

// ---------------------------------------------------- per-wave attention ---
// One wavefront attends one query over entries [t0, t1) of its index row.
// The entries are first copied to the wave's LDS (`row` below points at that
// copy, so every later key load waits on LDS rather than on a global load);
// logits go to the wave's LDS buffer `slog` (index t - t0; room for t1 - t0
// rounded up to 16), then become the unnormalised weights e^(x - m).

// Logits, bf16 I/O: rows are read as the V rows are (LPR lanes x 16 bytes
// per row, RPI whole rows per load instruction), so each load touches whole
// 128-byte lines; the vector memory path, not the arithmetic, bounds the
// gather.  Each lane forms its 8 products with four bf16 dot2 instructions
// (bf16 products are exact in fp32; the sums are fp32) and the row's lanes
// add their partial sums.
template <int D>
__device__ __forceinline__ void logits_bf16(const bf16_t* __restrict__ qrow,
                                            const bf16_t* __restrict__ K,
                                            const int32_t* __restrict__ row, int t0, int t1,
                                            int N, float scale, float* slog, int& bad) {
  constexpr int EPL = 8, LPR = D / EPL, RPI = kWave / LPR;
  const int l = lane_id();
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  const uint4 q4 = *reinterpret_cast<const uint4*>(qrow + e0);
  bf16x2 qp[4];
  __builtin_memcpy(qp, &q4, 16);
  for (int tb = t0; tb < t1; tb += RPI * kUnroll) {
    const int nu = min(kUnroll, (t1 - tb + RPI - 1) / RPI);   // loads holding rows (uniform)
    uint4 kv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const int jr = row[t - t0];                  // t - t0 < t1 - t0 + RPI: inside the slack
      const int j = t < t1 ? jr : -1;
      ok[u] = j >= 0 && j < N;
      bad |= (t < t1 && j >= N) ? 1 : 0;
      // row 0 stands in for an invalid entry, whose logit is -inf below
      kv[u] = *reinterpret_cast<const uint4*>(K + static_cast<size_t>(ok[u] ? j : 0) * D + e0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      bf16x2 kp[4];
      __builtin_memcpy(kp, &kv[u], 16);
      float dot = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) dot = __builtin_amdgcn_fdot2_f32_bf16(kp[i], qp[i], dot, false);
      dot = group_sum<LPR>(dot);
      const int t = tb + u * RPI + g;
      if ((l % LPR) == 0 && t < t1) slog[t - t0] = ok[u] ? dot * scale : -INFINITY;
    }
  }
}

// Logits, fp32 I/O: each row is spread over LPR lanes, partial dots reduced
// across them.
template <int D>
__device__ __forceinline__ void logits_f32(const float* __restrict__ qrow,
                                           const float* __restrict__ K,
                                           const int32_t* __restrict__ row, int t0, int t1,
                                           int N, float scale, float* slog, int& bad) {
  constexpr int EPL = 4, LPR = D / EPL, RPI = kWave / LPR;
  const int l = lane_id();
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  const float4 q4 = *reinterpret_cast<const float4*>(qrow + e0);
  for (int tb = t0; tb < t1; tb += RPI * kUnroll) {
    const int nu = min(kUnroll, (t1 - tb + RPI - 1) / RPI);   // loads holding rows (uniform)
    float4 kv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const int jr = row[t - t0];                  // t - t0 < t1 - t0 + RPI: inside the slack
      const int j = t < t1 ? jr : -1;
      ok[u] = j >= 0 && j < N;
      bad |= (t < t1 && j >= N) ? 1 : 0;
      kv[u] = *reinterpret_cast<const float4*>(K + static_cast<size_t>(ok[u] ? j : 0) * D + e0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      float dot = __builtin_fmaf(q4.w, kv[u].w, __builtin_fmaf(q4.z, kv[u].z,
                  __builtin_fmaf(q4.y, kv[u].y, q4.x * kv[u].x)));
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, kWave);
      const int t = tb + u * RPI + g;
      if ((l % LPR) == 0 && t < t1) slog[t - t0] = ok[u] ? dot * scale : -INFINITY;
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void logits(const T* qrow, const T* K, const int32_t* row, int t0,
                                       int t1, int N, float scale, float* slog, int& bad) {
  if constexpr (sizeof(T) == 2)
    logits_bf16<D>(qrow, K, row, t0, t1, N, scale, slog, bad);
  else
    logits_f32<D>(qrow, K, row, t0, t1, N, scale, slog, bad);
}

// Logits are kept in base 2: the kernels scale the dot products by
// softmax_scale * log2(e), so e^(x - m) of the natural-base logits is
// 2^(x' - m') of the stored ones, one hardware exp2 each (a -inf logit gives
// exactly 0).
constexpr float kLog2e = 1.44269504088896340736f;

// Softmax numerators in place: slog[t] <- 2^(slog[t] - m).  Returns m (-inf
// when no entry is valid) and the sum.
__device__ __forceinline__ float softmax_weights(float* slog, int n, float& sum) {
  const int l = lane_id();
  float mx = -INFINITY;
  for (int t = l; t < n; t += kWave) mx = fmaxf(mx, slog[t]);
  mx = wave_max(mx);
  float s = 0.0f;
  if (mx != -INFINITY) {
    for (int t = l; t < n; t += kWave) {
      const float x = slog[t];
      const float p = __builtin_amdgcn_exp2f(x - mx);
      slog[t] = p;
      s += p;
    }
  }
  sum = wave_sum(s);
  return mx;
}

// acc <- sum_t w_t V[j_t] over [t0, t1): each row spread over LPR lanes
// (EPL elements each), partial sums reduced across the row groups; lanes of
// group 0 end up holding elements e0 .. e0 + EPL - 1.
template <typename T, int D>
__device__ __forceinline__ void weighted_rows(const T* __restrict__ V,
                                              const int32_t* __restrict__ row, int t0, int t1,
                                              int N, const float* slog,
                                              float (&acc)[Vec<T>::kElems]) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL, RPI = kWave / LPR;
  const int l = lane_id();
  const int g = l / LPR, e0 = (l % LPR) * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  for (int tb = t0; tb < t1; tb += RPI * kUnroll) {
    const int nu = min(kUnroll, (t1 - tb + RPI - 1) / RPI);   // loads holding rows (uniform)
    uint4 vv[kUnroll];
    float wt[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const int jr = row[t - t0];                  // t - t0 < t1 - t0 + RPI: inside the slack
      const float wr = slog[t - t0];
      const int j = t < t1 ? jr : -1;
      const bool ok = j >= 0 && j < N;
      wt[u] = ok ? wr : 0.0f;   // an invalid entry loads row 0 with weight 0
      vv[u] = *reinterpret_cast<const uint4*>(V + static_cast<size_t>(ok ? j : 0) * D + e0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      float vf[EPL];
      Vec<T>::unpack(vv[u], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(wt[u], vf[e], acc[e]);
    }
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      acc[e] = o == 32 ? sum_xor32(acc[e]) : o == 16 ? sum_xor16(acc[e])
                                                   : acc[e] + __shfl_xor(acc[e], o, kWave);
  }
}

// Per-wave LDS of the gather kernels: the entries and the logits of up to k
// entries (+16 slack each: the loops read up to 15 entries past a segment's
// end and discard them, so the reads need no guard).
__host__ __device__ constexpr int gather_slog_floats(int k) { return (k + 16 + 3) / 4 * 4; }
__host__ __device__ constexpr int gather_wave_floats(int k) { return 2 * gather_slog_floats(k); }

// Copies entries [t0, t1) of a global index row to the wave's LDS.
__device__ __forceinline__ void stage_entries(const int32_t* __restrict__ row, int t0, int t1,
                                              int* sidx) {
  for (int t = t0 + lane_id(); t < t1; t += kWave) sidx[t - t0] = row[t];
  wave_sync();
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void gather_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int32_t* __restrict__ idx, int k, int Nq, int Nk, float scale, T* __restrict__ O) {
  // Nq query rows (and idx, O rows) and Nk key rows per head: equal in the
  // forward, one query against a key cache when decoding
  constexpr int EPL = Vec<T>::kElems;
  constexpr int LPR = D / EPL;
  extern __shared__ float slog_all[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform, scalar
  const int l = lane_id();
  float* slog = slog_all + w * gather_wave_floats(k);
  int* sidx = reinterpret_cast<int*>(slog + gather_slog_floats(k));
  const int h = blockIdx.y;
  const int q = blockIdx.x * kWaves + w;
  if (q >= Nq) return;
  const size_t hN = static_cast<size_t>(h) * Nq;
  const T* Kh = K + static_cast<size_t>(h) * Nk * D;
  const T* Vh = V + static_cast<size_t>(h) * Nk * D;
  const int N = Nk;
  stage_entries(idx + (hN + q) * k, 0, k, sidx);
  const int32_t* row = sidx;
  int bad = 0;
  logits<T, D>(Q + (hN + q) * D, Kh, row, 0, k, N, scale * kLog2e, slog, bad);
  if (bad) atomicOr(&g_index_error_flag, 1);
  wave_sync();
  float sum;
  const float mx = softmax_weights(slog, k, sum);
  T* out = O + (hN + q) * D;
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  float acc[EPL];
  if (mx == -INFINITY) {  // no valid entry: zero output
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    if (g == 0) *reinterpret_cast<uint4*>(out + e0) = Vec<T>::pack(acc);
    return;
  }
  wave_sync();
  weighted_rows<T, D>(Vh, row, 0, k, N, slog, acc);
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] /= sum;
    *reinterpret_cast<uint4*>(out + e0) = Vec<T>::pack(acc);
  }
}

// --------------------------------------------- split gather, bf16 rows ---
// The split gather serves the fused forward, whose rows hold keys in [0, N)
// only, so an entry is clamped into range (one v_med3) rather than checked:
// the few slack entries a last partial load reads past the segment (stale
// LDS words) then address a real row, and their results are dropped.  Row
// offsets are 32-bit byte offsets from the head's base (the host keeps the
// head's rows under 4 GiB), and whole blocks of kUnroll loads run as
// straight-line code; only the segment's last partial block tests each load.
template <int D>
__device__ __forceinline__ unsigned row_offset(const int* __restrict__ row, int t, int N,
                                               unsigned lane_off) {
  const int j = min(max(row[t], 0), N - 1);
  return static_cast<unsigned>(j) * static_cast<unsigned>(D * 2) + lane_off;
}

// group_sum over aligned groups of G lanes (G <= 16) for U values at once,
// one butterfly step across all of them at a time: no DPP step then waits
// on the one before it.
template <int G, int U>
__device__ __forceinline__ void group_sum_n(float (&v)[U]) {
  static_assert(G >= 1 && G <= 16 && (G & (G - 1)) == 0, "power-of-two groups up to 16");
  if constexpr (G >= 2) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] += dpp_f<kDppQuadXor1>(v[u]);
  }
  if constexpr (G >= 4) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] += dpp_f<kDppQuadXor2>(v[u]);
  }
  if constexpr (G >= 8) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] += dpp_f<kDppHalfMirror>(v[u]);
  }
  if constexpr (G >= 16) {
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] += dpp_f<kDppMirror>(v[u]);
  }
}

template <int D>
__device__ __forceinline__ void logits_bf16_split(const bf16_t* __restrict__ qrow,
                                                  const bf16_t* __restrict__ Kh,
                                                  const int* __restrict__ row, int n, int N,
                                                  float scale, float* __restrict__ slog) {
  constexpr int EPL = 8, LPR = D / EPL, RPI = kWave / LPR, BLK = RPI * kUnroll;
  const int l = lane_id();
  const int g = l / LPR;
  const unsigned lane_off = static_cast<unsigned>((l % LPR) * EPL * 2);
  const char* kb = reinterpret_cast<const char*>(Kh);
  const uint4 q4 = *reinterpret_cast<const uint4*>(qrow + (l % LPR) * EPL);
  bf16x2 qp[4];
  __builtin_memcpy(qp, &q4, 16);
  auto dot_of = [&](const uint4& kv) {   // this lane's part of the row's dot product
    bf16x2 kp[4];
    __builtin_memcpy(kp, &kv, 16);
    float dot = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) dot = __builtin_amdgcn_fdot2_f32_bf16(kp[i], qp[i], dot, false);
    return dot;
  };
  int tb = 0;
  for (; tb + BLK <= n; tb += BLK) {
    uint4 kv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      kv[u] = *reinterpret_cast<const uint4*>(kb + row_offset<D>(row, tb + u * RPI + g, N, lane_off));
    float dot[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) dot[u] = dot_of(kv[u]);
    group_sum_n<LPR>(dot);
    if ((l % LPR) == 0) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) slog[tb + u * RPI + g] = dot[u] * scale;
    }
  }
  if (tb < n) {
    const int nu = (n - tb + RPI - 1) / RPI;   // loads holding rows (uniform)
    uint4 kv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      kv[u] = *reinterpret_cast<const uint4*>(kb + row_offset<D>(row, tb + u * RPI + g, N, lane_off));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const float dot = group_sum<LPR>(dot_of(kv[u]));
      if ((l % LPR) == 0 && t < n) slog[t] = dot * scale;
    }
  }
}

template <int D>
__device__ __forceinline__ void weighted_rows_bf16_split(const bf16_t* __restrict__ Vh,
                                                         const int* __restrict__ row, int n,
                                                         int N, const float* __restrict__ slog,
                                                         float (&acc)[8]) {
  constexpr int EPL = 8, LPR = D / EPL, RPI = kWave / LPR, BLK = RPI * kUnroll;
  const int l = lane_id();
  const int g = l / LPR;
  const unsigned lane_off = static_cast<unsigned>((l % LPR) * EPL * 2);
  const char* vb = reinterpret_cast<const char*>(Vh);
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
  auto add_row = [&](const uint4& v, float w) {
    float vf[EPL];
    Vec<bf16_t>::unpack(v, vf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = __builtin_fmaf(w, vf[e], acc[e]);
  };
  int tb = 0;
  for (; tb + BLK <= n; tb += BLK) {
    uint4 vv[kUnroll];
    float wt[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = tb + u * RPI + g;
      wt[u] = slog[t];
      vv[u] = *reinterpret_cast<const uint4*>(vb + row_offset<D>(row, t, N, lane_off));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) add_row(vv[u], wt[u]);
  }
  if (tb < n) {
    const int nu = (n - tb + RPI - 1) / RPI;   // loads holding rows (uniform)
    uint4 vv[kUnroll];
    float wt[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const float wr = slog[t];
      wt[u] = t < n ? wr : 0.0f;   // slack entries past the segment weigh nothing
      vv[u] = *reinterpret_cast<const uint4*>(vb + row_offset<D>(row, t, N, lane_off));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      add_row(vv[u], wt[u]);
    }
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1) {
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      acc[e] = o == 32 ? sum_xor32(acc[e]) : o == 16 ? sum_xor16(acc[e])
                                                   : acc[e] + __shfl_xor(acc[e], o, kWave);
  }
}

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
  float m = -INFINITY, lsum = 0.0f;
  if (l < R) {
    m = recs[static_cast<size_t>(l) * (D + 4)];
    if (m != -INFINITY) lsum = recs[static_cast<size_t>(l) * (D + 4) + 1];
  }
  const float M = wave_max(m);
  T* out = O + static_cast<size_t>(q) * D + l * EPM;
  float acc[EPM];
#pragma unroll
  for (int e = 0; e < EPM; ++e) acc[e] = 0.0f;
  if (M == -INFINITY) {  // no valid entry: zero output
#pragma unroll
    for (int e = 0; e < EPM; ++e) out[e] = io<T>::from_f32(0.0f);
    return;
  }
  const float wr = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
  const float L = wave_sum(wr * lsum);
#pragma unroll 4
  for (int r = 0; r < R; ++r) {
    const float wv = __shfl(wr, r, kWave);
    if (wv != 0.0f) {
      const float* a = recs + static_cast<size_t>(r) * (D + 4) + 4 + l * EPM;
#pragma unroll
      for (int e = 0; e < EPM; ++e) acc[e] = __builtin_fmaf(wv, a[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPM; ++e) out[e] = io<T>::from_f32(acc[e] / L);
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

// ------------------------------------------------------------ backward ---
// Backward of the attention over index sets (page "mhpq.cn/news/1098205",
// §2.3: the forward keeps the hard top-k; in the backward the selected
// positions' gradients flow as usual and the others get none; the scorer is
// reached through the selected positions' attention weights).  With
// p_t = softmax(l)_t, dp_t = dO·V[j_t], delta = sum_t p_t dp_t and
// dl_t = p_t (dp_t - delta):
//   G_i = sum_t dl_t K[j_t],  dQ_i = scale · G_i              (row pass)
//   dV_j = sum over (i, t) with j_t = j of p_t dO_i            (key pass)
//   H_j = sum over the same of dl_t Q_i,  dK_j = scale · H_j   (key pass)
// The scorer's gradients need no further gathers: a kept pair's score
// receives its logit's gradient dl_t (straight-through), so
//   dq_low_i = score_scale · sum_t dl_t k_low[j_t] = score_scale · G_i·Pk,
//   dk_low_j = score_scale · H_j·Pq,
// by linearity (bwd.hip computes them from G and H).  With scorer gradients
// the passes store G and H unscaled (out_scale 1), else scale·G and scale·H.
// The row pass writes (p_t, dl_t) in idx's layout; bwd.hip groups them by
// key, and the key pass gathers the rows of the queries that kept each key,
// as the forward gathers key rows.
constexpr int kBwdChunk = 512;     // key-pass entries staged in LDS at a time

__host__ __device__ constexpr int bwd_row_wave_floats(int k) { return 3 * gather_slog_floats(k); }
__host__ __device__ constexpr int bwd_key_wave_floats() { return 3 * gather_slog_floats(kBwdChunk); }

template <int EPL>
__device__ __forceinline__ void store_f32_row(float* dst, const float (&v)[EPL], float f) {
#pragma unroll
  for (int e = 0; e < EPL; e += 4)
    *reinterpret_cast<float4*>(dst + e) = make_float4(v[e] * f, v[e + 1] * f, v[e + 2] * f, v[e + 3] * f);
}

// Cross-group combination for the row pass: lanes holding the same row
// elements in different row groups (xor partners LPR .. 32).
template <int LPR>
__device__ __forceinline__ float groups_sum(float v) {
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
    v = o == 32 ? sum_xor32(v) : o == 16 ? sum_xor16(v) : v + __shfl_xor(v, o, kWave);
  return v;
}
template <int LPR>
__device__ __forceinline__ float groups_max(float v) {
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
    v = o == 32 ? max_xor32(v) : o == 16 ? max_xor16(v) : fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// K pass of the backward row, one read of each kept K row: the logits
// (base 2, into slog) and, per row group over the entries it loads, the sums
//   S = sum e_t, U = sum e_t dp_t, A = sum e_t dp_t K_t, B = sum e_t K_t,
// with e_t = 2^(l_t - m) for the group's running maximum m (the sums are
// rescaled when m grows).  dp_t comes from sdp.  Then
//   p_t = e_t / S, delta = U / S, sum_t dl_t K_t = (A - delta B) / S
// once the groups are combined at the largest m.
template <typename T, int D>
__device__ __forceinline__ void bwd_logits_online(const T* __restrict__ qrow,
                                                  const T* __restrict__ K,
                                                  const int32_t* __restrict__ row, int n, int N,
                                                  float scale2, float* slog,
                                                  const float* sdp, int& bad, float& m,
                                                  float& S, float& U,
                                                  float (&A)[Vec<T>::kElems],
                                                  float (&B)[Vec<T>::kElems]) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL, RPI = kWave / LPR;
  const int l = lane_id();
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  float qf[EPL];
  Vec<T>::unpack(*reinterpret_cast<const uint4*>(qrow + e0), qf);
  m = -INFINITY;
  S = U = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) A[e] = B[e] = 0.0f;
  for (int tb = 0; tb < n; tb += RPI * kUnroll) {
    const int nu = min(kUnroll, (n - tb + RPI - 1) / RPI);   // loads holding rows (uniform)
    uint4 kv[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      const int jr = row[t];                       // t < n + RPI: inside the slack
      const int j = t < n ? jr : -1;
      ok[u] = j >= 0 && j < N;
      bad |= (t < n && j >= N) ? 1 : 0;
      kv[u] = *reinterpret_cast<const uint4*>(K + static_cast<size_t>(ok[u] ? j : 0) * D + e0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (u >= nu) break;
      const int t = tb + u * RPI + g;
      float kf[EPL];
      Vec<T>::unpack(kv[u], kf);
      float dot = 0.0f;
      if constexpr (sizeof(T) == 2) {
        bf16x2 kp[4], qp[4];
        const uint4 q4 = *reinterpret_cast<const uint4*>(qrow + e0);
        __builtin_memcpy(kp, &kv[u], 16);
        __builtin_memcpy(qp, &q4, 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) dot = __builtin_amdgcn_fdot2_f32_bf16(kp[i], qp[i], dot, false);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = __builtin_fmaf(qf[e], kf[e], dot);
      }
      dot = group_sum<LPR>(dot);
      const float lt = ok[u] ? dot * scale2 : -INFINITY;
      if ((l % LPR) == 0 && t < n) slog[t] = lt;
      if (lt > m) {                 // the whole group agrees: lt and m are group values
        const float c = __builtin_amdgcn_exp2f(m - lt);   // m = -inf gives 0
        S *= c;
        U *= c;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          A[e] *= c;
          B[e] *= c;
        }
        m = lt;
      }
      const float ew = ok[u] ? __builtin_amdgcn_exp2f(lt - m) : 0.0f;
      const float ed = ok[u] ? ew * sdp[t] : 0.0f;
      S += ew;
      U += ed;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        A[e] = __builtin_fmaf(ed, kf[e], A[e]);
        B[e] = __builtin_fmaf(ew, kf[e], B[e]);
      }
    }
  }
  // combine the groups at the largest maximum
  const float M = groups_max<LPR>(m);
  const float c = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
  S = groups_sum<LPR>(S * c);
  U = groups_sum<LPR>(U * c);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    A[e] = groups_sum<LPR>(A[e] * c);
    B[e] = groups_sum<LPR>(B[e] * c);
  }
  m = M;
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const int32_t* __restrict__ idx, int k, int N, float scale,
    float out_scale, float* __restrict__ dQ, float2* __restrict__ lpd,
    float4* __restrict__ stats) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int SL = gather_slog_floats(k);
  float* sl = bwd_lds + w * bwd_row_wave_floats(k);      // logits
  float* sd = sl + SL;                                    // dp_t
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const int h = blockIdx.y;
  const int q = blockIdx.x * kWaves + w;
  if (q >= N) return;
  const size_t hN = static_cast<size_t>(h) * N;
  stage_entries(idx + (hN + q) * k, 0, k, sidx);
  int bad = 0;
  // dp_t = dO·V_t first (V rows), then one pass over the K rows
  logits<T, D>(dO + (hN + q) * D, V + hN * D, sidx, 0, k, N, 1.0f, sd, bad);
  wave_sync();
  float m, S, U, A[EPL], B[EPL];
  bwd_logits_online<T, D>(Q + (hN + q) * D, K + hN * D, sidx, k, N, scale * kLog2e, sl, sd, bad,
                          m, S, U, A, B);
  if (bad) atomicOr(&g_index_error_flag, 1);
  wave_sync();
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  // (logit, dp_t) in idx's layout and the row's (max, 1/S, delta): the fill
  // forms p_t and dl_t from them (entries that name no key are never read)
  float2* er = lpd + (hN + q) * static_cast<size_t>(k);
  for (int t = l; t < k; t += kWave) er[t] = make_float2(sl[t], sd[t]);
  float acc[EPL];
  if (m == -INFINITY) {    // no valid entry: no gradient from this row
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    if (g == 0) store_f32_row<EPL>(dQ + (hN + q) * D + e0, acc, 1.0f);
    if (l == 0) stats[hN + q] = make_float4(-INFINITY, 0.0f, 0.0f, 0.0f);
    return;
  }
  const float inv = 1.0f / S;
  const float delta = U * inv;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = (A[e] - delta * B[e]) * inv;
  if (g == 0) store_f32_row<EPL>(dQ + (hN + q) * D + e0, acc, out_scale);
  if (l == 0) stats[hN + q] = make_float4(m, inv, delta, 0.0f);
}

// Row pass, part r of a key-range split (see bwd.hip): the entries of the
// row whose keys lie in [bounds[r], bounds[r+1]) -- one segment of a row
// whose valid entries are an ascending prefix, else the whole row with the
// other keys masked -- give (logit, dp_t) in idx's layout and the part's
// record (m, S, U, -, A[D], B[D]).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_rows_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const T* __restrict__ dO, const int32_t* __restrict__ idx, const int* __restrict__ seg,
    const int* __restrict__ bounds, int k, int N, float scale, float2* __restrict__ lpd,
    float* __restrict__ part) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL, R = kGatherRanges, PS = 2 * D + 4;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  // consecutive workgroups land on consecutive XCDs: part r runs on XCD r
  const int r = static_cast<int>(blockIdx.x) % R;
  const int q = static_cast<int>(blockIdx.x) / R * kWaves + w;
  const int h = blockIdx.y;
  if (q >= N) return;
  const int SL = gather_slog_floats(k);
  float* sl = bwd_lds + w * bwd_row_wave_floats(k);
  float* sd = sl + SL;
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const size_t hN = static_cast<size_t>(h) * N, row = hN + q;
  const int* sg = seg + row * (R + 1);
  const bool sorted = __builtin_amdgcn_readfirstlane(sg[0]) >= 0;
  const int t0 = sorted ? __builtin_amdgcn_readfirstlane(sg[r]) : 0;
  const int t1 = sorted ? __builtin_amdgcn_readfirstlane(sg[r + 1]) : k;
  float* rec = part + (row * R + r) * PS;
  if (t0 >= t1) {
    if (l == 0) rec[0] = -INFINITY;   // empty part: the merge skips it
    return;
  }
  const int lo = bounds[h * (R + 1) + r], hi = bounds[h * (R + 1) + r + 1];
  const int32_t* ir = idx + row * k;
  const int n = t1 - t0;
  for (int t = l; t < n; t += kWave) {
    const int j = ir[t0 + t];
    sidx[t] = j >= lo && j < hi ? j : -1;
  }
  wave_sync();
  int bad = 0;
  logits<T, D>(dO + row * D, V + hN * D, sidx, 0, n, N, 1.0f, sd, bad);
  wave_sync();
  float m, S, U, A[EPL], B[EPL];
  bwd_logits_online<T, D>(Q + row * D, K + hN * D, sidx, n, N, scale * kLog2e, sl, sd, bad, m, S,
                          U, A, B);
  wave_sync();
  float2* er = lpd + row * k + t0;
  for (int t = l; t < n; t += kWave)
    if (sidx[t] >= 0) er[t] = make_float2(sl[t], sd[t]);
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < EPL; e += 4) {
      *reinterpret_cast<float4*>(rec + 4 + e0 + e) = make_float4(A[e], A[e + 1], A[e + 2], A[e + 3]);
      *reinterpret_cast<float4*>(rec + 4 + D + e0 + e) =
          make_float4(B[e], B[e + 1], B[e + 2], B[e + 3]);
    }
  }
  if (l == 0) *reinterpret_cast<float4*>(rec) = make_float4(m, S, U, 0.0f);
}

// Key pass, part r: the key's records from rows of slices [r S/8, (r+1) S/8)
// (consecutive in its segment) give the part's (dV[D], H[D]).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_keys_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ dO, const int* __restrict__ seg_off,
    const int* __restrict__ seg_cnt, const int* __restrict__ slice_pre, int S, long long total,
    const BwdEntry* __restrict__ rec, int N, int k, float* __restrict__ part) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL, R = kGatherRanges;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  const int r = static_cast<int>(blockIdx.x) % R;
  const int j = static_cast<int>(blockIdx.x) / R * kWaves + w;
  const int h = blockIdx.y;
  if (j >= N) return;
  constexpr int SL = gather_slog_floats(kBwdChunk);
  float* sp = bwd_lds + w * bwd_key_wave_floats();
  float* sd = sp + SL;
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const size_t hN = static_cast<size_t>(h) * N, key = hN + j;
  const int s0 = r * (S / R), s1 = (r + 1) * (S / R);
  const int a0 = slice_pre[static_cast<size_t>(s0) * total + key];
  const int a1 = s1 < S ? slice_pre[static_cast<size_t>(s1) * total + key] : seg_cnt[key];
  const size_t o0 = hN * static_cast<size_t>(k) + static_cast<unsigned>(seg_off[key] + a0);
  const int n = a1 - a0;
  const unsigned uk = static_cast<unsigned>(k);
  const T* Qh = Q + hN * D;
  const T* dOh = dO + hN * D;
  float av[EPL], ak[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) av[e] = ak[e] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kBwdChunk) {
    const int m = min(kBwdChunk, n - c0);
    for (int t = l; t < m; t += kWave) {
      const BwdEntry re = rec[o0 + c0 + t];
      sidx[t] = static_cast<int>(static_cast<unsigned>(re.e) / uk);
      sp[t] = re.p;
      sd[t] = re.dl;
    }
    wave_sync();
    float tmp[EPL];
    weighted_rows<T, D>(dOh, sidx, 0, m, N, sp, tmp);
#pragma unroll
    for (int e = 0; e < EPL; ++e) av[e] += tmp[e];
    weighted_rows<T, D>(Qh, sidx, 0, m, N, sd, tmp);
#pragma unroll
    for (int e = 0; e < EPL; ++e) ak[e] += tmp[e];
    wave_sync();
  }
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  float* pr = part + (key * R + r) * 2 * D;
  if (g == 0) {
    store_f32_row<EPL>(pr + e0, av, 1.0f);
    store_f32_row<EPL>(pr + D + e0, ak, 1.0f);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) void bwd_keys_kernel(
    const T* __restrict__ Q, const T* __restrict__ dO, const int* __restrict__ seg_off,
    const int* __restrict__ seg_cnt, const BwdEntry* __restrict__ rec, int N, int k,
    float out_scale, float* __restrict__ dK, float* __restrict__ dV) {
  constexpr int EPL = Vec<T>::kElems, LPR = D / EPL;
  extern __shared__ float bwd_lds[];
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  constexpr int SL = gather_slog_floats(kBwdChunk);
  float* sp = bwd_lds + w * bwd_key_wave_floats();
  float* sd = sp + SL;
  int* sidx = reinterpret_cast<int*>(sd + SL);
  const int h = blockIdx.y;
  const int j = blockIdx.x * kWaves + w;
  if (j >= N) return;
  const size_t hN = static_cast<size_t>(h) * N;
  const T* Qh = Q + hN * D;
  const T* dOh = dO + hN * D;
  const size_t o0 = hN * static_cast<size_t>(k) + static_cast<unsigned>(seg_off[hN + j]);
  const int n = seg_cnt[hN + j];
  const unsigned uk = static_cast<unsigned>(k);
  float av[EPL], ak[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) av[e] = ak[e] = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kBwdChunk) {
    const int m = min(kBwdChunk, n - c0);
    for (int t = l; t < m; t += kWave) {
      const BwdEntry r = rec[o0 + c0 + t];
      sidx[t] = static_cast<int>(static_cast<unsigned>(r.e) / uk);   // e = i*k + t
      sp[t] = r.p;
      sd[t] = r.dl;
    }
    wave_sync();
    float tmp[EPL];
    weighted_rows<T, D>(dOh, sidx, 0, m, N, sp, tmp);
#pragma unroll
    for (int e = 0; e < EPL; ++e) av[e] += tmp[e];
    weighted_rows<T, D>(Qh, sidx, 0, m, N, sd, tmp);
#pragma unroll
    for (int e = 0; e < EPL; ++e) ak[e] += tmp[e];
    wave_sync();    // the chunk's LDS is read before the next one is staged
  }
  const int g = l / LPR, e0 = (l % LPR) * EPL;
  if (g == 0) {
    store_f32_row<EPL>(dV + (hN + j) * D + e0, av, 1.0f);
    store_f32_row<EPL>(dK + (hN + j) * D + e0, ak, out_scale);
  }
}

template <typename T, int D>
hipError_t bwd_passes_t(const BwdArgs& a, hipStream_t s) {
  static std::atomic<int> lds_rows[kMaxDevices], lds_keys[kMaxDevices];
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_rows_kernel<T, D>),
                                    kWaves * bwd_row_wave_floats(kKMax) * 4, lds_rows);
  if (e != hipSuccess) return e;
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_keys_kernel<T, D>),
                         kWaves * bwd_key_wave_floats() * 4, lds_keys);
  if (e != hipSuccess) return e;
  static std::atomic<int> lds_rs[kMaxDevices], lds_ks[kMaxDevices];
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_rows_split_kernel<T, D>),
                         kWaves * bwd_row_wave_floats(kKMax) * 4, lds_rs);
  if (e != hipSuccess) return e;
  e = set_lds_limit_once(reinterpret_cast<const void*>(&bwd_keys_split_kernel<T, D>),
                         kWaves * bwd_key_wave_floats() * 4, lds_ks);
  if (e != hipSuccess) return e;
  const int nb = (a.N + kWaves - 1) / kWaves;
  const dim3 grid(nb, a.nh), grid_split(nb * kGatherRanges, a.nh);
  const float out_scale = a.scorer ? 1.0f : a.scale;
  const size_t lds_r = static_cast<size_t>(kWaves) * bwd_row_wave_floats(a.k) * 4;
  const size_t lds_k = static_cast<size_t>(kWaves) * bwd_key_wave_floats() * 4;
  if (a.pass == 0 && !a.split_rows) {
    hipLaunchKernelGGL((bwd_rows_kernel<T, D>), grid, dim3(kThreads), lds_r, s,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                       static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.idx, a.k, a.N,
                       a.scale, out_scale, a.dQ, a.epd, a.stats);
  } else if (a.pass == 0) {
    hipLaunchKernelGGL((bwd_rows_split_kernel<T, D>), grid_split, dim3(kThreads), lds_r, s,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.K),
                       static_cast<const T*>(a.V), static_cast<const T*>(a.dO), a.idx,
                       a.row_seg, a.bounds, a.k, a.N, a.scale, a.epd, a.part);
  } else if (!a.split_keys) {
    hipLaunchKernelGGL((bwd_keys_kernel<T, D>), grid, dim3(kThreads), lds_k, s,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.dO), a.seg_off,
                       a.seg_cnt, a.rec, a.N, a.k, out_scale, a.dK, a.dV);
  } else {
    hipLaunchKernelGGL((bwd_keys_split_kernel<T, D>), grid_split, dim3(kThreads), lds_k, s,
                       static_cast<const T*>(a.Q), static_cast<const T*>(a.dO), a.seg_off,
                       a.seg_cnt, a.slice_pre, a.slices, static_cast<long long>(a.nh) * a.N,
                       a.rec, a.N, a.k, a.part);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_pass(const BwdArgs& a, hipStream_t s) {
  if (a.dtype == 0) {
    if (a.D == 64) return bwd_passes_t<float, 64>(a, s);
    if (a.D == 128) return bwd_passes_t<float, 128>(a, s);
  } else {
    if (a.D == 64) return bwd_passes_t<bf16_t, 64>(a, s);
    if (a.D == 128) return bwd_passes_t<bf16_t, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

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
