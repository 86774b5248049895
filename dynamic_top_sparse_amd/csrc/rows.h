// Per-wave row helpers shared by the gather attention (gather.hip) and the
// backward's passes (bwd.hip): one wavefront streams the K or V rows named by
// an index row with 16-byte loads, several loads in flight per lane.
#pragma once

#include "sa_internal.h"

namespace sa {
namespace {

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

}  // namespace
}  // namespace sa
