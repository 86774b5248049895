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

// --------------------------------------------- split gather, bf16 rows ---
// Rows whose entries all hold keys in [0, N) (the fused forward's rows, and
// the backward's part segments) are read as trusted: an entry is clamped
// into range (one v_med3) rather than checked:
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

}  // namespace
}  // namespace sa
