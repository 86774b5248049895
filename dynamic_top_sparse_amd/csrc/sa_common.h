// Device-side helpers shared by the kernels of libsparse_attn (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef uint16_t bf16_t;  // storage of a bfloat16 value
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kWave = 64;

// ------------------------------------------------------------ conversion ---
__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 for finite values.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
  __device__ __forceinline__ static float from_f32(float v) { return v; }
};
template <> struct io<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// ------------------------------------------------------------- ordering ---
// Monotone map of fp32 onto uint32: a < b  <=>  key(a) < key(b); -0.0 and
// +0.0 map to the same key (equal scores tie, and the tie goes to the lower
// key index).
__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.0f) f = 0.0f;  // canonicalise -0.0
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ---------------------------------------------------------- exact score ---
// The fp32 score that decides the selection: the dot product of the fp32
// low-dimensional rows, accumulated with fused multiply-adds in ascending
// coordinate order, then multiplied by score_scale.  Every kernel that needs
// the exact score (re-rank, fallback, dump) calls this one function.
template <int DP>
__device__ __forceinline__ float exact_score(const float* __restrict__ q,
                                             const float* __restrict__ k, float scale) {
  float acc = 0.0f;
#pragma unroll
  for (int c = 0; c < DP; ++c) acc = __builtin_fmaf(q[c], k[c], acc);
  return acc * scale;
}

// Margin between the bf16 MFMA score and the exact fp32 score of query
// (qn = ||q_low||, qr = ||q_low - bf16(q_low)||) against any key of the
// head (kn = max ||k_low||, kr = max residual).  With q~, k~ the bf16 rows:
//   q·k - q~·k~ = q·(k - k~) + (q - q~)·k~,  |.| <= qn*kr + qr*||k~||
// and ||k~|| <= kn (1 + 2^-8).  Both the MFMA and the exact dot product add
// at most d_proj rounding errors of 2^-23 relative to qn*kn each (d_proj <=
// 128), covered with ample room by the 2^-13 term; the final 2^-10 factor
// and the absolute floor cover the rounding of this expression itself and
// flushed subnormals.
__device__ __forceinline__ float score_margin(float qn, float qr, float kn, float kr,
                                              float scale) {
  const float m = scale * (qn * kr + (1.01f * qr + 0.0001220703125f * qn) * kn);
  return m * (1.0f + 1.0f / 1024.0f) + 1e-28f;
}

// ------------------------------------------------------ wave primitives ---
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}

// --------------------------------------------------- workspace header ---
// A few counters at the start of the workspace (all int64 / int32).
struct WsHeader {
  unsigned long long fallback_queries;   // resolved by the exact fallback
  unsigned long long overflow_queries;   // candidate buffer too small
  unsigned long long candidates;         // candidates written by the filter
  unsigned long long rescored;           // keys re-scored exactly in the re-rank
  unsigned long long queries;            // queries processed
  unsigned int key_norm_max;             // max ||k_low|| of the chunk (fp32 bits)
  unsigned int key_res_max;              // max ||k_low - bf16(k_low)|| (fp32 bits)
  unsigned int fb_count;                 // queries queued for the fallback
  unsigned int fb_next;                  // fallback work-queue cursor
  unsigned int pad[6];
};
static_assert(sizeof(WsHeader) % 16 == 0, "header keeps 16-byte alignment");

}  // namespace sa
