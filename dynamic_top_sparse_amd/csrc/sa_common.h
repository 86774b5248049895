// Device-side helpers shared by the kernels of libsparse_attn (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef uint16_t bf16_t;  // storage of a bfloat16 value
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));   // operand of the bf16 dot2 instruction

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
// Non-negative values get the sign bit set, negative ones all bits flipped:
// u ^ ((u >> 31, arithmetic) | sign bit), with no compare or select.  Adding
// +0.0 first turns -0.0 into +0.0 (round to nearest) and changes nothing else.
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}
// Inverse on keys of non-NaN values: a key with the sign bit set came from a
// non-negative value (clear the bit), any other from a negative one (flip all).
__device__ __forceinline__ float key_to_float(uint32_t k) {
  const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(k) >> 31);
  return __uint_as_float(k ^ (~m | 0x80000000u));
}

// ---------------------------------------------------------- exact score ---
// The fp32 score that decides the selection, in one fixed evaluation order
// shared by every kernel that needs it (re-rank, fallback, dump):
//   p_g = q[4g]k[4g] + q[4g+1]k[4g+1] + ... as a chain of fused multiply-adds
//         over the 4 coordinates of group g (g = 0 .. DP/4-1),
//   then an xor-butterfly over the groups: at step o (1, 2, ..., DP/8) every
//   p_g becomes p_g + p_{g^o}; the result is p_0 · scale.
// A wavefront evaluates it with one lane per group and group_sum() (whose
// steps are exactly these); exact_score() below is the same arithmetic for
// one thread.
template <int DP>
__device__ __forceinline__ float group_partial(const float4 q, const float4 k) {
  return __builtin_fmaf(q.w, k.w, __builtin_fmaf(q.z, k.z, __builtin_fmaf(q.y, k.y,
         __builtin_fmaf(q.x, k.x, 0.0f))));
}

template <int DP>
__device__ __forceinline__ float exact_score(const float* __restrict__ q,
                                             const float* __restrict__ k, float scale) {
  constexpr int G = DP / 4;
  float p[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    p[g] = group_partial<DP>(make_float4(q[4 * g], q[4 * g + 1], q[4 * g + 2], q[4 * g + 3]),
                             make_float4(k[4 * g], k[4 * g + 1], k[4 * g + 2], k[4 * g + 3]));
#pragma unroll
  for (int o = 1; o < G; o <<= 1) {
    float t[G];
#pragma unroll
    for (int g = 0; g < G; ++g) t[g] = p[g] + p[g ^ o];
#pragma unroll
    for (int g = 0; g < G; ++g) p[g] = t[g];
  }
  return p[0] * scale;
}

// ------------------------------------------------- 16-bit filter operands ---
// The filter scores pairs with a 16-bit MFMA (fp16 by default, bf16 as an
// option).  Rows are scaled by a power of two before rounding so that the
// largest element lands in [2^14, 2^15): each query row has its own exponent
// e_q, each key head one exponent E for all its keys.  Elements that would
// become subnormal are flushed to zero; the residual norms below include
// them, so no precision assumption about the MFMA is needed.
__device__ __forceinline__ int scale_exponent(float maxabs) {
  if (!(maxabs > 0.0f)) return 0;
  int p;
  (void)__builtin_frexpf(maxabs, &p);       // maxabs = f * 2^p, f in [0.5, 1)
  const int e = 15 - p;
  return e < -64 ? -64 : (e > 64 ? 64 : e);
}

struct FiltF16 {
  typedef __attribute__((ext_vector_type(8))) _Float16 vec8;
  __device__ __forceinline__ static uint16_t round(float x) {
    if (fabsf(x) < 6.103515625e-05f) x = 0.0f;   // below the fp16 normal range
    const _Float16 h = static_cast<_Float16>(x);
    uint16_t u;
    __builtin_memcpy(&u, &h, 2);
    return u;
  }
  __device__ __forceinline__ static float back(uint16_t u) {
    _Float16 h;
    __builtin_memcpy(&h, &u, 2);
    return static_cast<float>(h);
  }
  __device__ __forceinline__ static f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
    vec8 va, vb;
    __builtin_memcpy(&va, &a, 16);
    __builtin_memcpy(&vb, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(va, vb, c, 0, 0, 0);
  }
};

struct FiltBf16 {
  __device__ __forceinline__ static uint16_t round(float x) {
    if (fabsf(x) < 1.1754943508e-38f) x = 0.0f;  // below the fp32/bf16 normal range
    return f32_to_bf16(x);
  }
  __device__ __forceinline__ static float back(uint16_t u) { return bf16_to_f32(u); }
  __device__ __forceinline__ static f32x16 mfma(uint4 a, uint4 b, f32x16 c) {
    bf16x8 va, vb;
    __builtin_memcpy(&va, &a, 16);
    __builtin_memcpy(&vb, &b, 16);
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, vb, c, 0, 0, 0);
  }
};

// Margin between the 16-bit MFMA score and the exact fp32 score of a query
// (qn = ||q_low||, qr = ||q_low - q~||, q~ the rounded row in true units)
// against any key of the head (kn = max ||k_low||, kr = max ||k_low - k~||):
//   q·k - q~·k~ = q·(k - k~) + (q - q~)·k~,   |.| <= qn*kr + qr*||k~||,
// with ||k~|| <= kn (1 + 2^-8).  The MFMA sum and the exact fp32 evaluation
// each add at most (d_proj + 8) roundings of 2^-23 relative to qn*kn
// (covered twice by the eps term); the final factor and the absolute floor
// cover the rounding of this expression and flushed tiny values.
__device__ __forceinline__ float score_margin(float qn, float qr, float kn, float kr,
                                              float scale, int dp) {
  const float eps = static_cast<float>(dp + 16) * (1.0f / 4194304.0f);
  const float m = scale * (qn * kr + (1.01f * qr + eps * qn) * kn);
  return m * (1.0f + 1.0f / 1024.0f) + 1e-28f;
}

// ------------------------------------------------------ wave primitives ---
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// v[l] + v[l ^ 16] (or ^ 32) in every lane.  gfx950's permlane swaps move
// rows 1 and 3 of one register into rows 0 and 2 of another (the 32 variant:
// the upper half into the lower); swapping a register with itself leaves
// each lane holding its own value and its partner's, one in each result.
// These are VALU operations, unlike a shuffle through the LDS crossbar.
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Lane partners inside a 16-lane row through DPP (VALU, no LDS): swaps of
// neighbours and of pairs in each quad, then the mirrors of each half-row
// and of the row.  Applied in that order, each step combines two disjoint
// groups that already agree, so a reduction leaves every lane of the row
// with the same value.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // row_half_mirror
constexpr int kDppMirror = 0x140;       // row_mirror
template <int Ctrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}
template <int Ctrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, Ctrl, 0xF, 0xF, false);
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
  v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return v;
}

// Sum over aligned groups of G lanes (G a power of two up to 64), every lane
// of a group getting the group's sum.  The steps are the xor-butterfly with
// partners l^1, l^2, l^4, l^8, l^16, l^32 in that order: the mirror steps
// pair a lane with l^7 or l^15, which at that point hold the same values as
// l^4 and l^8.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "power-of-two groups");
  if constexpr (G >= 2) v += dpp_f<kDppQuadXor1>(v);
  if constexpr (G >= 4) v += dpp_f<kDppQuadXor2>(v);
  if constexpr (G >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (G >= 32) v = sum_xor16(v);
  if constexpr (G >= 64) v = sum_xor32(v);
  return v;
}

__device__ __forceinline__ float wave_max(float v) { return row_max16(max_xor16(max_xor32(v))); }
__device__ __forceinline__ float wave_sum(float v) { return row_sum16(sum_xor16(sum_xor32(v))); }
__device__ __forceinline__ int wave_sum_i(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  v = static_cast<int>(r[0] + r[1]);
  r = __builtin_amdgcn_permlane16_swap(static_cast<unsigned>(v), static_cast<unsigned>(v), false, false);
  v = static_cast<int>(r[0] + r[1]);
  v += dpp_i<kDppQuadXor1>(v);
  v += dpp_i<kDppQuadXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  v += dpp_i<kDppMirror>(v);
  return v;
}
// Inclusive prefix sum over the wave: a Hillis-Steele scan inside each
// 16-lane row (DPP row shifts; a lane with no source within its row adds 0),
// then the totals of the rows before are added from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111>(v);   // row_shr:1
  v += dpp_i<0x112>(v);   // row_shr:2
  v += dpp_i<0x114>(v);   // row_shr:4
  v += dpp_i<0x118>(v);   // row_shr:8
  const int row = lane_id() >> 4;
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// --------------------------------------------------- workspace header ---
// A few counters at the start of the workspace (all int64 / int32).
struct WsHeader {
  unsigned long long fallback_queries;   // resolved by the exact fallback
  unsigned long long overflow_queries;   // candidate lists overflowed (first pass)
  unsigned long long candidates;         // candidates written by the filter
  unsigned long long rescored;           // keys re-scored exactly in the re-rank
  unsigned long long queries;            // queries resolved
  unsigned long long retried;            // queries filtered again with a proven threshold
  unsigned int fb_count;                 // queries queued for the fallback
  unsigned int fb_next;                  // fallback work-queue cursor
  unsigned int margin_violations;        // re-scored keys outside [s~ - m, s~ + m]
  unsigned int wide_queries;             // re-ranked from their lists in memory
};
static_assert(sizeof(WsHeader) % 16 == 0, "header keeps 16-byte alignment");

}  // namespace sa
