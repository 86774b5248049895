// The scorer contraction on 16-bit MFMA and the streaming per-query filter
// (page "mhpq.cn/news/1098205", §2.2: scores are scaled dot products of the
// low-dimensional rows, S = d_proj^-1/2 · q_low·k_lowᵀ; §3.2: torch.topk
// keeps the k best keys per query).  No score matrix is ever written: tiles of
// 32 keys x 32 queries live in MFMA accumulators and are reduced on the spot.
//
// The 16-bit MFMA result s~ differs from the exact fp32 score s by at most a
// margin m_i per query (a Cauchy-Schwarz bound built from the row norms the
// projection kernel stores).  The filter therefore proves, rather than
// guesses, that it keeps every key of the exact top-k:
//   1. sample pass: every 16th key is scored and each lane keeps the maximum
//      of its 16 rows per tile ("block maxima");
//   2. threshold: tau_i is (a lower rounding of) the r-th largest block
//      maximum, r = ceil(beta * k * sample / valid keys);
//   3. filter pass: every valid key with s~ >= tau_i - m_i is appended to the
//      query's candidate list.
// The re-rank kernel then checks that at least k candidates have
// s~ - m_i >= tau_i; that makes tau_i a lower bound of the k-th best exact
// score, so no key outside the list can belong to the top-k.  Queries whose
// check fails, or whose list overflows, are handed to the exact fallback.
//
// MFMA orientation (v_mfma_f32_32x32x16_f16 or _bf16, by the filter
// precision): A = 32 keys from LDS, B = 32 queries held in registers.  Lane l then owns query l%32 and, in its 16
// accumulators, keys 8*(r/4) + 4*(l/32) + r%4 of the tile, so the threshold
// is one register per lane and each lane appends to its own list.
#include <float.h>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kWaveQueries = 64;

template <int DP>
struct Tile {
  static constexpr int kUnits = DP / 8;          // 16-byte units per key row
  static constexpr int kKSteps = DP / 16;        // MFMA k-steps
  static constexpr int kChunkUnits = kKeysPerChunk * kUnits;
};

// Swizzled position (in 16-byte units) of unit u of key row `key` within a
// staged chunk: the XOR spreads the 32 rows an A-fragment read touches over
// the LDS banks.
template <int DP>
__device__ __forceinline__ int lds_unit(int key, int u) {
  constexpr int U = Tile<DP>::kUnits;
  return key * U + (u ^ (key & (U - 1)));
}

// A thread's share of a staged key chunk is held in a plain register array
// between the global loads (issued a chunk ahead) and the LDS writes.
template <int DP>
struct Stage {
  static constexpr int kPerThread = Tile<DP>::kChunkUnits / kThreads;
};

// (native clang vectors: HIP's uint4 wrapper keeps the array in scratch)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DP>
__device__ __forceinline__ void chunk_load(u32x4 (&r)[Stage<DP>::kPerThread],
                                           const bf16_t* __restrict__ rows, int key0) {
  const u32x4* src = reinterpret_cast<const u32x4*>(rows + static_cast<size_t>(key0) * DP);
#pragma unroll
  for (int i = 0; i < Stage<DP>::kPerThread; ++i) r[i] = src[threadIdx.x + i * kThreads];
}

template <int DP>
__device__ __forceinline__ void chunk_store(const u32x4 (&r)[Stage<DP>::kPerThread],
                                            uint4* __restrict__ lds) {
  constexpr int U = Tile<DP>::kUnits;
  u32x4* dst = reinterpret_cast<u32x4*>(lds);
#pragma unroll
  for (int i = 0; i < Stage<DP>::kPerThread; ++i) {
    const int e = threadIdx.x + i * kThreads;
    dst[lds_unit<DP>(e / U, e % U)] = r[i];
  }
}

// B fragments (queries) of one 32-query block: lane l holds query row l%32,
// model coordinates [16*ks + 8*(l/32), +8), as raw 16-bit values.
template <int DP>
__device__ __forceinline__ void load_query_frags(uint4 (&b)[Tile<DP>::kKSteps],
                                                 const bf16_t* __restrict__ q16, int q) {
  const int l = lane_id();
  const uint4* row = reinterpret_cast<const uint4*>(q16 + static_cast<size_t>(q) * DP);
#pragma unroll
  for (int ks = 0; ks < Tile<DP>::kKSteps; ++ks) b[ks] = row[2 * ks + (l >> 5)];
}

template <int DP, typename F>
__device__ __forceinline__ f32x16 tile_scores(const uint4* __restrict__ lds, int tile_in_chunk,
                                              const uint4 (&b)[Tile<DP>::kKSteps]) {
  const int l = lane_id();
  const int key = tile_in_chunk * 32 + (l & 31);
  f32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < Tile<DP>::kKSteps; ++ks)
    acc = F::mfma(lds[lds_unit<DP>(key, 2 * ks + (l >> 5))], b[ks], acc);
  return acc;
}

// Factor that turns a raw MFMA sum of query q into its filter score
// s~ = sum * 2^-(e_q + E) * score_scale (exact power-of-two rescaling).
__device__ __forceinline__ float score_factor(float qinv, float kinv, float scale) {
  return scale * qinv * kinv;
}

// Key row of accumulator r for this lane, relative to the tile base.
__device__ __forceinline__ int acc_row(int r, int half) {
  return 8 * (r >> 2) + 4 * half + (r & 3);
}

// ------------------------------------------------------------ sample pass ---
template <int DP, typename F>
__global__ __launch_bounds__(kThreads) void sample_maxima_kernel(
    const bf16_t* __restrict__ q16, const bf16_t* __restrict__ samp,
    const float4* __restrict__ qstat, const uint32_t* __restrict__ kstat, float scale, int N,
    int Npad, int Ns, int NB, int causal, float* __restrict__ bm) {
  __shared__ uint4 lds[2 * Tile<DP>::kChunkUnits];
  const int h = blockIdx.y;
  const int q0 = blockIdx.x * kQueriesPerBlock;
  const int w = threadIdx.x >> 6;
  const int l = lane_id();
  const int half = l >> 5;
  const int qw = q0 + w * kWaveQueries;
  const bf16_t* qh = q16 + static_cast<size_t>(h) * Npad * DP;
  const bf16_t* sh = samp + static_cast<size_t>(h) * (Npad / kSampleStride) * DP;
  float* bmh = bm + static_cast<size_t>(h) * NB * Npad;

  uint4 b0[Tile<DP>::kKSteps], b1[Tile<DP>::kKSteps];
  load_query_frags<DP>(b0, qh, qw + (l & 31));
  load_query_frags<DP>(b1, qh, qw + 32 + (l & 31));
  const int qa = qw + (l & 31), qb = qw + 32 + (l & 31);
  const float kinv = __builtin_ldexpf(
      1.0f, -scale_exponent(__uint_as_float(kstat[kKeyStatWords * h + 2])));
  const float fa = score_factor(qstat[static_cast<size_t>(h) * Npad + qa].z, kinv, scale);
  const float fb = score_factor(qstat[static_cast<size_t>(h) * Npad + qb].z, kinv, scale);

  // sample keys t with stride*t <= last query of the block (causal), else all
  int s_end = Ns;
  if (causal) s_end = min(Ns, (min(N, q0 + kQueriesPerBlock) - 1) / kSampleStride + 1);
  const int nchunks = (s_end + kKeysPerChunk - 1) / kKeysPerChunk;
  u32x4 regs[Stage<DP>::kPerThread];
  chunk_load<DP>(regs, sh, 0);
  chunk_store<DP>(regs, lds);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const bool more = ch + 1 < nchunks;
    if (more) chunk_load<DP>(regs, sh, (ch + 1) * kKeysPerChunk);
    const uint4* buf = lds + (ch & 1) * Tile<DP>::kChunkUnits;
#pragma unroll 1
    for (int tt = 0; tt < kKeysPerChunk / 32; ++tt) {
      const int tbase = ch * kKeysPerChunk + tt * 32;
      if (tbase >= s_end) break;
      f32x16 a0 = tile_scores<DP, F>(buf, tt, b0);
      f32x16 a1 = tile_scores<DP, F>(buf, tt, b1);
      float m0 = -INFINITY, m1 = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = tbase + acc_row(r, half);
        const int j = t * kSampleStride;
        const bool ok = t < s_end;
        const bool ok0 = ok && (!causal || j <= qa);
        const bool ok1 = ok && (!causal || j <= qb);
        m0 = fmaxf(m0, ok0 ? a0[r] : -INFINITY);
        m1 = fmaxf(m1, ok1 ? a1[r] : -INFINITY);
      }
      const int tile = tbase / 32;
      bmh[static_cast<size_t>(2 * tile + half) * Npad + qa] = m0 * fa;
      bmh[static_cast<size_t>(2 * tile + half) * Npad + qb] = m1 * fb;
    }
    if (more) chunk_store<DP>(regs, lds + ((ch + 1) & 1) * Tile<DP>::kChunkUnits);
    __syncthreads();
  }
}

// -------------------------------------------------------------- threshold ---
// One thread per query: a 4-bit-digit radix select over the top 16 bits of
// the block maxima's order keys gives a value <= the r-th largest block
// maximum (rounding down only adds candidates).
__global__ __launch_bounds__(kThreads) void threshold_kernel(
    const float* __restrict__ bm, int N, int Npad, int Ns, int NB, int k, int causal, int capH,
    float beta, float* __restrict__ tau) {
  __shared__ int hist[16 * kThreads];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int q = blockIdx.x * kThreads + tid;
  const float* bmh = bm + static_cast<size_t>(h) * NB * Npad;
  if (q >= Npad) return;  // whole-block uniform: Npad is a multiple of 256
  float result = -INFINITY;
  const int n_valid = causal ? q + 1 : N;
  const bool active = q < N && n_valid > 2 * capH - 64;
  const int ns_valid = causal ? min(Ns, q / kSampleStride + 1) : Ns;
  const int nb = 2 * ((ns_valid + 31) / 32);
  const int k_i = min(k, n_valid);
  int r = static_cast<int>(ceilf(beta * static_cast<float>(k_i) * static_cast<float>(ns_valid) /
                                  static_cast<float>(n_valid)));
  r = max(1, min(r, nb));
  uint32_t prefix = 0;
  int K = r;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 28 - 4 * pass;
    const uint32_t pmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 4));
#pragma unroll
    for (int d = 0; d < 16; ++d) hist[d * kThreads + tid] = 0;
    if (active) {
      for (int e = 0; e < nb; ++e) {
        const uint32_t key = order_key(bmh[static_cast<size_t>(e) * Npad + q]);
        if ((key & pmask) == prefix) hist[((key >> shift) & 15u) * kThreads + tid] += 1;
      }
      int cum = 0, digit = 0;
      for (int d = 15; d >= 0; --d) {
        const int c = hist[d * kThreads + tid];
        if (cum + c >= K) { digit = d; break; }
        cum += c;
      }
      K -= cum;
      prefix |= static_cast<uint32_t>(digit) << shift;
    }
  }
  if (active) {
    // block maxima are stored as filter scores already (score factor applied)
    if (prefix > order_key(-INFINITY)) result = key_to_float(prefix);
  }
  tau[static_cast<size_t>(h) * Npad + q] = active ? result : -INFINITY;
}

// ------------------------------------------------------------ filter pass ---
// Bit r of the result is set when accumulator r misses the threshold: the
// sign bit of v - thr is shifted in with one v_alignbit per accumulator
// (v >= thr exactly when v - thr >= +0; masked -inf scores always miss).
__device__ __forceinline__ unsigned miss_bits(const f32x16& a, float thr) {
  unsigned nb = 0;
#pragma unroll
  for (int r = 15; r >= 0; --r) nb = __builtin_amdgcn_alignbit(nb, __float_as_uint(a[r] - thr), 31);
  return nb;
}

// Rows of a lane's accumulators are key offsets r + (r & 12) (+4 for the
// upper half-wave), increasing in r, so the keys beyond `lim` (relative to
// the lane's first key) form a suffix of r.  Returns the mask of the valid
// accumulators.
__device__ __forceinline__ unsigned valid_rows(int lim) {
  if (lim < 0) return 0u;
  int r0 = min(4, lim + 1) + min(4, max(0, lim - 7)) + min(4, max(0, lim - 15)) +
           min(4, max(0, lim - 23));
  return r0 >= 16 ? 0xFFFFu : ((1u << r0) - 1u);
}


template <int DP, typename F>
__global__ __launch_bounds__(kThreads) void filter_kernel(
    const bf16_t* __restrict__ q16, const bf16_t* __restrict__ k16,
    const float4* __restrict__ qstat, const uint32_t* __restrict__ kstat,
    const float* __restrict__ tau, int N, int Npad, int causal, int capH, float scale,
    const int* __restrict__ qlist, const int* __restrict__ qlist_count,
    uint2* __restrict__ cand, int* __restrict__ cnt, WsHeader* __restrict__ hdr) {
  __shared__ uint4 lds[2 * Tile<DP>::kChunkUnits];
  __shared__ float4 stash_all[8 * kThreads];   // 32 scores per lane, [8][threads]
  __shared__ int s_kend[kThreads / kWave];
  float4* stash4 = stash_all + threadIdx.x;
  const float* stash = reinterpret_cast<const float*>(stash4);
  const int h = blockIdx.y;
  const int w = threadIdx.x >> 6;
  const int l = lane_id();
  const int half = l >> 5;
  const size_t hq = static_cast<size_t>(h) * Npad;
  // Queries of this lane (blocks 0 and 1).  Normally 256 consecutive rows per
  // workgroup (causal: the longest rows first); in list mode (a retry with a
  // new threshold) rows listed in qlist for this head.
  int qq[2];
  bool live[2];
  if (qlist == nullptr) {
    const int nqb = Npad / kQueriesPerBlock;
    const int qblk = causal ? (nqb - 1 - static_cast<int>(blockIdx.x)) : static_cast<int>(blockIdx.x);
    const int qw = qblk * kQueriesPerBlock + w * kWaveQueries;
    qq[0] = qw + (l & 31);
    qq[1] = qw + 32 + (l & 31);
    live[0] = qq[0] < N;
    live[1] = qq[1] < N;
  } else {
    const int count = qlist_count[h];
    const int slot0 = static_cast<int>(blockIdx.x) * kQueriesPerBlock;
    if (slot0 >= count) return;                 // whole workgroup: nothing listed here
    const int sa = slot0 + w * kWaveQueries + (l & 31);
    live[0] = sa < count;
    live[1] = sa + 32 < count;
    qq[0] = live[0] ? qlist[hq + sa] : 0;
    qq[1] = live[1] ? qlist[hq + sa + 32] : 0;
  }
  // first live query of the wave (causal diagonal test) and the keys the
  // workgroup must stream
  int qmin = min(live[0] ? qq[0] : 0x7FFFFFFF, live[1] ? qq[1] : 0x7FFFFFFF);
  int qmax = max(live[0] ? qq[0] : -1, live[1] ? qq[1] : -1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    qmin = min(qmin, __shfl_xor(qmin, o, kWave));
    qmax = max(qmax, __shfl_xor(qmax, o, kWave));
  }
  if (l == 0) s_kend[w] = qmax;
  __syncthreads();
  int kend = N;
  if (causal) {
    int m = -1;
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) m = max(m, s_kend[i]);
    kend = min(N, m + 1);
  }
  const int qw = qmin;
  const bf16_t* qh = q16 + hq * DP;
  const bf16_t* kh = k16 + hq * DP;
  const float kn = __uint_as_float(kstat[kKeyStatWords * h]);
  const float kr = __uint_as_float(kstat[kKeyStatWords * h + 1]);
  const float kinv =
      __builtin_ldexpf(1.0f, -scale_exponent(__uint_as_float(kstat[kKeyStatWords * h + 2])));

  const int qa = qq[0], qb = qq[1];
  uint4 b0[Tile<DP>::kKSteps], b1[Tile<DP>::kKSteps];
  load_query_frags<DP>(b0, qh, qa);
  load_query_frags<DP>(b1, qh, qb);

  // Per-lane threshold on the raw MFMA sum: pairs with s~ >= tau - m pass,
  // where s~ = sum * f and f = score_factor(...) is a power-of-two multiple of
  // the score scale.  The bound is moved down by a few ulps so that rounding
  // of the scaled score can never drop such a pair.
  float thr[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int q = qq[bb];
    float t = INFINITY;
    if (live[bb]) {
      const float tq = tau[hq + q];
      if (tq == -INFINITY) {
        t = -FLT_MAX;
      } else {
        const float4 st = qstat[hq + q];
        const float m = score_margin(st.x, st.y, kn, kr, scale, DP);
        float lim = tq - m;
        lim -= fabsf(lim) * (1.0f / 1048576.0f) + 1e-30f;
        t = lim / score_factor(st.z, kinv, scale);
        t -= fabsf(t) * (1.0f / 1048576.0f) + 1e-30f;
      }
    }
    thr[bb] = t;
  }
  uint2* list[2];
  list[0] = cand + ((hq + qa) * 2 + half) * static_cast<size_t>(capH);
  list[1] = cand + ((hq + qb) * 2 + half) * static_cast<size_t>(capH);
  unsigned count[2] = {0u, 0u};
  const unsigned last = static_cast<unsigned>(capH - 1);

  const int nchunks = (kend + kKeysPerChunk - 1) / kKeysPerChunk;
  u32x4 regs[Stage<DP>::kPerThread];
  chunk_load<DP>(regs, kh, 0);
  chunk_store<DP>(regs, lds);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const bool more = ch + 1 < nchunks;
    if (more) chunk_load<DP>(regs, kh, (ch + 1) * kKeysPerChunk);   // in flight during this chunk
    const uint4* buf = lds + (ch & 1) * Tile<DP>::kChunkUnits;
    const int ntiles = min(kKeysPerChunk / 32, (kend - ch * kKeysPerChunk + 31) / 32);
    // accumulators of two tiles: the next tile's MFMAs run while this tile's
    // scores are filtered (past the last tile they read stale LDS, unused)
    f32x16 acc[2][2];
    acc[0][0] = tile_scores<DP, F>(buf, 0, b0);
    acc[0][1] = tile_scores<DP, F>(buf, 0, b1);
#pragma unroll
    for (int tt = 0; tt < kKeysPerChunk / 32; ++tt) {
      if (tt >= ntiles) break;
      if (tt + 1 < kKeysPerChunk / 32) {
        acc[(tt + 1) & 1][0] = tile_scores<DP, F>(buf, tt + 1, b0);
        acc[(tt + 1) & 1][1] = tile_scores<DP, F>(buf, tt + 1, b1);
      }
      const int tbase = ch * kKeysPerChunk + tt * 32;
      const unsigned jbase = static_cast<unsigned>(tbase + 4 * half);
      const bool edge = (tbase + 32 > N) || (causal && tbase + 31 > qw);
      // bits 0-15: hits of query block 0, bits 16-31: query block 1
      unsigned bits = (~miss_bits(acc[tt & 1][0], thr[0]) & 0xFFFFu) |
                      (~miss_bits(acc[tt & 1][1], thr[1]) << 16);
      if (edge) {
        const int lim0 = (causal ? min(N - 1, qq[0]) : N - 1) - static_cast<int>(jbase);
        const int lim1 = (causal ? min(N - 1, qq[1]) : N - 1) - static_cast<int>(jbase);
        bits &= valid_rows(lim0) | (valid_rows(lim1) << 16);
      }
      if (bits) {
        // park this lane's 32 tile scores (lane-interleaved: conflict-free)
        // so that its hits can be read by index
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          const f32x16& a = acc[tt & 1][bb];
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4)
            stash4[(4 * bb + v4) * kThreads] =
                make_float4(a[4 * v4], a[4 * v4 + 1], a[4 * v4 + 2], a[4 * v4 + 3]);
        }
        do {
          const unsigned b = static_cast<unsigned>(__builtin_ctz(bits));
          bits &= bits - 1;
          const unsigned r = b & 15u;
          const float v = stash[(b >> 2) * (4 * kThreads) + (b & 3u)];
          // accumulator r holds key row r + (r & 12) + 4*half of the tile
          const uint2 e = make_uint2(jbase + r + (r & 12u), __float_as_uint(v));
          if (b < 16) {
            list[0][min(count[0], last)] = e;
            ++count[0];
          } else {
            list[1][min(count[1], last)] = e;
            ++count[1];
          }
        } while (bits);
      }
    }
    if (more) chunk_store<DP>(regs, lds + ((ch + 1) & 1) * Tile<DP>::kChunkUnits);
    __syncthreads();
  }
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    if (live[bb]) cnt[(hq + qq[bb]) * 2 + half] = static_cast<int>(count[bb]);
  }
  int mine = 0;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) mine += live[bb] ? static_cast<int>(min(count[bb], last + 1)) : 0;
  const int tot = wave_sum_i(mine);
  if (l == 0 && tot) atomicAdd(&hdr->candidates, static_cast<unsigned long long>(tot));
}

template <int DP, typename F>
hipError_t sample_t(const Plan& p, const Bufs& b, int nh, float scale, hipStream_t s) {
  const dim3 grid(p.Npad / kQueriesPerBlock, nh);
  hipLaunchKernelGGL((sample_maxima_kernel<DP, F>), grid, dim3(kThreads), 0, s, b.qlo16, b.ksamp,
                     b.qstat, b.kstat, scale, p.N, p.Npad, p.Ns, p.NB, p.causal, b.bm);
  return hipGetLastError();
}

template <int DP, typename F>
hipError_t filter_t(const Plan& p, const Bufs& b, int nh, float scale, bool retry,
                    hipStream_t s) {
  const dim3 grid(p.Npad / kQueriesPerBlock, nh);
  hipLaunchKernelGGL((filter_kernel<DP, F>), grid, dim3(kThreads), 0, s, b.qlo16, b.klo16,
                     b.qstat, b.kstat, b.tau, p.N, p.Npad, p.causal, p.capH, scale,
                     retry ? b.rlist : static_cast<int*>(nullptr),
                     retry ? b.rcount : static_cast<int*>(nullptr), b.cand, b.cnt, b.hdr);
  return hipGetLastError();
}

template <typename F>
hipError_t sample_f(const Plan& p, const Bufs& b, int nh, float scale, hipStream_t s) {
  switch (p.dp) {
    case 16: return sample_t<16, F>(p, b, nh, scale, s);
    case 32: return sample_t<32, F>(p, b, nh, scale, s);
    case 64: return sample_t<64, F>(p, b, nh, scale, s);
    case 128: return sample_t<128, F>(p, b, nh, scale, s);
  }
  return hipErrorInvalidValue;
}

template <typename F>
hipError_t filter_f(const Plan& p, const Bufs& b, int nh, float scale, bool retry,
                    hipStream_t s) {
  switch (p.dp) {
    case 16: return filter_t<16, F>(p, b, nh, scale, retry, s);
    case 32: return filter_t<32, F>(p, b, nh, scale, retry, s);
    case 64: return filter_t<64, F>(p, b, nh, scale, retry, s);
    case 128: return filter_t<128, F>(p, b, nh, scale, retry, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_sample_maxima(const Plan& p, const Bufs& b, int nh, float score_scale,
                                hipStream_t s) {
  return p.filt ? sample_f<FiltBf16>(p, b, nh, score_scale, s)
                : sample_f<FiltF16>(p, b, nh, score_scale, s);
}

hipError_t launch_threshold(const Plan& p, const Bufs& b, int nh, float score_scale,
                            hipStream_t s) {
  const dim3 grid(p.Npad / kThreads, nh);
  (void)score_scale;
  hipLaunchKernelGGL(threshold_kernel, grid, dim3(kThreads), 0, s, b.bm, p.N, p.Npad, p.Ns,
                     p.NB, p.k, p.causal, p.capH, kTauBeta, b.tau);
  return hipGetLastError();
}

hipError_t launch_filter(const Plan& p, const Bufs& b, int nh, float score_scale, bool retry,
                         hipStream_t s) {
  return p.filt ? filter_f<FiltBf16>(p, b, nh, score_scale, retry, s)
                : filter_f<FiltF16>(p, b, nh, score_scale, retry, s);
}

}  // namespace sa
