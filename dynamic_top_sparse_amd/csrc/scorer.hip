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
// staged chunk.  gfx950's LDS serves a 128-bit read 16 lanes at a time over
// 64 banks (256 bytes), i.e. 16 keys at one unit: XOR-ing the unit with bits
// 1..3 of the key puts those 16 rows of 128 bytes on 16 distinct bank groups
// (the bank-conflict counter reads 0).
template <int DP>
__device__ __forceinline__ int lds_unit(int key, int u) {
  constexpr int U = Tile<DP>::kUnits;
  return key * U + (u ^ ((key >> 1) & (U - 1)));
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

// ------------------------------------------------------------ sample pass ---
// Block maxima of one lane's 16 accumulators (keys 8*(r/4) + r%4 + 4*half of
// the tile, in r order) for blocks of B consecutive accumulators, stored as
// values e0 .. e0 + 16/B - 1 of the query's row of maxima.
// The maxima are scaled by f (> 0) only when stored: rounding a product is
// monotonic in the other factor, so max(x) * f is exactly max(x * f).  Only
// the top 16 bits of each maximum's order key are kept: the threshold is
// selected on those bits alone (rounded down), so the rest would never be
// read.
__device__ __forceinline__ uint16_t max_key16(float v) {
  return static_cast<uint16_t>(order_key(v) >> 16);
}
__device__ __forceinline__ void store_block_maxima(f32x16 v, int B, float f,
                                                   uint16_t* __restrict__ dst, size_t stride) {
#pragma unroll
  for (int lvl = 0; lvl <= 4; ++lvl) {
    const int b = 1 << lvl;
    if (lvl > 0) {
#pragma unroll
      for (int r = 0; r < 16; r += b) v[r] = fmaxf(v[r], v[r + b / 2]);
    }
    if (B == b) {
#pragma unroll
      for (int g = 0; g < 16 / b; ++g) dst[g * stride] = max_key16(v[g * b] * f);
    }
  }
}

template <int DP, typename F>
__global__ __launch_bounds__(kThreads) void sample_maxima_kernel(
    const bf16_t* __restrict__ q16, const bf16_t* __restrict__ samp,
    const float4* __restrict__ qstat, const uint32_t* __restrict__ kstat, float scale, int N,
    int Npad, int Ns, int sstride, int k, int causal, int capH, float beta,
    uint16_t* __restrict__ bm) {
  __shared__ uint4 lds[2 * Tile<DP>::kChunkUnits];
  const int h = blockIdx.y;
  const int q0 = blockIdx.x * kQueriesPerBlock;
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);   // wave-uniform, scalar
  const int l = lane_id();
  const int half = l >> 5;
  const int qw = q0 + w * kWaveQueries;
  const bf16_t* qh = q16 + static_cast<size_t>(h) * Npad * DP;
  const bf16_t* sh = samp + static_cast<size_t>(h) * (Npad / sstride) * DP;
  // value e of query q of head h: bm[e * (heads * Npad) + h * Npad + q]
  uint16_t* bmh = bm + static_cast<size_t>(h) * Npad;
  const size_t stride = static_cast<size_t>(gridDim.y) * Npad;

  uint4 b0[Tile<DP>::kKSteps], b1[Tile<DP>::kKSteps];
  load_query_frags<DP>(b0, qh, qw + (l & 31));
  load_query_frags<DP>(b1, qh, qw + 32 + (l & 31));
  const int qq[2] = {qw + (l & 31), qw + 32 + (l & 31)};
  const float kinv = __builtin_ldexpf(
      1.0f, -scale_exponent(__uint_as_float(kstat[kKeyStatWords * h + 2])));
  const float fa = score_factor(qstat[static_cast<size_t>(h) * Npad + qq[0]].z, kinv, scale);
  const float fb = score_factor(qstat[static_cast<size_t>(h) * Npad + qq[1]].z, kinv, scale);
  // Per query: its block size and its last valid sample tile.  Only rows
  // that use a threshold store maxima, and only for their own valid samples,
  // so a row never exceeds sample_blocks() values.
  int Bq[2], last_tile[2];
  float run[2] = {-INFINITY, -INFINITY};   // running maximum of a block that spans tiles
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int q = qq[bb];
    const int n_valid = causal ? min(q + 1, N) : N;
    const int nsv = causal ? min(Ns, q / sstride + 1) : Ns;
    Bq[bb] = sample_block(nsv, sample_rank(min(k, n_valid), nsv, n_valid, beta));
    last_tile[bb] = q < N && n_valid > 2 * capH - 64 ? (nsv - 1) / 32 : -1;
  }

  const int sshift = __builtin_ctz(static_cast<unsigned>(sstride));
  // sample keys t with s*t <= last query of the block (causal), else all
  int s_end = Ns;
  if (causal) s_end = min(Ns, (min(N, q0 + kQueriesPerBlock) - 1) / sstride + 1);
  const int nchunks = (s_end + kKeysPerChunk - 1) / kKeysPerChunk;
  u32x4 regs[Stage<DP>::kPerThread];
  chunk_load<DP>(regs, sh, 0);
  chunk_store<DP>(regs, lds);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const bool more = ch + 1 < nchunks;
    if (more) chunk_load<DP>(regs, sh, (ch + 1) * kKeysPerChunk);
    const uint4* buf = lds + (ch & 1) * Tile<DP>::kChunkUnits;
#pragma unroll
    for (int tt = 0; tt < kKeysPerChunk / 32; ++tt) {
      const int tbase = ch * kKeysPerChunk + tt * 32;
      if (tbase >= s_end) break;
      f32x16 a[2];
      a[0] = tile_scores<DP, F>(buf, tt, b0);
      a[1] = tile_scores<DP, F>(buf, tt, b1);
      const int tile = tbase / 32;
      // samples past the end or after a query (causal) only occur on edge
      // tiles (a wave-uniform test: qw is the wave's first query)
      const bool edge = tbase + 32 > s_end || (causal && (tbase + 31) * sstride > qw);
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const float fq = bb ? fb : fa;   // > 0: scaling commutes with the maxima
        if (edge) {
          // valid rows: sample t < s_end and, causally, t * sstride <= the
          // query (sstride is a power of two), a prefix of the rows
          int lim = s_end - 1;
          if (causal) lim = min(lim, qq[bb] >> sshift);
          const unsigned vr = valid_rows(lim - (tbase + 4 * half));
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (!((vr >> r) & 1u)) a[bb][r] = -INFINITY;
        }
        if (tile > last_tile[bb]) continue;
        const int B = Bq[bb];
        if (B <= 16) {
          store_block_maxima(a[bb], B, fq, bmh + (2 * tile + half) * (16 / B) * stride + qq[bb],
                             stride);
        } else {
          float m = a[bb][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) m = fmaxf(m, a[bb][r]);
          run[bb] = fmaxf(run[bb], m * fq);
          const int G = B / 16;
          if (tile % G == G - 1 || tile == last_tile[bb]) {
            bmh[(2 * (tile / G) + half) * stride + qq[bb]] = max_key16(run[bb]);
            run[bb] = -INFINITY;
          }
        }
      }
    }
    if (more) chunk_store<DP>(regs, lds + ((ch + 1) & 1) * Tile<DP>::kChunkUnits);
    __syncthreads();
  }
}

// -------------------------------------------------------------- threshold ---
// tau is (a lower rounding of) the r-th largest of a query's block maxima,
// found by a 4-bit-digit radix select over the top 16 bits of their order
// keys, the part the sample pass stores (rounding down only adds
// candidates).  About beta * k keys are expected above it.
// A thread selects for two consecutive queries, whose maxima of one index
// share a 32-bit word, so each pass reads one word per index for both.  Eight
// of those loads are issued before any is counted, and each thread counts
// digits in its own LDS columns with LDS atomic adds (no read-modify-write
// round trip): the kernel is bound by load latency, not by arithmetic.
constexpr int kThrQ = 2;          // queries per thread
constexpr int kThrThreads = 256;  // 512 queries per workgroup
constexpr int kThrUnroll = 8;     // maxima loads in flight per thread

__global__ __launch_bounds__(kThrThreads) void threshold_kernel(
    const uint16_t* __restrict__ bm, int N, int Npad, int Ns, int sstride, int k, int causal,
    int capH, float beta, float* __restrict__ tau) {
  // counts of digit d for query j of thread t: hist[(d * kThrQ + j) * kThrThreads + t]
  __shared__ uint32_t hist[16 * kThrQ * kThrThreads];
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int q0 = (static_cast<int>(blockIdx.x) * kThrThreads + tid) * kThrQ;
  const size_t stride = static_cast<size_t>(gridDim.y) * Npad;   // between a query's maxima
  // maxima e of queries q0 and q0 + 1: the 32-bit word at bmh + e * stride
  const uint16_t* bmh = bm + static_cast<size_t>(h) * Npad + q0;
  int nb[kThrQ], K[kThrQ];
  uint32_t prefix[kThrQ];
  int nbmax = 0;
#pragma unroll
  for (int j = 0; j < kThrQ; ++j) {
    const int q = q0 + j;
    const int n_valid = causal ? q + 1 : N;
    const bool active = q < N && n_valid > 2 * capH - 64;
    const int ns_valid = causal ? min(Ns, q / sstride + 1) : Ns;
    const int k_i = min(k, n_valid);
    const int r0 = sample_rank(k_i, ns_valid, n_valid, beta);
    const int nbj = sample_blocks(ns_valid, sample_block(ns_valid, r0));
    nb[j] = active ? nbj : 0;    // an idle query reads nothing
    K[j] = min(r0, nbj);
    prefix[j] = 0;
    nbmax = max(nbmax, nb[j]);
  }
  uint32_t* col = hist + tid;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 28 - 4 * pass;
    const uint32_t pmask = pass == 0 ? 0u : (0xFFFFFFFFu << (shift + 4));
#pragma unroll
    for (int i = 0; i < 16 * kThrQ; ++i) col[i * kThrThreads] = 0u;
    for (int e0 = 0; e0 < nbmax; e0 += kThrUnroll) {
      uint32_t w[kThrUnroll];
#pragma unroll
      for (int u = 0; u < kThrUnroll; ++u) {
        const int e = min(e0 + u, nbmax - 1);   // past nbmax: a row already read, not counted
        w[u] = *reinterpret_cast<const uint32_t*>(bmh + static_cast<size_t>(e) * stride);
      }
#pragma unroll
      for (int u = 0; u < kThrUnroll; ++u) {
        const int e = e0 + u;
#pragma unroll
        for (int j = 0; j < kThrQ; ++j) {
          const uint32_t key = j ? (w[u] & 0xFFFF0000u) : (w[u] << 16);   // query q0 + j
          if (e < nb[j] && (key & pmask) == prefix[j])
            atomicAdd(&col[(((key >> shift) & 15u) * kThrQ + j) * kThrThreads], 1u);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kThrQ; ++j) {
      if (nb[j] == 0) continue;
      int cum = 0, digit = 0;
      for (int d = 15; d >= 0; --d) {
        const int c = static_cast<int>(col[(d * kThrQ + j) * kThrThreads]);
        if (cum + c >= K[j]) { digit = d; break; }
        cum += c;
      }
      K[j] -= cum;
      prefix[j] |= static_cast<uint32_t>(digit) << shift;
    }
  }
#pragma unroll
  for (int j = 0; j < kThrQ; ++j) {
    // block maxima are stored as filter scores already (score factor applied)
    float result = -INFINITY;
    if (nb[j] > 0 && prefix[j] > order_key(-INFINITY)) result = key_to_float(prefix[j]);
    tau[static_cast<size_t>(h) * Npad + q0 + j] = result;
  }
}

// ------------------------------------------------------------ filter pass ---
// The MFMA accumulates onto C = -thr (thr: the query's threshold on the raw
// sum), so a pair passes exactly when its accumulator's sign bit is clear.
// Bit r of the result is set when accumulator r misses; the sign bits are
// shifted in with one v_alignbit per accumulator.  Masked (-inf) rows miss.
__device__ __forceinline__ unsigned miss_bits(const f32x16& a) {
  unsigned nb = 0;
#pragma unroll
  for (int r = 15; r >= 0; --r) nb = __builtin_amdgcn_alignbit(nb, __float_as_uint(a[r]), 31);
  return nb;
}

template <int DP, typename F>
__device__ __forceinline__ f32x16 tile_scores_c(const uint4* __restrict__ lds, int tile_in_chunk,
                                                const uint4 (&b)[Tile<DP>::kKSteps],
                                                const f32x16& c) {
  const int l = lane_id();
  const int key = tile_in_chunk * 32 + (l & 31);
  f32x16 acc = F::mfma(lds[lds_unit<DP>(key, l >> 5)], b[0], c);
#pragma unroll
  for (int ks = 1; ks < Tile<DP>::kKSteps; ++ks)
    acc = F::mfma(lds[lds_unit<DP>(key, 2 * ks + (l >> 5))], b[ks], acc);
  return acc;
}

__device__ __forceinline__ int imax3(int a, int b, int c) { return max(max(a, b), c); }

// On an edge tile, rows past the end or above the causal diagonal are dropped
// from the hit mask and their accumulators set to the bit pattern 0x80000000,
// the smallest signed integer, so that no integer maximum picks them.
__device__ __forceinline__ unsigned mask_edge_rows(f32x16& a, unsigned bits, unsigned valid) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (!((valid >> r) & 1u)) a[r] = __int_as_float(static_cast<int>(0x80000000u));
  return bits & valid;
}

// Appends the passing accumulators of one 32-query block to the lane's list,
// in key order.  Accumulators start at -thr, so hits are exactly the
// non-negative ones, and as signed integers their bit patterns are the
// largest: a lane with a single hit (the common case) finds its value as the
// integer maximum of its 16 accumulators (eight three-way maxima).  That also
// holds for an all-pass lane (every valid row is listed, whatever its sign)
// with one valid row, because masked rows hold the smallest integer.  A lane
// cannot index its registers by a run-time number, so the rarer lane with
// more hits parks its values in its own LDS column (stash[r][lane]:
// conflict-free) and reads them back.
// The entry goes to byte (loff + 8 * min(count, last)) past `base`; in the
// main pass `base` is the wave's first list (a scalar register) and loff the
// lane's 32-bit list offset, so an append costs one 32-bit address add.
__device__ __forceinline__ void put_entry(uint2* base, unsigned loff, unsigned count,
                                          unsigned last, uint2 e) {
  *reinterpret_cast<uint2*>(reinterpret_cast<char*>(base) + (loff + (min(count, last) << 3))) = e;
}

// The key field of an entry is jenc + r (jenc = tile start + 16 * tile half;
// candidate_key() recovers the key).
__device__ __forceinline__ void drain_hits(const f32x16& a, unsigned bits,
                                           float* stash, unsigned jenc, uint2* lst,
                                           unsigned loff, unsigned& count, unsigned last) {
  const unsigned nb = static_cast<unsigned>(__builtin_popcount(bits));
  if (nb == 1u) {
    int x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = __float_as_int(a[r]);
    const int m = imax3(imax3(imax3(x[0], x[1], x[2]), imax3(x[3], x[4], x[5]),
                              imax3(x[6], x[7], x[8])),
                        imax3(x[9], x[10], x[11]), imax3(x[12], x[13], imax3(x[14], x[15], x[15])));
    const unsigned b = static_cast<unsigned>(__builtin_ctz(bits));
    // accumulator r holds key row r + (r & 12) (+4 in the upper half-wave)
    put_entry(lst, loff, count, last, make_uint2(jenc + b, static_cast<unsigned>(m)));
    ++count;
  }
  if (nb > 1u) {
#pragma unroll
    for (int r = 0; r < 16; ++r) stash[r * kThreads] = a[r];
    do {
      const unsigned b = static_cast<unsigned>(__builtin_ctz(bits));
      bits &= bits - 1u;
      const float v = stash[b * kThreads];
      put_entry(lst, loff, count, last, make_uint2(jenc + b, __float_as_uint(v)));
      ++count;
    } while (bits);
  }
}

template <int DP, typename F, int mode>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void filter_kernel(
    const bf16_t* __restrict__ q16, const bf16_t* __restrict__ k16,
    const float4* __restrict__ qstat, const uint32_t* __restrict__ kstat,
    const float* __restrict__ tau, float* __restrict__ thr_out, int N, int Npad, int causal,
    int capH, float scale, const int* __restrict__ qlist, const int* __restrict__ qlist_count,
    uint2* __restrict__ cand, int* __restrict__ cnt, int* __restrict__ rcnt,
    WsHeader* __restrict__ hdr) {
  __shared__ uint4 lds[2 * Tile<DP>::kChunkUnits];
  __shared__ float stash_all[16 * kThreads];   // 16 scores per lane, [16][threads]
  // per-wave last query, read before the first chunk barrier, so it can share
  // the stash's space
  int* s_kend = reinterpret_cast<int*>(stash_all);
  float* stash = stash_all + threadIdx.x;
  const int h = blockIdx.y;
  const int w = threadIdx.x >> 6;
  const int l = lane_id();
  const int half = l >> 5;
  const size_t hq = static_cast<size_t>(h) * Npad;
  // Queries of this lane (blocks 0 and 1).  Normally 256 consecutive rows per
  // workgroup (causal: the longest rows first); in list mode (a retry with a
  // new threshold) rows listed in qlist for this head.  Those are few, so
  // kRetrySplit workgroups share each 256 of them, one key segment each, in
  // two launches: mode 1 counts each segment's hits, mode 2 writes them at
  // the segment's offset in the query's list, which so stays in key order.
  const int nseg = qlist == nullptr ? 1 : kRetrySplit;
  const int seg = qlist == nullptr ? 0 : static_cast<int>(blockIdx.x) % kRetrySplit;
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
    const int slot0 = static_cast<int>(blockIdx.x) / kRetrySplit * kQueriesPerBlock;
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

  // Threshold on the raw MFMA sum: pairs with s~ >= tau - m pass, where
  // s~ = sum * f and f = score_factor(...) is a power-of-two multiple of the
  // score scale.  The bound is moved down by a few ulps so that rounding of
  // the scaled score can never drop such a pair.  tau = -inf keeps every
  // valid key (C = 0, all bits set).  The value used is stored for the
  // re-rank, which adds it back to the parked accumulators.
  f32x16 cinit[2];
  bool all_pass[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int q = qq[bb];
    float c = -INFINITY;     // idle lanes: every pair misses
    all_pass[bb] = false;
    if (live[bb]) {
      const float tq = tau[hq + q];
      float t = 0.0f;
      if (tq == -INFINITY) {
        all_pass[bb] = true;
      } else {
        const float4 st = qstat[hq + q];
        const float m = score_margin(st.x, st.y, kn, kr, scale, DP);
        float lim = tq - m;
        lim -= fabsf(lim) * (1.0f / 1048576.0f) + 1e-30f;
        t = lim / score_factor(st.z, kinv, scale);
        t -= fabsf(t) * (1.0f / 1048576.0f) + 1e-30f;
      }
      c = -t;
      if (half == 0) thr_out[hq + q] = t;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) cinit[bb][r] = c;
  }
  // list position of this workgroup's first entry (the hits of the earlier
  // segments come first); entries past the capacity land on the last slot,
  // and the re-rank sees the overflow from the counts
  uint2* list[2];
  unsigned last[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    int off = 0;
    if (mode == 2) {
      const int* rc = rcnt + ((hq + qq[bb]) * 2 + half) * kRetrySplit;
      for (int s2 = 0; s2 < seg; ++s2) off += rc[s2];
    }
    off = min(off, capH - 1);
    list[bb] = cand + ((hq + qq[bb]) * 2 + half) * static_cast<size_t>(capH) + off;
    last[bb] = static_cast<unsigned>(capH - 1 - off);
  }
  // Main pass: the wave's 128 lists are consecutive, so every append
  // addresses them from the first one (wave-uniform) plus a 32-bit lane
  // offset (at most 128 lists of capH <= 2048 entries: under 2 MB).  Retry
  // passes address each lane's own list.
  uint2* lbase[2] = {list[0], list[1]};
  unsigned loff[2] = {0u, 0u};
  if constexpr (mode == 0) {
    const int qfirst = __builtin_amdgcn_readfirstlane(qq[0] - (l & 31));
    uint2* wbase = cand + (hq + qfirst) * 2 * static_cast<size_t>(capH);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      lbase[bb] = wbase;
      loff[bb] = static_cast<unsigned>((((l & 31) + 32 * bb) * 2 + half) * capH) * 8u;
    }
  }
  unsigned count[2] = {0u, 0u};
  // all-pass lists take every valid key: their hit mask is all ones
  const unsigned apm[2] = {all_pass[0] ? 0xFFFFu : 0u, all_pass[1] ? 0xFFFFu : 0u};

  // this workgroup's chunks: all of [0, kend), or its segment of them
  const int nch_all = (kend + kKeysPerChunk - 1) / kKeysPerChunk;
  const int per_seg = (nch_all + nseg - 1) / nseg;
  const int ch0 = min(nch_all, seg * per_seg);
  const int nchunks = min(nch_all, ch0 + per_seg);
  u32x4 regs[Stage<DP>::kPerThread];
  if (ch0 < nchunks) {
    chunk_load<DP>(regs, kh, ch0 * kKeysPerChunk);
    chunk_store<DP>(regs, lds + (ch0 & 1) * Tile<DP>::kChunkUnits);
  }
  // Retire every load made so far (query fragments, thresholds): otherwise
  // the loop keeps waits for them on the memory counter, which stores and
  // the chunk prefetch share, and the MFMAs stall on those instead.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int ch = ch0; ch < nchunks; ++ch) {
    const bool more = ch + 1 < nchunks;
    if (more) chunk_load<DP>(regs, kh, (ch + 1) * kKeysPerChunk);   // in flight during this chunk
    const uint4* buf = lds + (ch & 1) * Tile<DP>::kChunkUnits;
    const int ntiles = min(kKeysPerChunk / 32, (kend - ch * kKeysPerChunk + 31) / 32);
    // The two query blocks' MFMA chains alternate with the other block's hit
    // handling, so a wave keeps the matrix core busy while its VALU work runs
    // (one set of accumulators per block: three waves per SIMD still fit).
    f32x16 a0 = tile_scores_c<DP, F>(buf, 0, b0, cinit[0]);
#pragma unroll
    for (int tt = 0; tt < kKeysPerChunk / 32; ++tt) {
      if (tt >= ntiles) break;
      f32x16 a1 = tile_scores_c<DP, F>(buf, tt, b1, cinit[1]);
      const int tbase = ch * kKeysPerChunk + tt * 32;
      const unsigned jbase = static_cast<unsigned>(tbase + 4 * half);   // key of accumulator 0
      const unsigned jenc = static_cast<unsigned>(tbase + 16 * half);   // entry encoding base
      const bool edge = (tbase + 32 > N) || (causal && tbase + 31 > qw);
      unsigned bits0 = (~miss_bits(a0) & 0xFFFFu) | apm[0];
      if (edge)
        bits0 = mask_edge_rows(a0, bits0, valid_rows((causal ? min(N - 1, qq[0]) : N - 1) -
                                                     static_cast<int>(jbase)));
      if (mode == 1)
        count[0] += __builtin_popcount(bits0);
      else
        drain_hits(a0, bits0, stash, jenc, lbase[0], loff[0], count[0], last[0]);
      if (tt + 1 < ntiles) {
        a0 = tile_scores_c<DP, F>(buf, tt + 1, b0, cinit[0]);
      } else if constexpr (mode == 1) {
        // The hardware does not hold back a VALU read of VGPRs an MFMA is
        // still writing.  On a chunk's last tile no chain runs here, and in
        // the counting pass block 0's handling is a popcount, so little
        // would separate a1's last MFMA from its first read below: pad 16
        // wait states (12 are needed after a 32x32x16 MFMA on gfx950).
        // tests/test_mfma_hazards.py checks every path of the built code.
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
      }
      unsigned bits1 = (~miss_bits(a1) & 0xFFFFu) | apm[1];
      if (edge)
        bits1 = mask_edge_rows(a1, bits1, valid_rows((causal ? min(N - 1, qq[1]) : N - 1) -
                                                     static_cast<int>(jbase)));
      if (mode == 1)
        count[1] += __builtin_popcount(bits1);
      else
        drain_hits(a1, bits1, stash, jenc, lbase[1], loff[1], count[1], last[1]);
    }
    if (more) chunk_store<DP>(regs, lds + ((ch + 1) & 1) * Tile<DP>::kChunkUnits);
    __syncthreads();
  }
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    if (live[bb]) {
      if (mode == 0)
        cnt[(hq + qq[bb]) * 2 + half] = static_cast<int>(count[bb]);
      else if (mode == 1)
        rcnt[((hq + qq[bb]) * 2 + half) * kRetrySplit + seg] = static_cast<int>(count[bb]);
    }
  }
  int mine = 0;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb)
    mine += live[bb] && mode != 1 ? static_cast<int>(min(count[bb], last[bb] + 1)) : 0;
  const int tot = wave_sum_i(mine);
  if (l == 0 && tot) atomicAdd(&hdr->candidates, static_cast<unsigned long long>(tot));
}

template <int DP, typename F>
hipError_t sample_t(const Plan& p, const Bufs& b, int nh, float scale, hipStream_t s) {
  const dim3 grid(p.Npad / kQueriesPerBlock, nh);
  hipLaunchKernelGGL((sample_maxima_kernel<DP, F>), grid, dim3(kThreads), 0, s, b.qlo16, b.ksamp,
                     b.qstat, b.kstat, scale, p.N, p.Npad, p.Ns, p.sstride, p.k, p.causal,
                     p.capH, kTauBeta, b.bm);
  return hipGetLastError();
}

template <int DP, typename F>
hipError_t filter_t(const Plan& p, const Bufs& b, int nh, float scale, bool retry,
                    hipStream_t s) {
  const dim3 grid(p.Npad / kQueriesPerBlock * (retry ? kRetrySplit : 1), nh);
  if (!retry) {
    hipLaunchKernelGGL((filter_kernel<DP, F, 0>), grid, dim3(kThreads), 0, s, b.qlo16, b.klo16,
                       b.qstat, b.kstat, b.tau, b.thr, p.N, p.Npad, p.causal, p.capH, scale,
                       static_cast<int*>(nullptr), static_cast<int*>(nullptr), b.cand, b.cnt,
                       b.rcnt, b.hdr);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((filter_kernel<DP, F, 1>), grid, dim3(kThreads), 0, s, b.qlo16, b.klo16,
                     b.qstat, b.kstat, b.tau, b.thr, p.N, p.Npad, p.causal, p.capH, scale, b.rlist,
                     b.rcount, b.cand, b.cnt, b.rcnt, b.hdr);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((filter_kernel<DP, F, 2>), grid, dim3(kThreads), 0, s, b.qlo16, b.klo16,
                     b.qstat, b.kstat, b.tau, b.thr, p.N, p.Npad, p.causal, p.capH, scale, b.rlist,
                     b.rcount, b.cand, b.cnt, b.rcnt, b.hdr);
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
  const dim3 grid(p.Npad / (kThrThreads * kThrQ), nh);   // Npad is a multiple of 512
  (void)score_scale;
  hipLaunchKernelGGL(threshold_kernel, grid, dim3(kThrThreads), 0, s, b.bm, p.N, p.Npad, p.Ns,
                     p.sstride, p.k, p.causal, p.capH, kTauBeta, b.tau);
  return hipGetLastError();
}

hipError_t launch_filter(const Plan& p, const Bufs& b, int nh, float score_scale, bool retry,
                         hipStream_t s) {
  return p.filt ? filter_f<FiltBf16>(p, b, nh, score_scale, retry, s)
                : filter_f<FiltF16>(p, b, nh, score_scale, retry, s);
}

}  // namespace sa
