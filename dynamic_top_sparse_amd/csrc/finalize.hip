// Exact re-rank of the filter's candidates, and the exact fallback.
//
// The selection rule (page "mhpq.cn/news/1098205", §3.2: torch.topk over the
// scores, masked keys excluded first, all keys kept when fewer than k are
// valid) is applied to the exact fp32 score s of exact_score().  Ties go to
// the lower key index; rows are written in ascending key order, then -1.
//
// Re-rank, one wavefront per query.  Each candidate carries its 16-bit MFMA
// score s~; with the per-query margin m every exact score lies in
// [l, u] = [s~ - m, s~ + m] (rounded outwards).  Let lo be the k-th largest l
// and hi the (k+1)-th largest u (or tau if larger).  Then
//   u < lo   -> the key is certainly out (its exact score is below the k-th),
//   l > hi   -> certainly in (at most k-1 other keys can reach its score),
// and only the remaining "uncertain" keys are re-scored exactly, in fp32,
// and ranked by (s descending, key ascending) to fill the rest of the row.
// The candidate list of each query half is already in ascending key order
// (the filter streams keys in order), so the output row is a merge.
//
// A query whose list overflowed, or whose threshold turned out too high, is
// not lost: the k-th best lower bound among the candidates it does hold is a
// proven threshold (k keys reach it), so the query is queued to be filtered
// again with it.  Only what remains unresolved after that second round goes
// to the exact fallback.
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;   // fallback workgroup
constexpr int kPrefetch = 12;                      // candidate entries per lane loaded a query ahead

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}


// Wave-wide min / max of 32- and 64-bit keys: permlane swaps across rows,
// then DPP partners inside each row (VALU only; see sa_common.h).
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce_key(T v, Op op) {
  auto both = [&](auto swap) {
    if constexpr (sizeof(T) == 8) {
      const auto lo = swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
      const auto hi = swap(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(v >> 32), false, false);
      const T a = (static_cast<T>(hi[0]) << 32) | lo[0];
      const T b = (static_cast<T>(hi[1]) << 32) | lo[1];
      v = op(a, b);
    } else {
      const auto r = swap(v, v, false, false);
      v = op(static_cast<T>(r[0]), static_cast<T>(r[1]));
    }
  };
  both([](uint32_t x, uint32_t y, bool, bool) { return __builtin_amdgcn_permlane32_swap(x, y, false, false); });
  both([](uint32_t x, uint32_t y, bool, bool) { return __builtin_amdgcn_permlane16_swap(x, y, false, false); });
  auto step = [&](auto ctrl) {
    constexpr int C = decltype(ctrl)::value;
    if constexpr (sizeof(T) == 8) {
      const uint32_t lo = static_cast<uint32_t>(dpp_i<C>(static_cast<int>(static_cast<uint32_t>(v))));
      const uint32_t hi = static_cast<uint32_t>(dpp_i<C>(static_cast<int>(static_cast<uint32_t>(v >> 32))));
      v = op(v, (static_cast<T>(hi) << 32) | lo);
    } else {
      v = op(v, static_cast<T>(dpp_i<C>(static_cast<int>(v))));
    }
  };
  step(std::integral_constant<int, kDppQuadXor1>{});
  step(std::integral_constant<int, kDppQuadXor2>{});
  step(std::integral_constant<int, kDppHalfMirror>{});
  step(std::integral_constant<int, kDppMirror>{});
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_key(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_key(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
  return wave_reduce_key(v, [](unsigned long long a, unsigned long long b) { return a < b ? a : b; });
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  return wave_reduce_key(v, [](unsigned long long a, unsigned long long b) { return a > b ? a : b; });
}

// Value of a key held by lane `src` (wave-uniform), read with v_readlane.
template <typename KeyT>
__device__ __forceinline__ KeyT lane_key(KeyT v, int src) {
  if constexpr (sizeof(KeyT) == 8) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(v), src);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(v >> 32), src);
    return (static_cast<KeyT>(hi) << 32) | lo;
  } else {
    return static_cast<KeyT>(__builtin_amdgcn_readlane(static_cast<uint32_t>(v), src));
  }
}
template <typename KeyT>
__device__ __forceinline__ KeyT wave_min_k(KeyT v);
template <> __device__ __forceinline__ uint32_t wave_min_k(uint32_t v) { return wave_min_u32(v); }
template <> __device__ __forceinline__ unsigned long long wave_min_k(unsigned long long v) { return wave_min_u64(v); }
template <typename KeyT>
__device__ __forceinline__ KeyT wave_max_k(KeyT v);
template <> __device__ __forceinline__ uint32_t wave_max_k(uint32_t v) { return wave_max_u32(v); }
template <> __device__ __forceinline__ unsigned long long wave_max_k(unsigned long long v) { return wave_max_u64(v); }

template <typename KeyT>
__device__ __forceinline__ int key_bits(KeyT span) {
  return sizeof(KeyT) == 8 ? 64 - __builtin_clzll(static_cast<unsigned long long>(span))
                           : 32 - __builtin_clz(static_cast<uint32_t>(span));
}

// K-th largest (1-based) key among the elements a wavefront owns, exactly.
// `each(fn)` calls fn(key, valid) once per element slot with a uniform trip
// count.  The key range is cut into 256 buckets, the bucket holding the K-th
// key is kept, and this repeats until at most 64 keys are left; those are
// ranked directly.  Buckets spread keys that share their leading bits, so the
// LDS histogram sees few colliding atomics.  The histogram holds 16-bit
// counts, two buckets per word (512 B): callers pass fewer than 65536 keys.
// Requires 1 <= K <= #valid keys.
template <typename KeyT, typename Each>
__device__ KeyT wave_select_in(int K, int* hist, KeyT* cbuf, Each each, KeyT lo, KeyT hi) {
  const int l = lane_id();
  int in_range = 65;
  while (lo != hi) {
    const KeyT span = hi - lo;
    const int nb = key_bits<KeyT>(span);
    const int shift = nb > 8 ? nb - 8 : 0;          // (span >> shift) < 256
    reinterpret_cast<int2*>(hist)[l] = make_int2(0, 0);   // 256 bins, 4 per lane
    wave_sync();
    each([&](KeyT key, bool ok) {
      if (ok && key >= lo && key <= hi) {
        const int b = static_cast<int>((key - lo) >> shift);
        atomicAdd(&hist[b >> 1], 1 << ((b & 1) << 4));
      }
    });
    wave_sync();
    const int2 h2 = reinterpret_cast<const int2*>(hist)[63 - l];   // lane L: bins 255-4L ..
    const int c[4] = {static_cast<int>(static_cast<uint32_t>(h2.y) >> 16), h2.y & 0xFFFF,
                      static_cast<int>(static_cast<uint32_t>(h2.x) >> 16), h2.x & 0xFFFF};
    const int sum = c[0] + c[1] + c[2] + c[3];
    const int incl = wave_incl_scan(sum);
    const unsigned long long crossing = __ballot(incl >= K);
    const int F = crossing ? __builtin_ctzll(crossing) : 0;
    int digit = 0, above = 0, cnt = 0;
    if (l == F) {
      int cum = incl - sum;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (cum + c[t] >= K) { digit = 255 - 4 * l - t; cnt = c[t]; break; }
        cum += c[t];
      }
      above = cum;
    }
    digit = __builtin_amdgcn_readlane(digit, F);
    above = __builtin_amdgcn_readlane(above, F);
    cnt = __builtin_amdgcn_readlane(cnt, F);
    K -= above;
    const KeyT nlo = lo + (static_cast<KeyT>(digit) << shift);
    const KeyT width = (static_cast<KeyT>(1) << shift) - 1;
    hi = (hi - nlo) < width ? hi : nlo + width;
    lo = nlo;
    in_range = cnt;
    wave_sync();
    if (cnt <= 64) break;
  }
  if (lo == hi) return lo;          // every remaining key is equal
  // gather the <= 64 keys of [lo, hi] and rank them
  int base = 0;
  each([&](KeyT key, bool ok) {
    const bool in = ok && key >= lo && key <= hi;
    const unsigned long long m = __ballot(in);
    if (in) cbuf[base + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0))] = key;
    base += __builtin_popcountll(m);
  });
  wave_sync();
  const int m = base;
  (void)in_range;
  const KeyT mine = l < m ? cbuf[l] : static_cast<KeyT>(0);
  int greater = 0, equal = 0;
  for (int u = 0; u < m; ++u) {
    const KeyT o = lane_key(mine, u);
    greater += o > mine ? 1 : 0;
    equal += o == mine ? 1 : 0;
  }
  const unsigned long long hit = __ballot(l < m && greater < K && greater + equal >= K);
  const int src = hit ? __builtin_ctzll(hit) : 0;
  const KeyT result = lane_key(mine, src);
  wave_sync();
  return result;
}

// As wave_select_in, with the key range found first.
template <typename KeyT, typename Each>
__device__ KeyT wave_select(int K, int* hist, KeyT* cbuf, Each each) {
  KeyT lo = ~static_cast<KeyT>(0), hi = 0;
  each([&](KeyT key, bool ok) {
    if (ok) {
      lo = key < lo ? key : lo;
      hi = key > hi ? key : hi;
    }
  });
  return wave_select_in<KeyT>(K, hist, cbuf, each, wave_min_k(lo), wave_max_k(hi));
}

__device__ __forceinline__ int lane_rank(unsigned long long mask) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
      static_cast<uint32_t>(mask >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0)));
}

// Writes the merge of the ascending, disjoint lists a[0..na) and b[0..nb) to
// out[0..na+nb): each lane finds where its run of 8 outputs starts with a
// binary search along the cross diagonal, then merges its run sequentially.
__device__ __forceinline__ void merge_rows(const int* a, int na, const int* b, int nb,
                                           int32_t* __restrict__ out) {
  constexpr int T = 8;
  const int total = na + nb;
  for (int start = lane_id() * T; start < total; start += kWave * T) {
    int lo = max(0, start - nb), hi = min(start, na);
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a[mid] < b[start - mid - 1]) lo = mid + 1; else hi = mid;
    }
    int ia = lo, ib = start - lo;
    int va = ia < na ? a[ia] : INT_MAX, vb = ib < nb ? b[ib] : INT_MAX;
    const int n = min(T, total - start);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (t < n) {
        const bool from_a = va < vb;
        out[start + t] = from_a ? va : vb;
        if (from_a) {
          ++ia;
          va = ia < na ? a[ia] : INT_MAX;
        } else {
          ++ib;
          vb = ib < nb ? b[ib] : INT_MAX;
        }
      }
    }
  }
}

// Entries of the ascending list a[0..n) that are below x.
__device__ __forceinline__ int count_below(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ unsigned long long rank_key(float s, int j) {
  return (static_cast<unsigned long long>(order_key(s)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - static_cast<uint32_t>(j));
}

// Per-wave LDS of the re-rank: histogram (512 B), the uncertain keys with
// their exact and filter scores (ucap x 12 B; ucap >= 128, so the filter
// scores' 512 B double as the selects' rank buffer, which is never in use
// while they are), and room
// for lcap candidates (8 B each: order key of the filter score, key index),
// whose key array becomes the output row in place.  A query with more than
// lcap candidates is ranked from its lists in global memory instead, and only
// the keys that can still be kept (fewer than k + ucap) reach LDS.
__host__ __device__ constexpr size_t rerank_lds_per_wave(int cap, int ucap) {
  return (512 + static_cast<size_t>(ucap) * 12 + static_cast<size_t>(cap) * 8 + 15) / 16 * 16;
}

// Re-rank waves per SIMD at most: the kernel is built for four
// (amdgpu_waves_per_eu(4): at most 128 VGPRs).
constexpr int kRerankWavesPerSimd = 4;

// Workgroups of the re-rank one CU holds at once: LDS (160 KB per CU) and
// the waves' registers both bound it.
inline int rerank_groups_per_cu(int wpb, size_t per_wave) {
  const int by_lds = static_cast<int>(163840 / (static_cast<size_t>(wpb) * per_wave));
  const int by_regs = 4 * kRerankWavesPerSimd / wpb;
  return max(1, min(by_lds, by_regs));
}

// Waves of the re-rank one CU holds for a per-wave LDS size (workgroups of
// up to four waves within 64 KB).
inline int rerank_waves_per_cu(size_t per_wave) {
  int wpb = static_cast<int>((64 * 1024) / per_wave);
  wpb = wpb < 1 ? 1 : (wpb > 4 ? 4 : wpb);
  return rerank_groups_per_cu(wpb, per_wave) * wpb;
}

// LDS candidate room of a re-rank wave: the whole list capacity (2 capH)
// unless a smaller room, still at least k + ucap, lets more waves share a CU
// (queries with more candidates then take the path over memory).
inline int rerank_lds_cap(int capH, int k, int ucap) {
  const int full = 2 * capH;
  int best = full, best_waves = rerank_waves_per_cu(rerank_lds_per_wave(full, ucap));
  for (int lc = full - 64; lc >= k + ucap && lc > 0; lc -= 64) {
    const int wv = rerank_waves_per_cu(rerank_lds_per_wave(lc, ucap));
    if (wv > best_waves) {
      best = lc;
      best_waves = wv;
    }
  }
  // the largest room that keeps that many waves
  for (int lc = best + 64; lc < full; lc += 64)
    if (rerank_waves_per_cu(rerank_lds_per_wave(lc, ucap)) == best_waves) best = lc;
  return best;
}

template <int DP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kRerankWavesPerSimd))) void finalize_kernel(
    const uint2* __restrict__ cand, const int* __restrict__ cnt, const int* __restrict__ rcnt,
    float* __restrict__ tau,
    const float* __restrict__ thr,
    const float4* __restrict__ qstat, const uint32_t* __restrict__ kstat,
    const float* __restrict__ q32, const float* __restrict__ k32, int N, int Npad, int k,
    int causal, int capH, int lcap, int ucap, float scale, int32_t* __restrict__ idx,
    const int* __restrict__ qlist, const int* __restrict__ qlist_count, int* __restrict__ rlist,
    int* __restrict__ rcount, int* __restrict__ fblist, int* __restrict__ seg, GatherRanges gr,
    WsHeader* __restrict__ hdr) {
  extern __shared__ unsigned char smem[];
  const int wpb = blockDim.x / kWave;
  // the wave index as a scalar: the query slots, and with them every query's
  // metadata loads and list addresses, are then wave-uniform scalar values
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = lane_id();
  unsigned char* base = smem + static_cast<size_t>(w) * rerank_lds_per_wave(lcap, ucap);
  int* hist = reinterpret_cast<int*>(base);
  int* uj = reinterpret_cast<int*>(base + 512);
  float* us = reinterpret_cast<float*>(base + 512 + ucap * 4);
  float* ut = reinterpret_cast<float*>(base + 512 + ucap * 8);
  // rank buffer of the selects (64 keys of 8 B): the filter scores' area,
  // read only between the classification and the exact re-score
  unsigned long long* cbuf = reinterpret_cast<unsigned long long*>(ut);
  uint32_t* ck = reinterpret_cast<uint32_t*>(base + 512 + ucap * 12);
  int* cj = reinterpret_cast<int*>(base + 512 + ucap * 12 + lcap * 4);

  const int h = blockIdx.y;
  const size_t hq = static_cast<size_t>(h) * Npad;
  // Statistics are kept per wave and added to the header once at the end:
  // one device-scope atomic per query on a shared word would serialise.
  // (32-bit, and each updated by plain arithmetic, so that they stay in
  // registers: a wave takes at most N of one head's queries)
  unsigned st_queries = 0, st_rescored = 0, st_overflow = 0, st_retried = 0;
  unsigned viol = 0;   // per lane: re-scored keys outside their margin interval
  unsigned st_wide = 0;
  // first pass: every query; retry pass: the queries listed for this head
  const int nq = qlist != nullptr ? qlist_count[h] : N;
  // Software pipeline over the wave's queries: while query i is ranked, the
  // candidate lists of query i+1 are loading into registers (the first
  // kPrefetch*64 entries) and the counts and thresholds of query i+2 are
  // loading too, so a query's staging rarely waits for memory.
  struct Meta {
    int q, r0, r1;
    float tq, tv;
    float4 st;
  };
  auto load_meta = [&](int slot) {
    Meta m;
    m.q = qlist != nullptr ? qlist[hq + slot] : slot;
    // One candidate list per query half; the retry pass counted its hits per
    // key segment.  An overflowing list still holds capH genuine candidates.
    m.r0 = 0;
    m.r1 = 0;
    if (qlist == nullptr) {
      m.r0 = cnt[(hq + m.q) * 2];
      m.r1 = cnt[(hq + m.q) * 2 + 1];
    } else {
      for (int s2 = 0; s2 < kRetrySplit; ++s2) {
        m.r0 += rcnt[(hq + m.q) * 2 * kRetrySplit + s2];
        m.r1 += rcnt[((hq + m.q) * 2 + 1) * kRetrySplit + s2];
      }
    }
    m.tq = tau[hq + m.q];
    m.tv = thr[hq + m.q];
    m.st = qstat[hq + m.q];
    return m;
  };
  uint2 pre[kPrefetch];
  // entries l, l+64, ... of the query's candidates (half 0, then half 1);
  // indices past the lists are clamped to a valid entry and never staged
  auto load_cands = [&](const Meta& m) {
    const int c0 = min(m.r0, capH), c = c0 + min(m.r1, capH);
    const uint2* list0 = cand + (hq + m.q) * 2 * static_cast<size_t>(capH);
    // list0 is wave-uniform: each lane adds a 32-bit byte offset to it
    const char* lb = reinterpret_cast<const char*>(list0);
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      const int i = min(l + kWave * j, max(c - 1, 0));
      const unsigned e = static_cast<unsigned>(i < c0 ? i : capH + (i - c0));
      pre[j] = *reinterpret_cast<const uint2*>(lb + e * 8u);
    }
  };
  const int stride = gridDim.x * wpb;
  int slot = blockIdx.x * wpb + w;
  Meta cur{}, nxt{};
  if (slot < nq) {
    cur = load_meta(slot);
    load_cands(cur);
  }
  if (slot + stride < nq) nxt = load_meta(slot + stride);
#pragma unroll 1
  for (; slot < nq; slot += stride) {
    wave_sync();  // the previous query's LDS reads are done
    const bool has_next = slot + stride < nq;
    Meta nn{};
    bool issued = false;
    // starts the loads for the next queries; called once per query, as soon
    // as the registers holding this query's candidates are free
    auto issue_next = [&]() {
      if (has_next) load_cands(nxt);
      if (slot + 2 * stride < nq) nn = load_meta(slot + 2 * stride);
      issued = true;
    };
    do {  // one query; `continue` ends it
    const int q = cur.q;
    int32_t* out = idx + (static_cast<size_t>(h) * N + q) * k;
    const int n_valid = causal ? q + 1 : N;
    const int k_i = min(k, n_valid);
    // Unresolved query: on the first pass, if a proven threshold is known
    // (k keys certainly score at least tau_new), filter it again with that
    // threshold; otherwise resolve it with the exact fallback.
    auto unresolved = [&](float tau_new) {
      const unsigned again = qlist == nullptr && tau_new == tau_new ? 1u : 0u;
      st_retried += again;
      st_queries += 1u - again;
      if (again) {
        if (l == 0) {
          // lowered by a few ulps: the retry re-derives its filter scores with
          // another threshold, which may round them differently
          tau[hq + q] = tau_new - (fabsf(tau_new) * (1.0f / 1048576.0f) + 1e-30f);
          rlist[hq + atomicAdd(&rcount[h], 1)] = q;
        }
      } else {
        if (l == 0) {
          const unsigned fslot = atomicAdd(&hdr->fb_count, 1u);
          fblist[fslot] = static_cast<int>(hq + q);
        }
      }
    };

    if (n_valid <= k) {  // every valid key is kept
      issue_next();
      for (int t = l; t < k; t += kWave) out[t] = t < n_valid ? t : -1;
      if (seg != nullptr && l <= kGatherRanges)
        seg[(hq + q) * (kGatherRanges + 1) + l] =
            l == kGatherRanges ? n_valid : min(gather_range_start(gr, l), n_valid);
      ++st_queries;
      continue;
    }
    const int r0 = cur.r0, r1 = cur.r1;
    const bool overflow = r0 > capH || r1 > capH;
    const int c0 = min(r0, capH), c1 = min(r1, capH);
    const int c = c0 + c1;
    // more candidates than LDS holds: rank them from the lists in memory
    const bool wide = c > lcap;
    st_wide += wide ? 1u : 0u;
    const float tq = cur.tq;
    st_overflow += overflow && qlist == nullptr ? 1u : 0u;
    // Stage the candidates in LDS once (index i runs over half 0, then half 1)
    // as (order key of the filter score s~ = sum * f, key index).  The
    // filter parked sum - thr (its accumulators start at -thr).
    const float4 st = cur.st;
    const float kinv =
        __builtin_ldexpf(1.0f, -scale_exponent(__uint_as_float(kstat[kKeyStatWords * h + 2])));
    const float f = scale * st.z * kinv;
    const float tv = cur.tv;
    uint32_t kmin = ~0u, kmax = 0u;
    const uint2* list0 = cand + (hq + q) * 2 * static_cast<size_t>(capH);
    const uint2* list1 = list0 + capH;
    {
      auto stage = [&](int i, uint2 e) {
        const uint32_t key = order_key((__uint_as_float(e.y) + tv) * f);
        if (!wide) {
          ck[i] = key;
          cj[i] = candidate_key(e.x);
        }
        kmin = min(kmin, key);
        kmax = max(kmax, key);
      };
#pragma unroll
      for (int j = 0; j < kPrefetch; ++j) {
        const int i = l + kWave * j;
        if (i < c) stage(i, pre[j]);
      }
      issue_next();
      #pragma unroll 16
      for (int i = kWave * kPrefetch + l; i < c; i += kWave)
        stage(i, i < c0 ? list0[i] : list1[i - c0]);
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    wave_sync();
    if (c < k_i + (overflow ? 0 : 1)) {
      // Too few keys for a proven bound: the threshold was set too high.
      // Retry with a lower one, guessed from an exponential fit to the tail
      // the candidates do show (c keys at or above tau - m, the largest at
      // s_max), aiming at about 1.5 k keys; the retry proves it or, failing
      // that, the query goes to the exact fallback.
      float guess = __builtin_nanf("");
      if (!overflow && c >= 2 && tq > -INFINITY) {
        const float base = tq - score_margin(st.x, st.y, __uint_as_float(kstat[kKeyStatWords * h]),
                                             __uint_as_float(kstat[kKeyStatWords * h + 1]),
                                             scale, DP);
        const float span = fmaxf(key_to_float(kmax) - base, 1e-6f);
        const float lambda = __logf(static_cast<float>(c)) / span;
        guess = base - __logf(1.5f * static_cast<float>(k_i) / static_cast<float>(c)) / lambda;
      }
      unresolved(guess);
      continue;
    }
    // entry i of the lists in memory (wide queries), four per lane in flight
    constexpr int WB = 4;
    auto glob_entries = [&](int i0, uint2 (&e)[WB]) {
#pragma unroll
      for (int t = 0; t < WB; ++t) {
        const int i = min(i0 + t * kWave + l, c - 1);
        e[t] = i < c0 ? list0[i] : list1[i - c0];
      }
    };
    auto each_cand = [&](auto fn) {
      if (!wide) {
        #pragma unroll 1
        for (int i0 = 0; i0 < c; i0 += kWave) {
          const int i = i0 + l;
          const bool ok = i < c;
          fn(ok ? ck[i] : 0u, ok);
        }
      } else {
        #pragma unroll 1
        for (int i0 = 0; i0 < c; i0 += WB * kWave) {
          uint2 e[WB];
          glob_entries(i0, e);
#pragma unroll
          for (int t = 0; t < WB; ++t) {
            const bool ok = i0 + t * kWave + l < c;
            fn(ok ? order_key((__uint_as_float(e[t].y) + tv) * f) : 0u, ok);
          }
        }
      }
    };
    // The k-th largest filter score gives lo = (k-th) - m, a proven threshold
    // for any subset of the keys: k of them score >= lo.
    const float m = score_margin(st.x, st.y, __uint_as_float(kstat[kKeyStatWords * h]),
                                 __uint_as_float(kstat[kKeyStatWords * h + 1]), scale, DP);
    auto lower = [&](float x) { return (x - m) - (fabsf(x) + m) * (1.0f / 4194304.0f); };
    auto upper = [&](float x) { return (x + m) + (fabsf(x) + m) * (1.0f / 4194304.0f); };
    // |s - s~| bound of the same interval: m + (|s~| + m) 2^-22
    const float mslop = m + m * (1.0f / 4194304.0f);
    const uint32_t ak = wave_select_in<uint32_t>(k_i, hist, reinterpret_cast<uint32_t*>(cbuf),
                                                 each_cand, kmin, kmax);
    const float lo = lower(key_to_float(ak));
    // The list covers every key that can reach the top-k only if the filter's
    // threshold is proven, i.e. the k best candidates are certainly above it.
    if (overflow || !(lo >= tq)) {
      unresolved(lo);
      continue;
    }
    // The upper bound of the k-th value stands in for that of the (k+1)-th:
    // it is not smaller, so a key above it is still certainly kept.
    const float hi = fmaxf(tq, upper(key_to_float(ak)));
    // Certainly kept: l > hi; certainly out: u < lo; uncertain otherwise.
    auto cls_of = [&](uint32_t key) {
      const float x = key_to_float(key);
      return lower(x) > hi ? 1 : (upper(x) < lo ? 0 : 2);
    };

    // One pass classifies and compacts: certainly-kept and uncertain keys
    // stay, in list order, in place in cj (a chunk is read before it is
    // written, and writes never pass the chunk); uncertain ones carry bit 31
    // and are also listed in uj (with their filter score in ut) for the
    // exact re-score.
    // (A wide query's kept and uncertain keys number under k + ucap <= lcap
    // while nU <= ucap, since the certainly kept ones score above the k-th;
    // writes past lcap are dropped and the query then fails the nU test.)
    int run = 0, n0c = 0, nU = 0;
    auto classify = [&](int i, uint32_t ckey, int key) {
      const bool ok = i < c;
      const int cc = ok ? cls_of(ckey) : 0;
      const unsigned long long mu = __ballot(cc == 2);
      const unsigned long long mk = __ballot(cc != 0);
      if (cc == 2) {
        const int pos = nU + lane_rank(mu);
        if (pos < ucap) {
          uj[pos] = key;
          ut[pos] = key_to_float(ckey);
        }
      }
      wave_sync();
      const int pos = run + lane_rank(mk);
      if (cc != 0 && pos < lcap) cj[pos] = cc == 2 ? (key | INT_MIN) : key;
      nU += __builtin_popcountll(mu);
      run += __builtin_popcountll(mk);
      n0c += __builtin_popcountll(__ballot(cc != 0 && i < c0));
    };
    if (!wide) {
      #pragma unroll 1
      for (int i0 = 0; i0 < c; i0 += kWave) {
        const int i = i0 + l;
        const bool ok = i < c;
        classify(i, ok ? ck[i] : 0u, ok ? cj[i] : 0);
      }
    } else {
      #pragma unroll 1
      for (int i0 = 0; i0 < c; i0 += WB * kWave) {
        uint2 e[WB];
        glob_entries(i0, e);
#pragma unroll
        for (int t = 0; t < WB; ++t)
          classify(i0 + t * kWave + l, order_key((__uint_as_float(e[t].y) + tv) * f),
                   candidate_key(e[t].x));
      }
    }
    const int need = k_i - (run - nU);
    if (nU > ucap || need > nU || run > lcap) {
      unresolved(__builtin_nanf(""));
      continue;
    }
    wave_sync();
    // exact re-score of the uncertain keys: G lanes per key, 16 bytes each
    {
      constexpr int G = DP / 4;
      constexpr int KPI = kWave / G;     // keys per pass
      constexpr int UNR = 8;             // passes in flight (32 keys at d_proj 64)
      const int g = l % G, grp = l / G;
      const float4 qv = reinterpret_cast<const float4*>(q32 + (hq + q) * DP)[g];
      #pragma unroll 1
      for (int u0 = 0; u0 < nU; u0 += KPI * UNR) {
        float4 kv[UNR];
        #pragma unroll
        for (int t = 0; t < UNR; ++t) {
          const int u = u0 + t * KPI + grp;
          kv[t] = u < nU ? reinterpret_cast<const float4*>(k32 + (hq + uj[u]) * DP)[g]
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        #pragma unroll
        for (int t = 0; t < UNR; ++t) {
          const float p = group_sum<G>(group_partial<DP>(qv, kv[t]));
          const int u = u0 + t * KPI + grp;
          if (g == 0 && u < nU) {
            const float sx = p * scale;
            us[u] = sx;
            // the exact score must lie in the interval the margin gives the
            // filter score (the bounds lower/upper use); a key outside it
            // means the rounding bound behind the margin is wrong
            const float sf = ut[u];
            viol += fabsf(sx - sf) > __builtin_fmaf(fabsf(sf), 1.0f / 4194304.0f, mslop) ? 1u : 0u;
          }
        }
      }
    }
    wave_sync();
    unsigned long long kth = ~0ull;
    if (need > 0) {
      kth = wave_select<unsigned long long>(need, hist, cbuf, [&](auto fn) {
        #pragma unroll 1
        for (int u0 = 0; u0 < nU; u0 += kWave) {
          const int u = u0 + l;
          fn(u < nU ? rank_key(us[u], uj[u]) : 0ull, u < nU);
        }
      });
    }
    // Drop the uncertain keys that lose (in place again); they are met in the
    // order they were listed in uj.
    int run2 = 0, n0 = 0, upos = 0;
    #pragma unroll 1
    for (int i0 = 0; i0 < run; i0 += kWave) {
      const int i = i0 + l;
      const bool ok = i < run;
      const int e = ok ? cj[i] : 0;
      const bool unc = e < 0;
      const unsigned long long mu = __ballot(unc);
      bool take = ok && !unc;
      if (unc) {
        const int pos = upos + lane_rank(mu);
        take = need > 0 && rank_key(us[pos], uj[pos]) >= kth;
      }
      upos += __builtin_popcountll(mu);
      const unsigned long long tk = __ballot(take);
      wave_sync();
      if (take) cj[run2 + lane_rank(tk)] = e & INT_MAX;
      run2 += __builtin_popcountll(tk);
      n0 += __builtin_popcountll(__ballot(take && i < n0c));
    }
    wave_sync();
    // The merged row goes to the order-key area (free by now, at least k
    // entries), then to out in coalesced stores, -1 past the kept keys.
    int* mrow = reinterpret_cast<int*>(ck);
    merge_rows(cj, n0, cj + n0, run2 - n0, mrow);
    // the row's key-range starts: entries below r*L in either list
    if (seg != nullptr && l <= kGatherRanges) {
      const int x = gather_range_start(gr, l);
      seg[(hq + q) * (kGatherRanges + 1) + l] =
          l == kGatherRanges ? run2 : count_below(cj, n0, x) + count_below(cj + n0, run2 - n0, x);
    }
    wave_sync();
    #pragma unroll 1
    for (int t = l; t < k; t += kWave) out[t] = t < run2 ? mrow[t] : -1;
    st_rescored += static_cast<unsigned>(nU);
    ++st_queries;
    } while (false);
    if (!issued) issue_next();
    cur = nxt;
    nxt = nn;
  }
  const unsigned st_viol = static_cast<unsigned>(wave_sum_i(static_cast<int>(viol)));
  if (l == 0) {
    if (st_queries) atomicAdd(&hdr->queries, static_cast<unsigned long long>(st_queries));
    if (st_rescored) atomicAdd(&hdr->rescored, static_cast<unsigned long long>(st_rescored));
    if (st_overflow)
      atomicAdd(&hdr->overflow_queries, static_cast<unsigned long long>(st_overflow));
    if (st_retried) atomicAdd(&hdr->retried, static_cast<unsigned long long>(st_retried));
    if (st_viol) atomicAdd(&hdr->margin_violations, st_viol);
    if (st_wide) atomicAdd(&hdr->wide_queries, st_wide);
  }
}

// ------------------------------------------------------------ fallback ---
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int& total) {
  const int w = threadIdx.x / kWave, l = lane_id();
  const int incl = wave_incl_scan(v);
  if (l == kWave - 1) tmp[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < kWavesPerBlock; ++i) {
    const int t = tmp[i];
    if (i < w) off += t;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + incl - v;
}

// Exact selection for queued queries: score every valid key exactly into a
// per-workgroup scratch row, find the k-th largest score by radix select,
// and write keys above it plus the lowest-index ties, in ascending order.
// Persistent: each workgroup takes queued queries until the queue is empty.
template <int DP>
__global__ __launch_bounds__(kThreads) void fallback_kernel(
    const float* __restrict__ q32, const float* __restrict__ k32, const int* __restrict__ fblist,
    int N, int Npad, int k, int causal, float scale, float* __restrict__ scratch,
    int32_t* __restrict__ idx, int* __restrict__ seg, GatherRanges gr, WsHeader* __restrict__ hdr) {
  __shared__ float qrow[DP];
  __shared__ int hist[256];
  __shared__ int tmp[kWavesPerBlock];
  __shared__ int s_item, s_digit, s_above;
  const int tid = threadIdx.x;
  const unsigned n_items = hdr->fb_count;
  float* row = scratch + static_cast<size_t>(blockIdx.x) * Npad;
  for (;;) {
    __syncthreads();
    if (tid == 0) s_item = static_cast<int>(atomicAdd(&hdr->fb_next, 1u));
    __syncthreads();
    const int item = s_item;
    if (item >= static_cast<int>(n_items)) break;
    const int entry = fblist[item];
    const int h = entry / Npad, q = entry % Npad;
    const size_t hq = static_cast<size_t>(h) * Npad;
    const int n_valid = causal ? q + 1 : N;
    const int k_i = min(k, n_valid);
    if (tid < DP) qrow[tid] = q32[(hq + q) * DP + tid];
    __syncthreads();
    for (int j = tid; j < n_valid; j += kThreads)
      row[j] = exact_score<DP>(qrow, k32 + (hq + j) * DP, scale);
    __syncthreads();
    // k_i-th largest order key
    uint32_t prefix = 0, pmask = 0;
    int K = k_i;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < n_valid; j += kThreads) {
        const uint32_t key = order_key(row[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
      }
      __syncthreads();
      const int cval = hist[255 - tid];   // thread t owns bin 255 - t
      int total;
      const int excl = block_excl_scan(cval, tmp, total);
      if (excl < K && excl + cval >= K) {
        s_digit = 255 - tid;
        s_above = excl;
      }
      __syncthreads();
      K -= s_above;
      prefix |= static_cast<uint32_t>(s_digit) << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    // Keys strictly above the k-th score, then ties in ascending key order.
    // Each thread owns a contiguous range of keys, so two block scans give
    // every thread its first output position.
    const int L = (n_valid + kThreads - 1) / kThreads;
    const int j0 = min(n_valid, tid * L), j1 = min(n_valid, j0 + L);
    int gt = 0, eq = 0;
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = order_key(row[j]);
      gt += key > prefix ? 1 : 0;
      eq += key == prefix ? 1 : 0;
    }
    int gt_total, eq_total;
    const int gt_before = block_excl_scan(gt, tmp, gt_total);
    const int eq_before = block_excl_scan(eq, tmp, eq_total);
    const int ties_needed = k_i - gt_total;
    int32_t* out = idx + (hq / Npad * static_cast<size_t>(N) + q) * k;
    int pos = gt_before + min(eq_before, ties_needed);
    int eq_seen = eq_before;
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = order_key(row[j]);
      const bool tie = key == prefix;
      if (key > prefix || (tie && eq_seen < ties_needed)) out[pos++] = j;
      eq_seen += tie ? 1 : 0;
    }
    for (int t = k_i + tid; t < k; t += kThreads) out[t] = -1;
    if (seg != nullptr) {
      __syncthreads();   // the row written above is visible to the workgroup
      if (tid <= kGatherRanges)
        seg[(hq + q) * (kGatherRanges + 1) + tid] =
            tid == kGatherRanges ? k_i : count_below(out, k_i, gather_range_start(gr, tid));
    }
    if (tid == 0) atomicAdd(&hdr->fallback_queries, 1ull);
  }
}

// Compute units of the current device (cached per device).
int resident_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int DP>
hipError_t finalize_t(const Plan& p, const Bufs& b, int nh, float scale, int32_t* idx,
                      bool retry, int* seg, hipStream_t s) {
  // the uncertain band is ~8x narrower with fp16 filter operands than bf16
  // (about 37 and 280 keys at the headline size)
  const int ucap = p.filt ? 512 : 128;   // at least 128: its filter scores hold the rank buffer
  const int lcap = rerank_lds_cap(p.capH, p.k, ucap);
  const size_t per_wave = rerank_lds_per_wave(lcap, ucap);
  int wpb = static_cast<int>((64 * 1024) / per_wave);
  wpb = wpb < 1 ? 1 : (wpb > 4 ? 4 : wpb);
  // persistent waves striding over the queries of their head: as many
  // workgroups as the chip holds at once (LDS or registers bound how many
  // fit on a CU), so every wave works until the end: a workgroup beyond them
  // would start only when one finishes and then run its whole share alone
  const int per_cu = rerank_groups_per_cu(wpb, per_wave);
  const int resident = resident_cus() * per_cu;
  int gx = (p.N + wpb - 1) / wpb;
  const int per_head = (resident + nh - 1) / nh;
  gx = gx < per_head ? gx : per_head;
  const dim3 grid(gx, nh);
  const size_t lds = static_cast<size_t>(wpb) * per_wave;
  // one limit for every launch (at most four waves of at most 64 KB in all),
  // so concurrent calls with other sizes never lower it under each other
  static std::atomic<int> lds_set[kMaxDevices];
  hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(&finalize_kernel<DP>),
                                    64 * 1024, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((finalize_kernel<DP>), grid, dim3(wpb * kWave), lds, s, b.cand, b.cnt, b.rcnt,
                     b.tau, b.thr, b.qstat, b.kstat, b.qlo32, b.klo32, p.N, p.Npad, p.k, p.causal,
                     p.capH, lcap, ucap, scale, idx, retry ? b.rlist : static_cast<int*>(nullptr),
                     retry ? b.rcount : static_cast<int*>(nullptr), b.rlist, b.rcount, b.fblist,
                     seg, gather_ranges(p.N, p.causal), b.hdr);
  return hipGetLastError();
}

template <int DP>
hipError_t fallback_t(const Plan& p, const Bufs& b, float scale, int32_t* idx, int* seg,
                      hipStream_t s) {
  hipLaunchKernelGGL((fallback_kernel<DP>), dim3(kFallbackBlocks), dim3(kThreads), 0, s,
                     b.qlo32, b.klo32, b.fblist, p.N, p.Npad, p.k, p.causal, scale,
                     b.fbscratch, idx, seg, gather_ranges(p.N, p.causal), b.hdr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_finalize(const Plan& p, const Bufs& b, int nh, float score_scale,
                           int32_t* idx_chunk, bool retry, int* seg, hipStream_t s) {
  switch (p.dp) {
    case 16: return finalize_t<16>(p, b, nh, score_scale, idx_chunk, retry, seg, s);
    case 32: return finalize_t<32>(p, b, nh, score_scale, idx_chunk, retry, seg, s);
    case 64: return finalize_t<64>(p, b, nh, score_scale, idx_chunk, retry, seg, s);
    case 128: return finalize_t<128>(p, b, nh, score_scale, idx_chunk, retry, seg, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fallback(const Plan& p, const Bufs& b, int nh, float score_scale,
                           int32_t* idx_chunk, int* seg, hipStream_t s) {
  (void)nh;
  switch (p.dp) {
    case 16: return fallback_t<16>(p, b, score_scale, idx_chunk, seg, s);
    case 32: return fallback_t<32>(p, b, score_scale, idx_chunk, seg, s);
    case 64: return fallback_t<64>(p, b, score_scale, idx_chunk, seg, s);
    case 128: return fallback_t<128>(p, b, score_scale, idx_chunk, seg, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace sa
