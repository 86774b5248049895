// C entry points of libsparse_attn: host-side validation, the workspace plan
// and the per-chunk launch sequence.  Declarations and the contract of each
// entry point are in include/sparse_attn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <algorithm>
#include <atomic>
#include <cstring>

#include "sa_internal.h"
#include "sparse_attn.h"

namespace sa {

namespace {

constexpr size_t kAlign = 256;

constexpr int kDefaultChunkHeads = 8;

// The filter operand type an options struct asks for: 0 = fp16, 1 = bf16,
// -1 = not a filter type.  NULL options mean the defaults.
int filter_of(const sa_options* o) {
  if (o == nullptr || o->filter_dtype == SA_F16) return 0;
  return o->filter_dtype == SA_BF16 ? 1 : -1;
}
sa_profile* profile_of(const sa_options* o) { return o == nullptr ? nullptr : o->profile; }

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int round_up(int x, int m) { return (x + m - 1) / m * m; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_D(int D) { return D == 64 || D == 128; }
bool supported_dp(int dp) { return dp == 16 || dp == 32 || dp == 64 || dp == 128; }

// Shape checks shared by every entry point that takes Q/K/V.
int check_dims(const sa_dims& d, int k) {
  if (d.B < 1 || d.H < 1 || d.N < 1) return SA_ERR_SHAPE;
  if (k < 1) return SA_ERR_SHAPE;
  if (static_cast<long long>(d.N) * k >= (1ll << 31)) return SA_ERR_SHAPE;
  if (static_cast<long long>(d.B) * d.H >= (1ll << 31)) return SA_ERR_SHAPE;
  if (k > SA_K_MAX) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

int check_scorer_args(const void* Q, const void* K, const void* Pq, const void* Pk,
                      const sa_dims& d, int dp, int k, int dtype, float score_scale) {
  if (!Q || !K || !Pq || !Pk) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (!supported_D(d.D) || !supported_dp(dp)) return SA_ERR_UNSUPPORTED;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (!(score_scale > 0.0f) || !std::isfinite(score_scale)) return SA_ERR_SHAPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(Pq) || !aligned16(Pk)) return SA_ERR_ALIGN;
  return SA_OK;
}

// As SA_TIMED, in an entry point: a launch error returns SA_ERR_HIP.
#define SA_TIMED_STATUS(name, call)            \
  do {                                         \
    const int t_ = prof_begin(prof, name, s);  \
    hipError_t e_ = (call);                    \
    prof_end(prof, t_, s);                     \
    if (e_ != hipSuccess) return SA_ERR_HIP;   \
  } while (0)

// Runs `call` between the optional timing events of `name` (into `prof`).
#define SA_TIMED(name, call)                   \
  do {                                         \
    const int t_ = prof_begin(prof, name, s);  \
    hipError_t e_ = (call);                    \
    prof_end(prof, t_, s);                     \
    if (e_ != hipSuccess) return e_;           \
  } while (0)

hipError_t run_topk_chunk(const Plan& p, const Bufs& b, const void* Q, const void* K,
                          const void* Pq, const void* Pk, int h0, int nh, float scale,
                          int32_t* idx_chunk, int first, int* seg, sa_profile* prof,
                          hipStream_t s, const float* smooth_gap = nullptr) {
  SA_TIMED("init", launch_init_chunk(p, b, first, s));
  SA_TIMED("project", launch_project(p, b, Q, K, Pq, Pk, h0, nh, s));
  SA_TIMED("pack", launch_pack_keys(p, b, nh, s));
  // the sample pass only matters when some query has more valid keys than
  // its candidate lists can hold outright
  const bool need_sample = p.N > 2 * p.capH - 64;
  if (need_sample) SA_TIMED("sample", launch_sample_maxima(p, b, nh, scale, s));
  SA_TIMED("threshold", launch_threshold(p, b, nh, scale, s));
  SA_TIMED("filter", launch_filter(p, b, nh, scale, false, s));
  SA_TIMED("rerank", launch_finalize(p, b, nh, scale, idx_chunk, false, seg, s));
  // queries whose threshold was not good enough, again with a proven one
  SA_TIMED("filter_retry", launch_filter(p, b, nh, scale, true, s));
  SA_TIMED("rerank_retry", launch_finalize(p, b, nh, scale, idx_chunk, true, seg, s));
  SA_TIMED("fallback", launch_fallback(p, b, nh, scale, idx_chunk, seg, s));
  if (smooth_gap != nullptr)
    SA_TIMED("smooth", launch_smooth(p, b, nh, scale, *smooth_gap, idx_chunk, s));
  return hipSuccess;
}

hipError_t timed_gather(const void* Q, const void* K, const void* V, const int32_t* idx, int k,
                        int nheads, int N, int D, float scale, int dtype, void* O,
                        sa_profile* prof, hipStream_t s) {
  SA_TIMED("gather", launch_gather(Q, K, V, idx, k, nheads, N, D, scale, dtype, O, s));
  return hipSuccess;
}

hipError_t timed_dump(const Plan& p, const Bufs& b, const void* Q, const void* K, const void* Pq,
                      const void* Pk, int h0, int nh, float scale, int row_begin, int row_count,
                      float* Sc, int first, sa_profile* prof, hipStream_t s) {
  SA_TIMED("init", launch_init_chunk(p, b, first, s));
  SA_TIMED("project", launch_project(p, b, Q, K, Pq, Pk, h0, nh, s));
  SA_TIMED("dump", launch_dump(p, b, nh, scale, row_begin, row_count, Sc, s));
  return hipSuccess;
}

hipError_t timed_band(int nheads, int N, int w_left, int w_right, int32_t* idx, int k,
                      sa_profile* prof, hipStream_t s) {
  SA_TIMED("band", launch_band(nheads, N, w_left, w_right, idx, k, s));
  return hipSuccess;
}

// Largest chunk (in heads) whose workspace fits ws_bytes; 0 if none.
int chunk_heads_for(const sa_dims& d, int dp, int k, int causal, int dtype, int with_idx,
                    size_t ws_bytes) {
  const int BH = d.B * d.H;
  Plan p1, p2;
  if (!make_plan(p1, d.B, d.H, d.N, d.D, dp, k, causal, dtype, with_idx, 1, 0)) return 0;
  if (BH == 1) return p1.total <= ws_bytes ? 1 : 0;
  if (!make_plan(p2, d.B, d.H, d.N, d.D, dp, k, causal, dtype, with_idx, 2, 0)) return 0;
  if (p1.total > ws_bytes) return 0;
  const size_t per_head = p2.total - p1.total;
  const size_t fixed = p1.total - per_head;
  size_t h = (ws_bytes - fixed) / per_head;
  if (h > static_cast<size_t>(BH)) h = BH;
  // keep head-chunk indices within int range of the queue entries
  while (h > 1) {
    Plan ph;
    if (make_plan(ph, d.B, d.H, d.N, d.D, dp, k, causal, dtype, with_idx, static_cast<int>(h), 0) &&
        ph.total <= ws_bytes)
      break;
    --h;
  }
  return static_cast<int>(h);
}

}  // namespace

bool make_plan(Plan& p, int B, int H, int N, int D, int dp, int k, int causal, int dtype,
               int with_idx, int heads_per_chunk, int filt) {
  p.B = B; p.H = H; p.N = N; p.D = D; p.dp = dp; p.k = k; p.causal = causal ? 1 : 0;
  p.dtype = dtype;
  p.filt = filt ? 1 : 0;
  p.BH = B * H;
  p.hc = heads_per_chunk < 1 ? 1 : (heads_per_chunk > p.BH ? p.BH : heads_per_chunk);
  p.Npad = round_up(N, kRowPad);
  // sample stride: the largest power of two <= beta*k/32 (in [1, 16]), so
  // that the sample rank stays near 48 and the threshold stays steady
  p.sstride = 1;
  while (p.sstride < kMaxSampleStride && 2 * p.sstride * 32 <= kTauBeta * k) p.sstride *= 2;
  p.Ns = (N + p.sstride - 1) / p.sstride;
  p.Nspad = p.Npad / p.sstride;
  // two query halves of capH candidates each (1.25 k, at least 256, at most
  // 2048; about 0.85 k land in a half at the headline size); a list that
  // overflows is filtered again with a proven threshold
  p.capH = std::min(2048, round_up(std::max(5 * k / 4, 256), 64));
  // block maxima per query: fewer than 8r + 40 (the block size keeps under
  // 8r blocks, plus tile rounding), with r <= beta*k/s + beta*k/n + 1 for the
  // rows that use a threshold (n > 2 capH - 64 valid keys)
  {
    const int rmax = static_cast<int>(kTauBeta * k / p.sstride +
                                      kTauBeta * k / std::max(1, 2 * p.capH - 64)) + 2;
    p.NB = 8 * rmax + 40;
  }
  p.with_idx = with_idx ? 1 : 0;
  // K and V rows of a head beyond one XCD's L2: the fused forward gathers by
  // key range (its row offsets are 32-bit bytes within one head)
  const size_t head_bytes = static_cast<size_t>(N) * D * (dtype ? 2 : 4);
  p.gsplit = N > 8192 && head_bytes <= 0xFFFFFFFFull ? 1 : 0;
  const size_t hc = static_cast<size_t>(p.hc);
  const size_t Np = static_cast<size_t>(p.Npad);
  // queue entries and per-chunk row indices are int
  if (hc * Np * 2 >= (1ull << 31)) return false;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p.off_hdr = take(sizeof(WsHeader));
  p.off_qlo32 = take(hc * Np * dp * 4);
  p.off_klo32 = take(hc * Np * dp * 4);
  p.off_qlo16 = take(hc * Np * dp * 2);
  p.off_klo16 = take(hc * Np * dp * 2);
  p.off_ksamp = take(hc * static_cast<size_t>(p.Nspad) * dp * 2);
  p.off_qstat = take(hc * Np * 16);
  p.off_kstat = take(hc * kKeyStatWords * 4);
  p.off_bm = take(hc * static_cast<size_t>(p.NB) * Np * 2);
  p.off_tau = take(hc * Np * 4);
  p.off_thr = take(hc * Np * 4);
  p.off_cand = take(hc * Np * 2 * static_cast<size_t>(p.capH) * 8);
  p.off_cnt = take(hc * Np * 2 * 4);
  p.off_rcnt = take(hc * Np * 2 * kRetrySplit * 4);
  p.off_rlist = take(hc * Np * 4);
  p.off_rcount = take(hc * 4);
  p.off_fblist = take(hc * Np * 4);
  p.off_fbscratch = take(static_cast<size_t>(kFallbackBlocks) * Np * 4);
  p.off_idx = take(p.with_idx ? hc * static_cast<size_t>(N) * k * 4 : 0);
  p.off_seg = take(p.gsplit ? hc * Np * (kGatherRanges + 1) * 4 : 0);
  p.off_part = take(p.gsplit ? Np * kGatherRanges * static_cast<size_t>(D + 4) * 4 : 0);
  p.total = off;
  return true;
}

hipError_t set_lds_limit_once(const void* kernel, int bytes, std::atomic<int>* flags) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached && flags[dev].load(std::memory_order_acquire) == bytes) return hipSuccess;
  // racing threads both set the same value: harmless
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && cached) flags[dev].store(bytes, std::memory_order_release);
  return e;
}

Bufs bufs_of(const Plan& p, void* ws) {
  unsigned char* base = static_cast<unsigned char*>(ws);
  Bufs b;
  b.hdr = reinterpret_cast<WsHeader*>(base + p.off_hdr);
  b.qlo32 = reinterpret_cast<float*>(base + p.off_qlo32);
  b.klo32 = reinterpret_cast<float*>(base + p.off_klo32);
  b.qlo16 = reinterpret_cast<bf16_t*>(base + p.off_qlo16);
  b.klo16 = reinterpret_cast<bf16_t*>(base + p.off_klo16);
  b.ksamp = reinterpret_cast<bf16_t*>(base + p.off_ksamp);
  b.qstat = reinterpret_cast<float4*>(base + p.off_qstat);
  b.kstat = reinterpret_cast<uint32_t*>(base + p.off_kstat);
  b.bm = reinterpret_cast<uint16_t*>(base + p.off_bm);
  b.tau = reinterpret_cast<float*>(base + p.off_tau);
  b.thr = reinterpret_cast<float*>(base + p.off_thr);
  b.cand = reinterpret_cast<uint2*>(base + p.off_cand);
  b.cnt = reinterpret_cast<int*>(base + p.off_cnt);
  b.rcnt = reinterpret_cast<int*>(base + p.off_rcnt);
  b.rlist = reinterpret_cast<int*>(base + p.off_rlist);
  b.rcount = reinterpret_cast<int*>(base + p.off_rcount);
  b.fblist = reinterpret_cast<int*>(base + p.off_fblist);
  b.fbscratch = reinterpret_cast<float*>(base + p.off_fbscratch);
  b.idx = p.with_idx ? reinterpret_cast<int32_t*>(base + p.off_idx) : nullptr;
  b.seg = p.gsplit ? reinterpret_cast<int*>(base + p.off_seg) : nullptr;
  b.part = p.gsplit ? reinterpret_cast<float*>(base + p.off_part) : nullptr;
  return b;
}

}  // namespace sa

using namespace sa;

extern "C" {

size_t sparse_attn_workspace_size_for_chunk(sa_dims d, int32_t d_proj, int32_t k, int32_t causal,
                                            int32_t dtype, int32_t with_idx,
                                            int32_t heads_per_chunk) {
  if (check_dims(d, k) != SA_OK || !supported_D(d.D) || !supported_dp(d_proj)) return 0;
  if (dtype != SA_F32 && dtype != SA_BF16) return 0;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, k, causal, dtype, with_idx, heads_per_chunk, 0))
    return 0;
  return p.total;
}

size_t sparse_attn_workspace_size(sa_dims d, int32_t d_proj, int32_t k, int32_t causal,
                                  int32_t dtype, int32_t with_idx) {
  if (d.B < 1 || d.H < 1) return 0;
  const long long BH = static_cast<long long>(d.B) * d.H;
  const int hc = BH < kDefaultChunkHeads ? static_cast<int>(BH) : kDefaultChunkHeads;
  return sparse_attn_workspace_size_for_chunk(d, d_proj, k, causal, dtype, with_idx, hc);
}

int sparse_attn_scores_topk(const void* Q, const void* K, const void* Pq, const void* Pk,
                            sa_dims d, int32_t d_proj, int32_t k, int32_t causal,
                            float score_scale, int32_t dtype, int32_t* idx, void* ws,
                            size_t ws_bytes, const sa_options* opts, void* stream) {
  int st = check_scorer_args(Q, K, Pq, Pk, d, d_proj, k, dtype, score_scale);
  if (st != SA_OK) return st;
  const int filt = filter_of(opts);
  if (filt < 0) return SA_ERR_UNSUPPORTED;
  sa_profile* prof = profile_of(opts);
  if (!idx || !ws) return SA_ERR_NULL;
  if (!aligned16(idx) || !aligned16(ws)) return SA_ERR_ALIGN;
  const int hc = chunk_heads_for(d, d_proj, k, causal, dtype, 0, ws_bytes);
  if (hc < 1) return SA_ERR_WORKSPACE;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, k, causal, dtype, 0, hc, filt))
    return SA_ERR_SHAPE;
  const Bufs b = bufs_of(p, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int h0 = 0; h0 < p.BH; h0 += p.hc) {
    const int nh = p.BH - h0 < p.hc ? p.BH - h0 : p.hc;
    int32_t* idx_chunk = idx + static_cast<size_t>(h0) * d.N * k;
    if (run_topk_chunk(p, b, Q, K, Pq, Pk, h0, nh, score_scale, idx_chunk, h0 == 0, nullptr,
                       prof, s) != hipSuccess)
      return SA_ERR_HIP;
  }
  return SA_OK;
}

int sparse_attn_gather(const void* Q, const void* K, const void* V, const int32_t* idx,
                       int32_t k, sa_dims d, float softmax_scale, int32_t dtype, void* O,
                       const sa_options* opts, void* stream) {
  if (!Q || !K || !V || !idx || !O) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (!supported_D(d.D)) return SA_ERR_UNSUPPORTED;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return SA_ERR_SHAPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(idx) || !aligned16(O))
    return SA_ERR_ALIGN;
  return timed_gather(Q, K, V, idx, k, d.B * d.H, d.N, d.D, softmax_scale, dtype, O,
                      profile_of(opts), static_cast<hipStream_t>(stream)) == hipSuccess
             ? SA_OK
             : SA_ERR_HIP;
}

// ------------------------------------------- gather with a workspace ---
namespace {
struct GatherPlan {
  size_t off_seg, off_list, off_count, off_part, total;
};
// The key-range path applies as in the fused forward: N > 8192 and a head's
// K rows addressable with 32-bit byte offsets (and every row numbered by an
// int32 in the list of rows it leaves to the single pass); total = 0
// otherwise.
GatherPlan gather_plan(const sa_dims& d, int dtype) {
  GatherPlan p{};
  const size_t esz = dtype == SA_F32 ? 4 : 2;
  const size_t rows = static_cast<size_t>(d.B) * d.H * d.N;
  if (!(d.N > 8192 && static_cast<size_t>(d.N) * d.D * esz <= 0xFFFFFFFFull &&
        rows <= 0x7FFFFFFFull))
    return p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p.off_seg = take(rows * (kGatherRanges + 1) * 4);
  p.off_list = take(rows * 4);
  p.off_count = take(4);
  p.off_part = take(static_cast<size_t>(d.N) * kGatherRanges * (static_cast<size_t>(d.D) + 4) * 4);
  p.total = off;
  return p;
}
}  // namespace

size_t sparse_attn_gather_workspace_size(sa_dims d, int32_t k, int32_t dtype) {
  if (check_dims(d, k) != SA_OK || !supported_D(d.D)) return 0;
  if (dtype != SA_F32 && dtype != SA_BF16) return 0;
  return gather_plan(d, dtype).total;
}

int sparse_attn_gather_ws(const void* Q, const void* K, const void* V, const int32_t* idx,
                          int32_t k, sa_dims d, float softmax_scale, int32_t dtype, void* O,
                          void* ws, size_t ws_bytes, const sa_options* opts, void* stream) {
  if (!Q || !K || !V || !idx || !O) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (!supported_D(d.D)) return SA_ERR_UNSUPPORTED;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return SA_ERR_SHAPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(idx) || !aligned16(O))
    return SA_ERR_ALIGN;
  sa_profile* prof = profile_of(opts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const GatherPlan p = gather_plan(d, dtype);
  if (p.total == 0)
    return timed_gather(Q, K, V, idx, k, d.B * d.H, d.N, d.D, softmax_scale, dtype, O, prof, s) ==
                   hipSuccess
               ? SA_OK
               : SA_ERR_HIP;
  if (!ws) return SA_ERR_NULL;
  if (!aligned16(ws)) return SA_ERR_ALIGN;
  if (ws_bytes < p.total) return SA_ERR_WORKSPACE;
  unsigned char* base = static_cast<unsigned char*>(ws);
  int* seg = reinterpret_cast<int*>(base + p.off_seg);
  int* list = reinterpret_cast<int*>(base + p.off_list);
  int* count = reinterpret_cast<int*>(base + p.off_count);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  const int BH = d.B * d.H;
  SA_TIMED_STATUS("gather_check", launch_gather_check(idx, k, BH, d.N, seg, list, count, s));
  const size_t esz = dtype == SA_F32 ? 4 : 2;
  const size_t head = static_cast<size_t>(d.N) * d.D * esz;
  for (int h = 0; h < BH; ++h) {
    if (launch_gather_split(static_cast<const unsigned char*>(Q) + h * head,
                            static_cast<const unsigned char*>(K) + h * head,
                            static_cast<const unsigned char*>(V) + h * head,
                            idx + static_cast<size_t>(h) * d.N * k, k, d.N, d.D, softmax_scale,
                            dtype, seg + static_cast<size_t>(h) * d.N * (kGatherRanges + 1), part,
                            static_cast<unsigned char*>(O) + h * head, prof, s) != hipSuccess)
      return SA_ERR_HIP;
  }
  // rows the ranges could not take (their merged output was zero) last
  SA_TIMED_STATUS("gather_rest", launch_gather_list(Q, K, V, idx, k, d.N, d.D, softmax_scale,
                                                    dtype, list, count, O, s));
  return SA_OK;
}

int sparse_attn_fwd(const void* Q, const void* K, const void* V, const void* Pq, const void* Pk,
                    sa_dims d, int32_t d_proj, int32_t k, int32_t causal, float score_scale,
                    float softmax_scale, int32_t dtype, void* O, int32_t* idx_or_null, void* ws,
                    size_t ws_bytes, const sa_options* opts, void* stream) {
  int st = check_scorer_args(Q, K, Pq, Pk, d, d_proj, k, dtype, score_scale);
  if (st != SA_OK) return st;
  const int filt = filter_of(opts);
  if (filt < 0) return SA_ERR_UNSUPPORTED;
  sa_profile* prof = profile_of(opts);
  if (!V || !O || !ws) return SA_ERR_NULL;
  if (!std::isfinite(softmax_scale)) return SA_ERR_SHAPE;
  if (!aligned16(V) || !aligned16(O) || !aligned16(ws)) return SA_ERR_ALIGN;
  if (idx_or_null && !aligned16(idx_or_null)) return SA_ERR_ALIGN;
  const int with_idx = idx_or_null ? 0 : 1;
  const int hc = chunk_heads_for(d, d_proj, k, causal, dtype, with_idx, ws_bytes);
  if (hc < 1) return SA_ERR_WORKSPACE;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, k, causal, dtype, with_idx, hc, filt))
    return SA_ERR_SHAPE;
  const Bufs b = bufs_of(p, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = dtype == SA_F32 ? 4 : 2;
  for (int h0 = 0; h0 < p.BH; h0 += p.hc) {
    const int nh = p.BH - h0 < p.hc ? p.BH - h0 : p.hc;
    int32_t* idx_chunk =
        idx_or_null ? idx_or_null + static_cast<size_t>(h0) * d.N * k : b.idx;
    if (run_topk_chunk(p, b, Q, K, Pq, Pk, h0, nh, score_scale, idx_chunk, h0 == 0,
                       p.gsplit ? b.seg : nullptr, prof, s) != hipSuccess)
      return SA_ERR_HIP;
    const size_t off = static_cast<size_t>(h0) * d.N * d.D * esz;
    const unsigned char* Qc = static_cast<const unsigned char*>(Q) + off;
    const unsigned char* Kc = static_cast<const unsigned char*>(K) + off;
    const unsigned char* Vc = static_cast<const unsigned char*>(V) + off;
    unsigned char* Oc = static_cast<unsigned char*>(O) + off;
    if (p.gsplit) {
      const size_t head = static_cast<size_t>(d.N) * d.D * esz;
      for (int hh = 0; hh < nh; ++hh) {
        if (launch_gather_split(Qc + hh * head, Kc + hh * head, Vc + hh * head,
                                idx_chunk + static_cast<size_t>(hh) * d.N * k, k, d.N, d.D,
                                softmax_scale, dtype,
                                b.seg + static_cast<size_t>(hh) * p.Npad * (kGatherRanges + 1),
                                b.part, Oc + hh * head, prof, s) != hipSuccess)
          return SA_ERR_HIP;
      }
    } else if (timed_gather(Qc, Kc, Vc, idx_chunk, k, nh, d.N, d.D, softmax_scale, dtype, Oc,
                            prof, s) != hipSuccess) {
      return SA_ERR_HIP;
    }
  }
  return SA_OK;
}

int sparse_attn_scores_topk_smoothed(const void* Q, const void* K, const void* Pq,
                                     const void* Pk, sa_dims d, int32_t d_proj, int32_t k,
                                     int32_t causal, float score_scale, float gap, int32_t dtype,
                                     int32_t* idx, void* ws, size_t ws_bytes,
                                     const sa_options* opts, void* stream) {
  if (k < 1) return SA_ERR_SHAPE;
  if (k >= SA_K_MAX) return SA_ERR_UNSUPPORTED;        // rows hold k + 1 entries
  const int k1 = k + 1;
  int st = check_scorer_args(Q, K, Pq, Pk, d, d_proj, k1, dtype, score_scale);
  if (st != SA_OK) return st;
  if (std::isnan(gap)) return SA_ERR_SHAPE;
  const int filt = filter_of(opts);
  if (filt < 0) return SA_ERR_UNSUPPORTED;
  sa_profile* prof = profile_of(opts);
  if (!idx || !ws) return SA_ERR_NULL;
  if (!aligned16(idx) || !aligned16(ws)) return SA_ERR_ALIGN;
  const int hc = chunk_heads_for(d, d_proj, k1, causal, dtype, 0, ws_bytes);
  if (hc < 1) return SA_ERR_WORKSPACE;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, k1, causal, dtype, 0, hc, filt))
    return SA_ERR_SHAPE;
  const Bufs b = bufs_of(p, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int h0 = 0; h0 < p.BH; h0 += p.hc) {
    const int nh = p.BH - h0 < p.hc ? p.BH - h0 : p.hc;
    int32_t* idx_chunk = idx + static_cast<size_t>(h0) * d.N * k1;
    if (run_topk_chunk(p, b, Q, K, Pq, Pk, h0, nh, score_scale, idx_chunk, h0 == 0, nullptr,
                       prof, s, &gap) != hipSuccess)
      return SA_ERR_HIP;
  }
  return SA_OK;
}

// ------------------------------------------------------------- decode ---
namespace {
struct DecodePlan {
  size_t off_qlo32, off_qlo16, off_qstat, off_scores, off_idx, off_hist, off_ccount, off_cand,
      off_selinfo, off_part, total;
};
DecodePlan decode_plan(const sa_dims& d, int dp, int k) {
  const size_t BH = static_cast<size_t>(d.B) * d.H;
  const size_t nsl = static_cast<size_t>(decode_slices(d.N));
  DecodePlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p.off_qlo32 = take(BH * dp * 4);
  p.off_qlo16 = take(BH * dp * 2);
  p.off_qstat = take(BH * 16);
  p.off_scores = take(BH * static_cast<size_t>(d.N) * 4);
  p.off_idx = take(BH * static_cast<size_t>(k) * 4);
  p.off_hist = take(BH * kDecodeHistBins * 4);
  p.off_ccount = take(BH * nsl * 4);
  p.off_cand = take(BH * nsl * kDecodeCandCap * 8);
  p.off_selinfo = take(BH * 8);
  p.off_part = take(BH * kGatherRanges * (static_cast<size_t>(d.D) + 4) * 4);
  p.total = off;
  return p;
}
}  // namespace

size_t sparse_attn_decode_workspace_size(sa_dims d, int32_t d_proj, int32_t k) {
  if (check_dims(d, k) != SA_OK || !supported_dp(d_proj)) return 0;
  return decode_plan(d, d_proj, k).total;
}

int sparse_attn_decode_append_keys(const void* K_new, const void* Pk, sa_dims d, int32_t d_proj,
                                   int32_t dtype, float* klow_cache, int32_t Ncap, int32_t pos,
                                   const sa_options* opts, void* stream) {
  if (!K_new || !Pk || !klow_cache) return SA_ERR_NULL;
  int st = check_dims(d, 1);
  if (st != SA_OK) return st;
  if (!supported_D(d.D) || !supported_dp(d_proj)) return SA_ERR_UNSUPPORTED;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (Ncap < 1 || pos < 0 || pos > Ncap - d.N) return SA_ERR_SHAPE;
  if (!aligned16(K_new) || !aligned16(Pk) || !aligned16(klow_cache)) return SA_ERR_ALIGN;
  sa_profile* prof = profile_of(opts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SA_TIMED_STATUS("decode_append", launch_project_rows(K_new, Pk, d.B * d.H, d.N, Ncap, d.D,
                                                       d_proj, dtype, 1,
                                                       klow_cache + static_cast<size_t>(pos) * d_proj,
                                                       nullptr, nullptr, s));
  return SA_OK;
}

namespace {
// Argument checks shared by both decode entry points (the workspace aside).
int check_decode_args(const void* q, const void* Kc, const void* Vc, const float* klow_cache,
                      const void* Pq, const sa_dims& d, int d_proj, int len, int k,
                      float score_scale, float softmax_scale, int dtype, const void* O,
                      const int32_t* idx_or_null, const int32_t* counts_or_null) {
  if (!q || !Kc || !Vc || !klow_cache || !Pq || !O) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (!supported_D(d.D) || !supported_dp(d_proj)) return SA_ERR_UNSUPPORTED;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (len < 1 || len > d.N) return SA_ERR_SHAPE;
  if (!(score_scale > 0.0f) || !std::isfinite(score_scale) || !std::isfinite(softmax_scale))
    return SA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(Kc) || !aligned16(Vc) || !aligned16(klow_cache) ||
      !aligned16(Pq) || !aligned16(O))
    return SA_ERR_ALIGN;
  if ((idx_or_null && !aligned16(idx_or_null)) || (counts_or_null && !aligned16(counts_or_null)))
    return SA_ERR_ALIGN;
  return SA_OK;
}

// The decode launches over a workspace laid out by decode_plan.
int run_decode(const void* q, const void* Kc, const void* Vc, const float* klow_cache,
               const void* Pq, const sa_dims& d, int d_proj, int len, int k, float score_scale,
               float softmax_scale, int dtype, void* O, int32_t* idx_or_null,
               int32_t* counts_or_null, void* ws, sa_profile* prof, hipStream_t s) {
  const DecodePlan p = decode_plan(d, d_proj, k);
  unsigned char* base = static_cast<unsigned char*>(ws);
  float* qlo32 = reinterpret_cast<float*>(base + p.off_qlo32);
  uint16_t* qlo16 = reinterpret_cast<uint16_t*>(base + p.off_qlo16);
  float4* qstat = reinterpret_cast<float4*>(base + p.off_qstat);
  float* scores = reinterpret_cast<float*>(base + p.off_scores);
  int32_t* idx = idx_or_null ? idx_or_null : reinterpret_cast<int32_t*>(base + p.off_idx);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + p.off_hist);
  int* ccount = reinterpret_cast<int*>(base + p.off_ccount);
  uint2* cand = reinterpret_cast<uint2*>(base + p.off_cand);
  int2* selinfo = reinterpret_cast<int2*>(base + p.off_selinfo);
  float* part = reinterpret_cast<float*>(base + p.off_part);
  const int BH = d.B * d.H;
  SA_TIMED_STATUS("decode_clear", launch_decode_clear(hist, BH, s));
  SA_TIMED_STATUS("decode_project", launch_project_rows(q, Pq, BH, 1, 1, d.D, d_proj, dtype, 0,
                                                        qlo32, qlo16, qstat, s));
  SA_TIMED_STATUS("decode_scores", launch_decode_scores(qlo32, 1, klow_cache, d.N, len, BH,
                                                        d_proj, score_scale, scores, hist, s));
  SA_TIMED_STATUS("decode_collect", launch_decode_collect(scores, d.N, len, BH, k, hist, cand,
                                                          ccount, selinfo, s));
  SA_TIMED_STATUS("decode_select", launch_decode_select(scores, len, BH, k, cand, ccount,
                                                        selinfo, idx, counts_or_null, d.N, s));
  SA_TIMED_STATUS("decode_gather", launch_decode_gather_part(q, Kc, Vc, idx, k, len, BH, d.N,
                                                             d.D, softmax_scale, dtype, part, s));
  SA_TIMED_STATUS("decode_gather_merge", launch_decode_gather_merge(part, BH, d.D, dtype, O, s));
  return SA_OK;
}
}  // namespace

size_t sparse_attn_decode_noalloc_max_bytes(void) { return decode_scratch_bytes(); }

int sparse_attn_decode_noalloc(const void* q, const void* Kc, const void* Vc,
                               const float* klow_cache, const void* Pq, sa_dims d,
                               int32_t d_proj, int32_t len, int32_t k, float score_scale,
                               float softmax_scale, int32_t dtype, void* O, int32_t* idx_or_null,
                               int32_t* counts_or_null, void* stream) {
  int st = check_decode_args(q, Kc, Vc, klow_cache, Pq, d, d_proj, len, k, score_scale,
                             softmax_scale, dtype, O, idx_or_null, counts_or_null);
  if (st != SA_OK) return st;
  if (decode_plan(d, d_proj, k).total > decode_scratch_bytes()) return SA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (decode_scratch(&ws) != hipSuccess) return SA_ERR_HIP;
  return run_decode(q, Kc, Vc, klow_cache, Pq, d, d_proj, len, k, score_scale, softmax_scale,
                    dtype, O, idx_or_null, counts_or_null, ws, nullptr,
                    static_cast<hipStream_t>(stream));
}

int sparse_attn_decode(const void* q, const void* Kc, const void* Vc, const float* klow_cache,
                       const void* Pq, sa_dims d, int32_t d_proj, int32_t len, int32_t k,
                       float score_scale, float softmax_scale, int32_t dtype, void* O,
                       int32_t* idx_or_null, int32_t* counts_or_null, void* ws, size_t ws_bytes,
                       const sa_options* opts, void* stream) {
  int st = check_decode_args(q, Kc, Vc, klow_cache, Pq, d, d_proj, len, k, score_scale,
                             softmax_scale, dtype, O, idx_or_null, counts_or_null);
  if (st != SA_OK) return st;
  if (!ws) return SA_ERR_NULL;
  if (!aligned16(ws)) return SA_ERR_ALIGN;
  if (ws_bytes < decode_plan(d, d_proj, k).total) return SA_ERR_WORKSPACE;
  return run_decode(q, Kc, Vc, klow_cache, Pq, d, d_proj, len, k, score_scale, softmax_scale,
                    dtype, O, idx_or_null, counts_or_null, ws, profile_of(opts),
                    static_cast<hipStream_t>(stream));
}

// ---------------------------------------------- block-granular selection ---
namespace {
constexpr int kBlockKbMaxApi = 32;
struct BlockPlan {
  size_t off_q32, off_k32, off_kbar, off_sel, total;
  int NB;
};
bool block_plan(BlockPlan& p, const sa_dims& d, int dp, int block, int kb) {
  if (block < 1 || kb < 1 || kb > kBlockKbMaxApi) return false;
  if (static_cast<long long>(block) * kb > SA_K_MAX) return false;
  const size_t BH = static_cast<size_t>(d.B) * d.H, N = static_cast<size_t>(d.N);
  p.NB = static_cast<int>((N + block - 1) / block);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  p.off_q32 = take(BH * N * dp * 4);
  p.off_k32 = take(BH * N * dp * 4);
  p.off_kbar = take(BH * static_cast<size_t>(p.NB) * dp * 4);
  p.off_sel = take(BH * N * kb * 4);
  p.total = off;
  return true;
}
int check_block_args(const sa_dims& d, int dp, int block, int kb) {
  int st = check_dims(d, 1);
  if (st != SA_OK) return st;
  if (block < 1 || kb < 1) return SA_ERR_SHAPE;
  if (kb > kBlockKbMaxApi || static_cast<long long>(block) * kb > SA_K_MAX)
    return SA_ERR_UNSUPPORTED;
  if (static_cast<long long>(d.N) * block * kb >= (1ll << 31)) return SA_ERR_SHAPE;
  if (!supported_D(d.D) || !supported_dp(dp)) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}
}  // namespace

size_t sparse_attn_block_workspace_size(sa_dims d, int32_t d_proj, int32_t block, int32_t kb) {
  if (check_block_args(d, d_proj, block, kb) != SA_OK) return 0;
  BlockPlan p;
  if (!block_plan(p, d, d_proj, block, kb)) return 0;
  return p.total;
}

static int block_common(const void* Q, const void* K, const void* Pq, const void* Pk,
                        const sa_dims& d, int d_proj, int block, int kb, int causal,
                        float score_scale, int dtype, void* ws, size_t ws_bytes,
                        sa_profile* prof, hipStream_t s, BlockPlan& p, float*& q32,
                        float*& k32, float*& kbar, int32_t*& sel) {
  if (!Q || !K || !Pq || !Pk || !ws) return SA_ERR_NULL;
  int st = check_block_args(d, d_proj, block, kb);
  if (st != SA_OK) return st;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (!(score_scale > 0.0f) || !std::isfinite(score_scale)) return SA_ERR_SHAPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(Pq) || !aligned16(Pk) || !aligned16(ws))
    return SA_ERR_ALIGN;
  if (!block_plan(p, d, d_proj, block, kb)) return SA_ERR_UNSUPPORTED;
  if (ws_bytes < p.total) return SA_ERR_WORKSPACE;
  unsigned char* base = static_cast<unsigned char*>(ws);
  q32 = reinterpret_cast<float*>(base + p.off_q32);
  k32 = reinterpret_cast<float*>(base + p.off_k32);
  kbar = reinterpret_cast<float*>(base + p.off_kbar);
  sel = reinterpret_cast<int32_t*>(base + p.off_sel);
  const int BH = d.B * d.H;
  SA_TIMED_STATUS("block_project", launch_project_rows(Q, Pq, BH, d.N, d.N, d.D, d_proj, dtype, 0,
                                                       q32, nullptr, nullptr, s));
  SA_TIMED_STATUS("block_project", launch_project_rows(K, Pk, BH, d.N, d.N, d.D, d_proj, dtype, 1,
                                                       k32, nullptr, nullptr, s));
  (void)causal;
  return SA_OK;
}

int sparse_attn_block_topk(const void* Q, const void* K, const void* Pq, const void* Pk,
                           sa_dims d, int32_t d_proj, int32_t block, int32_t kb, int32_t causal,
                           float score_scale, int32_t dtype, int32_t* idx, void* ws,
                           size_t ws_bytes, const sa_options* opts, void* stream) {
  if (!idx) return SA_ERR_NULL;
  if (!aligned16(idx)) return SA_ERR_ALIGN;
  sa_profile* prof = profile_of(opts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  BlockPlan p;
  float *q32, *k32, *kbar;
  int32_t* sel;
  int st = block_common(Q, K, Pq, Pk, d, d_proj, block, kb, causal, score_scale, dtype, ws,
                        ws_bytes, prof, s, p, q32, k32, kbar, sel);
  if (st != SA_OK) return st;
  const int BH = d.B * d.H;
  SA_TIMED_STATUS("block_select", launch_block_select(q32, k32, BH, d.N, d_proj, block, kb,
                                                      causal ? 1 : 0, score_scale, kbar, sel, s));
  SA_TIMED_STATUS("block_expand", launch_block_expand(sel, BH, d.N, block, kb, causal ? 1 : 0,
                                                      idx, s));
  return SA_OK;
}

int sparse_attn_block_scores_dump(const void* Q, const void* K, const void* Pq, const void* Pk,
                                  sa_dims d, int32_t d_proj, int32_t block, float score_scale,
                                  int32_t dtype, int32_t row_begin, int32_t row_count, float* S,
                                  void* ws, size_t ws_bytes, const sa_options* opts,
                                  void* stream) {
  if (!S) return SA_ERR_NULL;
  if (!aligned16(S)) return SA_ERR_ALIGN;
  if (row_begin < 0 || row_count < 1 || row_begin > d.N - row_count) return SA_ERR_SHAPE;
  sa_profile* prof = profile_of(opts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  BlockPlan p;
  float *q32, *k32, *kbar;
  int32_t* sel;
  int st = block_common(Q, K, Pq, Pk, d, d_proj, block, 1, 0, score_scale, dtype, ws, ws_bytes,
                        prof, s, p, q32, k32, kbar, sel);
  if (st != SA_OK) return st;
  const int BH = d.B * d.H;
  SA_TIMED_STATUS("block_means", launch_block_select(q32, k32, BH, d.N, d_proj, block, 1, 0,
                                                     score_scale, kbar, nullptr, s));
  SA_TIMED_STATUS("block_dump", launch_block_dump(q32, kbar, BH, d.N, p.NB, d_proj, score_scale,
                                                  row_begin, row_count, S, s));
  return SA_OK;
}

// ----------------------------------------------------------- backward ---
namespace {
struct BwdPlan {
  size_t off_dql, off_dkl, off_cnt, off_off, off_cnts, off_ent, off_epd, off_stats, off_seg,
      off_bounds, off_rpart, off_part, total;
  int nchunks, slices, split_rows, split_keys;
};
// Parts of the backward's passes: automatic picks the key-range split for
// heads of at least 2^22 row elements (N >= 32768 at D = 128: 16 MiB of bf16
// K and V rows and more), whose rows outgrow an XCD's L2 (measured, bf16 at
// D = 128: 32 heads of 32K, 38.2 against 38.6 ms whole; 4 x 8 causal heads
// of 64K, 119 against 128 ms); smaller heads run whole.
int bwd_parts_of(const sa_options* opts) { return opts != nullptr ? opts->bwd_parts : 0; }

BwdPlan bwd_plan(const sa_dims& d, int dp, int k, bool scorer, int parts) {
  const size_t BH = static_cast<size_t>(d.B) * d.H, N = static_cast<size_t>(d.N);
  const size_t ents = BH * N * static_cast<size_t>(k);
  BwdPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t lo = scorer ? BH * N * dp * 4 : 0;
  p.off_dql = take(lo);
  p.off_dkl = take(lo);
  p.off_cnt = take(BH * N * 4);
  p.off_off = take(BH * N * 4);
  const bool big = N * static_cast<size_t>(d.D) >= (size_t(1) << 22);
  p.split_rows = parts == SA_BWD_PARTS_SPLIT || (parts == SA_BWD_PARTS_AUTO && big) ? 1 : 0;
  p.slices = bwd_slices(d.N, k);
  // the key pass takes its parts from whole groups of row slices
  if (parts == SA_BWD_PARTS_SPLIT && p.slices % kGatherRanges != 0)
    p.slices = (p.slices + kGatherRanges - 1) / kGatherRanges * kGatherRanges;
  p.split_keys = p.split_rows && p.slices % kGatherRanges == 0 ? 1 : 0;
  p.off_cnts = take(static_cast<size_t>(p.slices) * BH * N * 4);
  p.off_ent = take(ents * sizeof(BwdEntry));
  p.off_epd = take(ents * 8);
  p.off_stats = take(BH * N * 16);
  p.off_seg = take(p.split_rows ? BH * N * (kGatherRanges + 1) * 4 : 0);
  p.off_bounds = take(p.split_rows ? BH * (kGatherRanges + 1) * 4 : 0);
  const size_t rpart = p.split_rows ? BH * N * kGatherRanges * (2 * d.D + 4) * 4 : 0;
  const size_t kpart = p.split_keys ? BH * N * kGatherRanges * (2 * d.D) * 4 : 0;
  p.off_rpart = take(rpart > kpart ? rpart : kpart);
  p.nchunks = scorer ? outer_sum_chunks(static_cast<long long>(BH * N)) : 0;
  p.off_part = take(scorer ? static_cast<size_t>(p.nchunks) * d.D * dp * 4 * 2 : 0);
  p.total = off;
  return p;
}
}  // namespace

size_t sparse_attn_bwd_workspace_size(sa_dims d, int32_t d_proj, int32_t k, int32_t scorer_grad,
                                      const sa_options* opts) {
  if (check_dims(d, k) != SA_OK || !supported_D(d.D)) return 0;
  if (scorer_grad && !supported_dp(d_proj)) return 0;
  const int parts = bwd_parts_of(opts);
  if (parts < SA_BWD_PARTS_AUTO || parts > SA_BWD_PARTS_SPLIT) return 0;
  return bwd_plan(d, d_proj, k, scorer_grad != 0, parts).total;
}

int sparse_attn_bwd(const void* Q, const void* K, const void* V, const void* Pq, const void* Pk,
                    const void* dO, const int32_t* idx, sa_dims d, int32_t d_proj, int32_t k,
                    float score_scale, float softmax_scale, int32_t dtype, float* dQ, float* dK,
                    float* dV, float* dPq, float* dPk, void* ws, size_t ws_bytes,
                    const sa_options* opts, void* stream) {
  if (!Q || !K || !V || !dO || !idx || !dQ || !dK || !dV || !ws) return SA_ERR_NULL;
  const bool scorer = dPq != nullptr || dPk != nullptr;
  if (scorer && (!dPq || !dPk || !Pq || !Pk)) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (!supported_D(d.D)) return SA_ERR_UNSUPPORTED;
  if (scorer && !supported_dp(d_proj)) return SA_ERR_UNSUPPORTED;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale) || (scorer && !std::isfinite(score_scale)))
    return SA_ERR_SHAPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(idx) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(ws))
    return SA_ERR_ALIGN;
  if (scorer && (!aligned16(Pq) || !aligned16(Pk) || !aligned16(dPq) || !aligned16(dPk)))
    return SA_ERR_ALIGN;
  const int parts = bwd_parts_of(opts);
  if (parts < SA_BWD_PARTS_AUTO || parts > SA_BWD_PARTS_SPLIT) return SA_ERR_SHAPE;
  const BwdPlan p = bwd_plan(d, d_proj, k, scorer, parts);
  if (ws_bytes < p.total) return SA_ERR_WORKSPACE;
  unsigned char* base = static_cast<unsigned char*>(ws);
  float* dql = reinterpret_cast<float*>(base + p.off_dql);
  float* dkl = reinterpret_cast<float*>(base + p.off_dkl);
  int* cnt = reinterpret_cast<int*>(base + p.off_cnt);
  int* offs = reinterpret_cast<int*>(base + p.off_off);
  int* cnts = reinterpret_cast<int*>(base + p.off_cnts);
  BwdEntry* rec = reinterpret_cast<BwdEntry*>(base + p.off_ent);
  BwdArgs a{};
  a.dtype = dtype;
  a.D = d.D;
  a.k = k;
  a.N = d.N;
  a.nh = d.B * d.H;
  a.scorer = scorer ? 1 : 0;
  a.scale = softmax_scale;
  a.Q = Q; a.K = K; a.V = V; a.dO = dO; a.idx = idx;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.seg_off = offs; a.seg_cnt = cnt; a.rec = rec;
  a.epd = reinterpret_cast<float2*>(base + p.off_epd);
  a.stats = reinterpret_cast<float4*>(base + p.off_stats);
  a.split_rows = p.split_rows;
  a.split_keys = p.split_keys;
  a.slices = p.slices;
  int* row_seg = reinterpret_cast<int*>(base + p.off_seg);
  int* bounds = reinterpret_cast<int*>(base + p.off_bounds);
  a.row_seg = row_seg;
  a.bounds = bounds;
  a.slice_pre = cnts;
  a.part = reinterpret_cast<float*>(base + p.off_rpart);
  const long long rows = static_cast<long long>(a.nh) * d.N;
  sa_profile* prof = profile_of(opts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SA_TIMED_STATUS("bwd_count", launch_bwd_hist(idx, a.nh, d.N, k, p.slices, cnts, s));
  SA_TIMED_STATUS("bwd_scan", launch_bwd_slice_prefix(cnts, p.slices, rows, cnt, s));
  SA_TIMED_STATUS("bwd_scan", launch_bwd_scan(cnt, a.nh, d.N, offs, s));
  a.pass = 0;
  if (p.split_rows) {
    SA_TIMED_STATUS("bwd_scan", launch_bwd_bounds(offs, cnt, a.nh, d.N, bounds, s));
    SA_TIMED_STATUS("bwd_scan", launch_bwd_row_ranges(idx, bounds, a.nh, d.N, k, row_seg, s));
  }
  SA_TIMED_STATUS("bwd_rows", launch_bwd_pass(a, s));
  if (p.split_rows)
    SA_TIMED_STATUS("bwd_rows_merge", launch_bwd_rows_merge(a.part, a.nh, d.N, d.D,
                                                           scorer ? 1.0f : softmax_scale, dQ,
                                                           a.stats, s));
  if (p.split_rows)
    SA_TIMED_STATUS("bwd_fill", launch_bwd_fill_parts(idx, a.epd, a.stats, row_seg, bounds, a.nh,
                                                      d.N, k, p.slices, cnts, offs, rec, s));
  else
    SA_TIMED_STATUS("bwd_fill", launch_bwd_fill(idx, a.epd, a.stats, a.nh, d.N, k, p.slices, cnts,
                                                offs, rec, s));
  a.pass = 1;
  if (p.split_keys && bwd_keys_two_launches(d.N, d.D)) {
    a.keys_which = 0;
    SA_TIMED_STATUS("bwd_keys_dv", launch_bwd_pass(a, s));
    a.keys_which = 1;
    SA_TIMED_STATUS("bwd_keys_h", launch_bwd_pass(a, s));
  } else {
    a.keys_which = -1;
    SA_TIMED_STATUS("bwd_keys", launch_bwd_pass(a, s));
  }
  if (p.split_keys)
    SA_TIMED_STATUS("bwd_keys_merge", launch_bwd_keys_merge(a.part, a.nh, d.N, d.D,
                                                           scorer ? 1.0f : softmax_scale, dK, dV,
                                                           s));
  if (scorer) {
    // dQ and dK hold G and H (unscaled): the scorer's low-dimensional
    // gradients first, then the full ones
    SA_TIMED_STATUS("bwd_scorer", launch_rows_times_p(dQ, Pk, dtype, rows, d.D, d_proj,
                                                      score_scale, dql, s));
    SA_TIMED_STATUS("bwd_scorer", launch_rows_times_p(dK, Pq, dtype, rows, d.D, d_proj,
                                                      score_scale, dkl, s));
    SA_TIMED_STATUS("bwd_scorer", launch_rows_times_pt(dql, Pq, dtype, rows, d.D, d_proj,
                                                       softmax_scale, dQ, s));
    SA_TIMED_STATUS("bwd_scorer", launch_rows_times_pt(dkl, Pk, dtype, rows, d.D, d_proj,
                                                       softmax_scale, dK, s));
    float* part = reinterpret_cast<float*>(base + p.off_part);
    const size_t psz = static_cast<size_t>(p.nchunks) * d.D * d_proj;
    SA_TIMED_STATUS("bwd_scorer", launch_outer_sum(Q, dtype, dql, rows, d.D, d_proj, part,
                                                   p.nchunks, dPq, s));
    SA_TIMED_STATUS("bwd_scorer", launch_outer_sum(K, dtype, dkl, rows, d.D, d_proj, part + psz,
                                                   p.nchunks, dPk, s));
  }
  return SA_OK;
}

int sparse_attn_dilated_indices(sa_dims d, int32_t window, int32_t dilation, int32_t* idx,
                                int32_t k, const sa_options* opts, void* stream) {
  if (!idx) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (window < 0 || dilation < 1) return SA_ERR_SHAPE;
  if (!aligned16(idx)) return SA_ERR_ALIGN;
  sa_profile* prof = profile_of(opts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SA_TIMED_STATUS("dilated", launch_dilated(d.B * d.H, d.N, window, dilation, idx, k, s));
  return SA_OK;
}

int sparse_attn_band_indices_per_batch(sa_dims d, const int32_t* radii, int32_t* idx,
                                       int32_t k, const sa_options* opts, void* stream) {
  if (!idx || !radii) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (!aligned16(idx)) return SA_ERR_ALIGN;
  sa_profile* prof = profile_of(opts);
  hipStream_t s = static_cast<hipStream_t>(stream);
  SA_TIMED_STATUS("band_batch", launch_band_batch(d.B, d.H, d.N, radii, idx, k, s));
  return SA_OK;
}

int sparse_attn_band_indices(sa_dims d, int32_t w_left, int32_t w_right, int32_t* idx,
                             int32_t k, const sa_options* opts, void* stream) {
  if (!idx) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (w_left < 0 || w_right < 0) return SA_ERR_SHAPE;
  if (!aligned16(idx)) return SA_ERR_ALIGN;
  return timed_band(d.B * d.H, d.N, w_left, w_right, idx, k, profile_of(opts),
                    static_cast<hipStream_t>(stream)) == hipSuccess
             ? SA_OK
             : SA_ERR_HIP;
}

int sparse_attn_scores_dump(const void* Q, const void* K, const void* Pq, const void* Pk,
                            sa_dims d, int32_t d_proj, int32_t causal, float score_scale,
                            int32_t dtype, int32_t row_begin, int32_t row_count, float* S,
                            void* ws, size_t ws_bytes, const sa_options* opts, void* stream) {
  int st = check_scorer_args(Q, K, Pq, Pk, d, d_proj, 1, dtype, score_scale);
  if (st != SA_OK) return st;
  if (!S || !ws) return SA_ERR_NULL;
  if (!aligned16(S) || !aligned16(ws)) return SA_ERR_ALIGN;
  if (row_begin < 0 || row_count < 1 || row_begin > d.N - row_count) return SA_ERR_SHAPE;
  // the dump needs only the projection buffers; size the chunk as for k = 1
  const int hc = chunk_heads_for(d, d_proj, 1, causal, dtype, 0, ws_bytes);
  if (hc < 1) return SA_ERR_WORKSPACE;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, 1, causal, dtype, 0, hc, 0)) return SA_ERR_SHAPE;
  const Bufs b = bufs_of(p, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int h0 = 0; h0 < p.BH; h0 += p.hc) {
    const int nh = p.BH - h0 < p.hc ? p.BH - h0 : p.hc;
    float* Sc = S + static_cast<size_t>(h0) * row_count * d.N;
    if (timed_dump(p, b, Q, K, Pq, Pk, h0, nh, score_scale, row_begin, row_count, Sc, h0 == 0,
                   profile_of(opts), s) != hipSuccess)
      return SA_ERR_HIP;
  }
  return SA_OK;
}

int sparse_attn_check_status(void* stream) {
  int v = 0;
  if (read_and_clear_device_flag(&v, static_cast<hipStream_t>(stream)) != hipSuccess)
    return SA_ERR_HIP;
  return v ? SA_ERR_DEVICE_INDEX : SA_OK;
}

int sparse_attn_workspace_stats(const void* ws, size_t ws_bytes, int64_t* out, int32_t n,
                                void* stream) {
  if (!ws || !out) return SA_ERR_NULL;
  if (ws_bytes < sizeof(WsHeader)) return SA_ERR_WORKSPACE;
  if (n < 0) return SA_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  WsHeader h;
  if (hipMemcpyAsync(&h, ws, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess)
    return SA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return SA_ERR_HIP;
  const int64_t vals[8] = {static_cast<int64_t>(h.fallback_queries),
                           static_cast<int64_t>(h.overflow_queries),
                           static_cast<int64_t>(h.candidates), static_cast<int64_t>(h.rescored),
                           static_cast<int64_t>(h.queries), static_cast<int64_t>(h.retried),
                           static_cast<int64_t>(h.margin_violations),
                           static_cast<int64_t>(h.wide_queries)};
  const int m = n < 8 ? n : 8;
  for (int i = 0; i < m; ++i) out[i] = vals[i];
  return m;
}

const char* sparse_attn_status_string(int status) {
  switch (status) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "a required pointer is NULL";
    case SA_ERR_SHAPE: return "invalid shape, scale or row range";
    case SA_ERR_UNSUPPORTED: return "unsupported head dim, d_proj, dtype or k";
    case SA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case SA_ERR_WORKSPACE: return "workspace too small";
    case SA_ERR_HIP: return "HIP launch or runtime error";
    case SA_ERR_DEVICE_INDEX: return "a gather saw an index >= N";
  }
  return "unknown status";
}

}  // extern "C"
