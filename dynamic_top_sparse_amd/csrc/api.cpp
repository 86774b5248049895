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

// 16-bit operand type of the MFMA filter (sparse_attn_set_filter_dtype).
std::atomic<int> g_filter_dtype{SA_F16};
constexpr int kDefaultChunkHeads = 8;

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

// Runs `call` between the optional timing events of `name`.
#define SA_TIMED(name, call)          \
  do {                                \
    prof_begin(name, s);              \
    hipError_t e_ = (call);           \
    prof_end(s);                      \
    if (e_ != hipSuccess) return e_;  \
  } while (0)

hipError_t run_topk_chunk(const Plan& p, const Bufs& b, const void* Q, const void* K,
                          const void* Pq, const void* Pk, int h0, int nh, float scale,
                          int32_t* idx_chunk, int first, int* seg, hipStream_t s) {
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
  return hipSuccess;
}

hipError_t timed_gather(const void* Q, const void* K, const void* V, const int32_t* idx, int k,
                        int nheads, int N, int D, float scale, int dtype, void* O,
                        hipStream_t s) {
  SA_TIMED("gather", launch_gather(Q, K, V, idx, k, nheads, N, D, scale, dtype, O, s));
  return hipSuccess;
}

hipError_t timed_dump(const Plan& p, const Bufs& b, const void* Q, const void* K, const void* Pq,
                      const void* Pk, int h0, int nh, float scale, int row_begin, int row_count,
                      float* Sc, int first, hipStream_t s) {
  SA_TIMED("init", launch_init_chunk(p, b, first, s));
  SA_TIMED("project", launch_project(p, b, Q, K, Pq, Pk, h0, nh, s));
  SA_TIMED("dump", launch_dump(p, b, nh, scale, row_begin, row_count, Sc, s));
  return hipSuccess;
}

hipError_t timed_band(int nheads, int N, int w_left, int w_right, int32_t* idx, int k,
                      hipStream_t s) {
  SA_TIMED("band", launch_band(nheads, N, w_left, w_right, idx, k, s));
  return hipSuccess;
}

// Largest chunk (in heads) whose workspace fits ws_bytes; 0 if none.
int chunk_heads_for(const sa_dims& d, int dp, int k, int causal, int dtype, int with_idx,
                    size_t ws_bytes) {
  const int BH = d.B * d.H;
  Plan p1, p2;
  if (!make_plan(p1, d.B, d.H, d.N, d.D, dp, k, causal, dtype, with_idx, 1)) return 0;
  if (BH == 1) return p1.total <= ws_bytes ? 1 : 0;
  if (!make_plan(p2, d.B, d.H, d.N, d.D, dp, k, causal, dtype, with_idx, 2)) return 0;
  if (p1.total > ws_bytes) return 0;
  const size_t per_head = p2.total - p1.total;
  const size_t fixed = p1.total - per_head;
  size_t h = (ws_bytes - fixed) / per_head;
  if (h > static_cast<size_t>(BH)) h = BH;
  // keep head-chunk indices within int range of the queue entries
  while (h > 1) {
    Plan ph;
    if (make_plan(ph, d.B, d.H, d.N, d.D, dp, k, causal, dtype, with_idx, static_cast<int>(h)) &&
        ph.total <= ws_bytes)
      break;
    --h;
  }
  return static_cast<int>(h);
}

}  // namespace

bool make_plan(Plan& p, int B, int H, int N, int D, int dp, int k, int causal, int dtype,
               int with_idx, int heads_per_chunk) {
  p.B = B; p.H = H; p.N = N; p.D = D; p.dp = dp; p.k = k; p.causal = causal ? 1 : 0;
  p.dtype = dtype;
  p.filt = g_filter_dtype.load() == SA_BF16 ? 1 : 0;
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
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, k, causal, dtype, with_idx, heads_per_chunk))
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
                            size_t ws_bytes, void* stream) {
  int st = check_scorer_args(Q, K, Pq, Pk, d, d_proj, k, dtype, score_scale);
  if (st != SA_OK) return st;
  if (!idx || !ws) return SA_ERR_NULL;
  if (!aligned16(idx) || !aligned16(ws)) return SA_ERR_ALIGN;
  const int hc = chunk_heads_for(d, d_proj, k, causal, dtype, 0, ws_bytes);
  if (hc < 1) return SA_ERR_WORKSPACE;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, k, causal, dtype, 0, hc)) return SA_ERR_SHAPE;
  const Bufs b = bufs_of(p, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int h0 = 0; h0 < p.BH; h0 += p.hc) {
    const int nh = p.BH - h0 < p.hc ? p.BH - h0 : p.hc;
    int32_t* idx_chunk = idx + static_cast<size_t>(h0) * d.N * k;
    if (run_topk_chunk(p, b, Q, K, Pq, Pk, h0, nh, score_scale, idx_chunk, h0 == 0, nullptr, s) !=
        hipSuccess)
      return SA_ERR_HIP;
  }
  return SA_OK;
}

int sparse_attn_gather(const void* Q, const void* K, const void* V, const int32_t* idx,
                       int32_t k, sa_dims d, float softmax_scale, int32_t dtype, void* O,
                       void* stream) {
  if (!Q || !K || !V || !idx || !O) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (!supported_D(d.D)) return SA_ERR_UNSUPPORTED;
  if (dtype != SA_F32 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return SA_ERR_SHAPE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(idx) || !aligned16(O))
    return SA_ERR_ALIGN;
  return timed_gather(Q, K, V, idx, k, d.B * d.H, d.N, d.D, softmax_scale, dtype, O,
                      static_cast<hipStream_t>(stream)) == hipSuccess
             ? SA_OK
             : SA_ERR_HIP;
}

int sparse_attn_fwd(const void* Q, const void* K, const void* V, const void* Pq, const void* Pk,
                    sa_dims d, int32_t d_proj, int32_t k, int32_t causal, float score_scale,
                    float softmax_scale, int32_t dtype, void* O, int32_t* idx_or_null, void* ws,
                    size_t ws_bytes, void* stream) {
  int st = check_scorer_args(Q, K, Pq, Pk, d, d_proj, k, dtype, score_scale);
  if (st != SA_OK) return st;
  if (!V || !O || !ws) return SA_ERR_NULL;
  if (!std::isfinite(softmax_scale)) return SA_ERR_SHAPE;
  if (!aligned16(V) || !aligned16(O) || !aligned16(ws)) return SA_ERR_ALIGN;
  if (idx_or_null && !aligned16(idx_or_null)) return SA_ERR_ALIGN;
  const int with_idx = idx_or_null ? 0 : 1;
  const int hc = chunk_heads_for(d, d_proj, k, causal, dtype, with_idx, ws_bytes);
  if (hc < 1) return SA_ERR_WORKSPACE;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, k, causal, dtype, with_idx, hc))
    return SA_ERR_SHAPE;
  const Bufs b = bufs_of(p, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esz = dtype == SA_F32 ? 4 : 2;
  for (int h0 = 0; h0 < p.BH; h0 += p.hc) {
    const int nh = p.BH - h0 < p.hc ? p.BH - h0 : p.hc;
    int32_t* idx_chunk =
        idx_or_null ? idx_or_null + static_cast<size_t>(h0) * d.N * k : b.idx;
    if (run_topk_chunk(p, b, Q, K, Pq, Pk, h0, nh, score_scale, idx_chunk, h0 == 0,
                       p.gsplit ? b.seg : nullptr, s) !=
        hipSuccess)
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
                                b.part, Oc + hh * head, s) != hipSuccess)
          return SA_ERR_HIP;
      }
    } else if (timed_gather(Qc, Kc, Vc, idx_chunk, k, nh, d.N, d.D, softmax_scale, dtype, Oc,
                            s) != hipSuccess) {
      return SA_ERR_HIP;
    }
  }
  return SA_OK;
}

int sparse_attn_band_indices(sa_dims d, int32_t w_left, int32_t w_right, int32_t* idx,
                             int32_t k, void* stream) {
  if (!idx) return SA_ERR_NULL;
  int st = check_dims(d, k);
  if (st != SA_OK) return st;
  if (w_left < 0 || w_right < 0) return SA_ERR_SHAPE;
  if (!aligned16(idx)) return SA_ERR_ALIGN;
  return timed_band(d.B * d.H, d.N, w_left, w_right, idx, k,
                    static_cast<hipStream_t>(stream)) == hipSuccess
             ? SA_OK
             : SA_ERR_HIP;
}

int sparse_attn_scores_dump(const void* Q, const void* K, const void* Pq, const void* Pk,
                            sa_dims d, int32_t d_proj, int32_t causal, float score_scale,
                            int32_t dtype, int32_t row_begin, int32_t row_count, float* S,
                            void* ws, size_t ws_bytes, void* stream) {
  int st = check_scorer_args(Q, K, Pq, Pk, d, d_proj, 1, dtype, score_scale);
  if (st != SA_OK) return st;
  if (!S || !ws) return SA_ERR_NULL;
  if (!aligned16(S) || !aligned16(ws)) return SA_ERR_ALIGN;
  if (row_begin < 0 || row_count < 1 || row_begin > d.N - row_count) return SA_ERR_SHAPE;
  // the dump needs only the projection buffers; size the chunk as for k = 1
  const int hc = chunk_heads_for(d, d_proj, 1, causal, dtype, 0, ws_bytes);
  if (hc < 1) return SA_ERR_WORKSPACE;
  Plan p;
  if (!make_plan(p, d.B, d.H, d.N, d.D, d_proj, 1, causal, dtype, 0, hc)) return SA_ERR_SHAPE;
  const Bufs b = bufs_of(p, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int h0 = 0; h0 < p.BH; h0 += p.hc) {
    const int nh = p.BH - h0 < p.hc ? p.BH - h0 : p.hc;
    float* Sc = S + static_cast<size_t>(h0) * row_count * d.N;
    if (timed_dump(p, b, Q, K, Pq, Pk, h0, nh, score_scale, row_begin, row_count, Sc, h0 == 0,
                   s) != hipSuccess)
      return SA_ERR_HIP;
  }
  return SA_OK;
}

int sparse_attn_set_filter_dtype(int32_t dtype) {
  if (dtype != SA_F16 && dtype != SA_BF16) return SA_ERR_UNSUPPORTED;
  g_filter_dtype.store(dtype);
  return SA_OK;
}

int sparse_attn_get_filter_dtype(void) { return g_filter_dtype.load(); }

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
  const int64_t vals[6] = {static_cast<int64_t>(h.fallback_queries),
                           static_cast<int64_t>(h.overflow_queries),
                           static_cast<int64_t>(h.candidates), static_cast<int64_t>(h.rescored),
                           static_cast<int64_t>(h.queries), static_cast<int64_t>(h.retried)};
  const int m = n < 6 ? n : 6;
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
