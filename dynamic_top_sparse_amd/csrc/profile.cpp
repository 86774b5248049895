// Optional per-kernel timing: pairs of HIP events around each launch.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <vector>

#include "sa_internal.h"
#include "sparse_attn.h"

namespace sa {

namespace {

struct Rec {
  char name[48];
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_open;             // recorded, not yet read
std::vector<hipEvent_t> g_free;      // events ready for reuse

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

void prof_begin(const char* name, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  Rec r;
  std::strncpy(r.name, name, sizeof(r.name) - 1);
  r.name[sizeof(r.name) - 1] = 0;
  r.a = take_event();
  r.b = take_event();
  if (!r.a || !r.b) return;
  hipEventRecord(r.a, s);
  g_open.push_back(r);
}

void prof_end(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on || g_open.empty()) return;
  hipEventRecord(g_open.back().b, s);
}

}  // namespace sa

using namespace sa;

extern "C" int sparse_attn_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return SA_OK;
}

extern "C" int sparse_attn_profile_read(sa_kernel_time* out, int32_t n) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!out && n > 0) return SA_ERR_NULL;
  int m = 0;
  for (const Rec& r : g_open) {
    if (hipEventSynchronize(r.b) != hipSuccess) return SA_ERR_HIP;
    if (m < n) {
      float ms = 0.0f;
      if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return SA_ERR_HIP;
      std::memcpy(out[m].name, r.name, sizeof(out[m].name));
      out[m].ms = ms;
      ++m;
    }
    g_free.push_back(r.a);
    g_free.push_back(r.b);
  }
  g_open.clear();
  return m;
}
