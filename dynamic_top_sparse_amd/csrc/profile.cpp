// Optional per-kernel timing: pairs of HIP events around each launch, kept
// in a record the caller owns (sa_profile).  Nothing here is process-wide:
// each record has its own mutex, and each launch's begin/end pair is matched
// by the slot index prof_begin returns, so calls on other threads that share
// the record cannot end each other's intervals.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "sa_internal.h"
#include "sparse_attn.h"

struct sa_profile {
  struct Rec {
    char name[48];
    hipEvent_t a, b;
    bool ended;
  };
  std::mutex mu;
  std::vector<Rec> open;            // recorded, not yet read
  std::vector<hipEvent_t> spare;    // events ready for reuse

  hipEvent_t take_event() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  ~sa_profile() {
    for (const Rec& r : open) {
      hipEventDestroy(r.a);
      hipEventDestroy(r.b);
    }
    for (hipEvent_t e : spare) hipEventDestroy(e);
  }
};

namespace sa {

int prof_begin(sa_profile* p, const char* name, hipStream_t s) {
  if (p == nullptr) return -1;
  std::lock_guard<std::mutex> lk(p->mu);
  sa_profile::Rec r;
  std::strncpy(r.name, name, sizeof(r.name) - 1);
  r.name[sizeof(r.name) - 1] = 0;
  r.a = p->take_event();
  r.b = p->take_event();
  r.ended = false;
  if (!r.a || !r.b) {
    if (r.a) p->spare.push_back(r.a);
    if (r.b) p->spare.push_back(r.b);
    return -1;
  }
  if (hipEventRecord(r.a, s) != hipSuccess) {
    p->spare.push_back(r.a);
    p->spare.push_back(r.b);
    return -1;
  }
  p->open.push_back(r);
  return static_cast<int>(p->open.size()) - 1;
}

void prof_end(sa_profile* p, int token, hipStream_t s) {
  if (p == nullptr || token < 0) return;
  std::lock_guard<std::mutex> lk(p->mu);
  if (token >= static_cast<int>(p->open.size())) return;
  sa_profile::Rec& r = p->open[static_cast<size_t>(token)];
  if (hipEventRecord(r.b, s) == hipSuccess) r.ended = true;
}

}  // namespace sa

extern "C" sa_profile* sparse_attn_profile_create(void) {
  return new (std::nothrow) sa_profile();
}

extern "C" void sparse_attn_profile_destroy(sa_profile* prof) { delete prof; }

extern "C" int sparse_attn_profile_read(sa_profile* prof, sa_kernel_time* out, int32_t n) {
  if (prof == nullptr) return SA_ERR_NULL;
  if (!out && n > 0) return SA_ERR_NULL;
  std::lock_guard<std::mutex> lk(prof->mu);
  int m = 0;
  int status = SA_OK;
  for (const sa_profile::Rec& r : prof->open) {
    if (status == SA_OK && r.ended) {
      if (hipEventSynchronize(r.b) != hipSuccess) {
        status = SA_ERR_HIP;
      } else if (m < n) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
          status = SA_ERR_HIP;
        } else {
          std::memcpy(out[m].name, r.name, sizeof(out[m].name));
          out[m].ms = ms;
          ++m;
        }
      }
    }
    prof->spare.push_back(r.a);
    prof->spare.push_back(r.b);
  }
  prof->open.clear();
  return status == SA_OK ? m : status;
}
