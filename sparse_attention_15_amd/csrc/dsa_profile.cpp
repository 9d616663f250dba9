// dsa_profile.cpp -- opt-in per-kernel timing.  While recording is on for a thread, every kernel
// the library launches from that thread is bracketed with a pair of hipEvents on the launch
// stream; dsa_profile_stop() waits for them and returns per-kernel totals.  Events come from a
// host-side pool that is reused across sessions; no device memory is involved.  When recording is
// off, a launch pays one thread-local flag test.
#include <string.h>

#include <string>
#include <vector>

#include "dsa.h"
#include "dsa_internal.h"

namespace dsa {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

struct State {
  bool on = false;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<Rec> recs;
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
};

thread_local State g_prof;

}  // namespace

LaunchScope::LaunchScope(const char* name, hipStream_t s) : name_(name), stream_(s), stop_(nullptr) {
  if (!g_prof.on) return;
  hipEvent_t a = g_prof.get(), b = g_prof.get();
  if (a == nullptr || b == nullptr) return;
  hipEventRecord(a, s);
  g_prof.recs.push_back(Rec{name, a, b});
  stop_ = b;
}

LaunchScope::~LaunchScope() {
  if (stop_ != nullptr) hipEventRecord(stop_, stream_);
}

}  // namespace dsa

extern "C" {

dsa_status dsa_profile_start(void) {
  dsa::g_prof.on = true;
  dsa::g_prof.used = 0;
  dsa::g_prof.recs.clear();
  return DSA_OK;
}

int dsa_profile_stop(dsa_kernel_time* out, int max_entries) {
  auto& P = dsa::g_prof;
  P.on = false;
  std::vector<dsa_kernel_time> agg;
  for (const auto& r : P.recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -1;
    dsa_kernel_time* e = nullptr;
    for (auto& x : agg)
      if (strncmp(x.name, r.name, sizeof x.name) == 0) e = &x;
    if (e == nullptr) {
      agg.push_back(dsa_kernel_time{});
      e = &agg.back();
      strncpy(e->name, r.name, sizeof e->name - 1);
    }
    e->launches += 1;
    e->total_ms += ms;
  }
  P.recs.clear();
  P.used = 0;
  const int n = (int)agg.size();
  for (int i = 0; i < n && i < max_entries && out != nullptr; ++i) out[i] = agg[i];
  return n;
}

}  // extern "C"
