// Opt-in launch timing: when enabled, every kernel launch the library makes is
// bracketed by a pair of hipEvents recorded on the launch stream, so a caller
// can read back per-kernel launch counts and summed GPU durations.  Disabled
// (the default) it costs one relaxed atomic load per launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <set>
#include <utility>
#include <string>
#include <vector>

#include "launch.hpp"

namespace csa {
namespace {

struct Rec {
  std::string name;
  hipEvent_t beg, end;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_free;

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

std::mutex g_lds_mu;
std::set<std::pair<int, const void*>> g_lds_done;

}  // namespace

hipError_t ensure_lds_limit(const void* kfn, size_t lds) {
  if (lds <= 65536) return hipSuccess;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_lds_mu);
  const auto key = std::make_pair(dev, kfn);
  if (g_lds_done.count(key)) return hipSuccess;
  e = hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) g_lds_done.insert(key);
  return e;
}

ProfScope::ProfScope(const char* name, hipStream_t st) : st_(st), idx_(-1) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  Rec r{name, take_event(), take_event()};
  if (!r.beg || !r.end) return;
  if (hipEventRecord(r.beg, st) != hipSuccess) return;
  g_recs.push_back(r);
  idx_ = (long)g_recs.size() - 1;
}

ProfScope::~ProfScope() {
  if (idx_ < 0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (idx_ < (long)g_recs.size()) (void)hipEventRecord(g_recs[idx_].end, st_);
}

}  // namespace csa

extern "C" {

void csa_profile_enable(int on) { csa::g_on.store(on ? 1 : 0); }

void csa_profile_reset(void) {
  std::lock_guard<std::mutex> lk(csa::g_mu);
  for (auto& r : csa::g_recs) {
    csa::g_free.push_back(r.beg);
    csa::g_free.push_back(r.end);
  }
  csa::g_recs.clear();
}

int csa_profile_query(const char* kernel, int* count, double* total_ms) {
  std::lock_guard<std::mutex> lk(csa::g_mu);
  int n = 0;
  double ms = 0.0;
  for (auto& r : csa::g_recs) {
    if (std::strcmp(r.name.c_str(), kernel) != 0) continue;
    if (hipEventSynchronize(r.end) != hipSuccess) return -1;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.beg, r.end) != hipSuccess) return -1;
    ms += t;
    ++n;
  }
  if (count) *count = n;
  if (total_ms) *total_ms = ms;
  return n > 0 ? 0 : 1;
}

int csa_profile_counter(const char* name, unsigned long long* value, int reset) {
  int which = -1;
  if (name == nullptr) return 1;
  if (std::strcmp(name, "indexer_prefill_fallback") == 0) which = csa::CNT_PREFILL_FALLBACK;
  else if (std::strcmp(name, "indexer_decode_fallback") == 0) which = csa::CNT_DECODE_FALLBACK;
  else if (std::strcmp(name, "step_timeout") == 0) which = csa::CNT_STEP_TIMEOUT;
  else if (std::strcmp(name, "indexer_decode_second_round") == 0) which = csa::CNT_DECODE_SECOND_ROUND;
  if (which < 0 || value == nullptr) return 1;
  return csa::counter_read(which, value, reset != 0) == hipSuccess ? 0 : -1;
}

}  // extern "C"
