// Optional per-kernel-class timing with HIP events on the launch stream.
#include <mutex>
#include <vector>

#include "host.hpp"

namespace mo {

namespace {
struct Record {
  int cls;
  hipEvent_t a, b;
};
std::mutex g_mu;
bool g_on = false;
std::vector<Record> g_recs;
thread_local int g_quiet = 0;   // KTimerOff scopes on this thread

void clear_locked() {
  for (Record& r : g_recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
}
}  // namespace

KTimerOff::KTimerOff() { ++g_quiet; }
KTimerOff::~KTimerOff() { --g_quiet; }

KTimer::KTimer(int cls, hipStream_t st) : cls_(cls), st_(st) {
  if (g_quiet) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  if (hipEventCreate(&a_) != hipSuccess) return;
  if (hipEventCreate(&b_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    return;
  }
  if (hipEventRecord(a_, st_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    (void)hipEventDestroy(b_);
    return;
  }
  active_ = true;
}

KTimer::~KTimer() {
  if (!active_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  (void)hipEventRecord(b_, st_);
  g_recs.push_back({cls_, a_, b_});
}

bool timing_enabled() {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_on;
}

}  // namespace mo

extern "C" {

mo_status mo_timing_enable(int32_t on) {
  mo::clear_error();
  std::lock_guard<std::mutex> lk(mo::g_mu);
  mo::clear_locked();
  mo::g_on = on != 0;
  return MO_OK;
}

mo_status mo_timing_read(int32_t kclass, double* total_ms, int64_t* launches) {
  mo::clear_error();
  if (kclass < 0 || kclass >= MO_KC_COUNT || !total_ms || !launches)
    return mo::fail(MO_EINVAL, "bad arguments");
  std::lock_guard<std::mutex> lk(mo::g_mu);
  double t = 0.0;
  int64_t n = 0;
  for (const auto& r : mo::g_recs) {
    if (r.cls != kclass) continue;
    MO_HIP_TRY(hipEventSynchronize(r.b));
    float ms = 0.f;
    MO_HIP_TRY(hipEventElapsedTime(&ms, r.a, r.b));
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return MO_OK;
}

}  // extern "C"
