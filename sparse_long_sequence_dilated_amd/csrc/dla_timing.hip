// Opt-in per-launch timing of libdla kernels (a profiling aid).
//
// When enabled, each kernel launch made by the library is bracketed by two
// HIP events recorded on the launch's own stream.  dla_timing_collect() waits
// for the recorded events of one kernel family, returns the launch count and
// summed duration, and hands those events back to a pool, so that a timed
// launch costs two hipEventRecord calls and no event creation once the pool
// has grown to the number of launches in flight.  This process-wide record
// (guarded by a mutex, host memory only) is the one piece of global state
// the library keeps; nothing is recorded while timing is off.
#include <string.h>

#include <mutex>
#include <vector>

#include "dla_kernels.h"

namespace dla {

namespace {
struct Rec {
  const char* name;
  hipEvent_t start, stop;
};
std::mutex g_mu;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_free;   // created events ready for reuse
bool g_on = false;

// An event from the pool (or a new one); false if none could be made.
bool take_event(hipEvent_t& e) {
  if (!g_free.empty()) {
    e = g_free.back();
    g_free.pop_back();
    return true;
  }
  return hipEventCreate(&e) == hipSuccess;
}
}  // namespace

TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : name_(name), stream_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  if (!take_event(start_)) return;
  if (!take_event(stop_)) {
    g_free.push_back(start_);
    return;
  }
  if (hipEventRecord(start_, stream_) != hipSuccess) {
    g_free.push_back(start_);
    g_free.push_back(stop_);
    return;
  }
  active_ = true;
}

TimedLaunch::~TimedLaunch() {
  if (!active_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(stop_, stream_) == hipSuccess) {
    g_recs.push_back(Rec{name_, start_, stop_});
  } else {
    // start_ was recorded: wait for it before the event is reused
    (void)hipEventSynchronize(start_);
    g_free.push_back(start_);
    g_free.push_back(stop_);
  }
}

}  // namespace dla

using namespace dla;

extern "C" int dla_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
  return DLA_OK;
}

extern "C" int dla_timing_collect(const char* name, int64_t* launches, double* total_ms) {
  clear_error();
  if (!name || !launches || !total_ms) return fail(DLA_E_INVALID, "null argument");
  std::lock_guard<std::mutex> lk(g_mu);
  int64_t count = 0;
  double sum = 0.0;
  int rc = DLA_OK;
  std::vector<Rec> keep;
  for (const Rec& r : g_recs) {
    if (strcmp(r.name, name) != 0) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess && rc == DLA_OK)
      rc = fail(DLA_E_HIP, "timing event: %s", hipGetErrorString(e));
    g_free.push_back(r.start);
    g_free.push_back(r.stop);
    ++count;
    sum += ms;
  }
  g_recs.swap(keep);
  *launches = count;
  *total_ms = sum;
  return rc;
}
