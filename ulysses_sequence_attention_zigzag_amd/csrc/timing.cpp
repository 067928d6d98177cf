// Kernel timing: when enabled, every launcher brackets its launch with a pair
// of hipEvents recorded on the launch stream; reading sums the elapsed times
// per kernel class.  Disabled (the default) it costs one branch per launch.

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "usp_internal.h"

namespace usp {
namespace {

struct Rec {
  int cls;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_enabled = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

TimingScope::TimingScope(int cls, hipStream_t stream) : cls_(cls), stream_(stream) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_enabled) return;
  start_ = take_event();
  stop_ = take_event();
  if (start_ && stop_ && hipEventRecord(static_cast<hipEvent_t>(start_), stream_) == hipSuccess) {
    active_ = true;
  }
}

TimingScope::~TimingScope() {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!active_) {
    if (start_) g_pool.push_back(static_cast<hipEvent_t>(start_));
    if (stop_) g_pool.push_back(static_cast<hipEvent_t>(stop_));
    return;
  }
  if (hipEventRecord(static_cast<hipEvent_t>(stop_), stream_) == hipSuccess)
    g_recs.push_back({cls_, static_cast<hipEvent_t>(start_), static_cast<hipEvent_t>(stop_)});
}

}  // namespace usp

using namespace usp;

extern "C" {

usp_status usp_timing_enable(int enable) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_enabled = enable != 0;
  return USP_OK;
}

usp_status usp_timing_reset(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  for (auto& r : g_recs) {
    (void)hipEventSynchronize(r.stop);
    g_pool.push_back(r.start);
    g_pool.push_back(r.stop);
  }
  g_recs.clear();
  return USP_OK;
}

usp_status usp_timing_read(int kernel_class, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) {
    set_error("null output pointer");
    return USP_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  double t = 0.0;
  int64_t n = 0;
  for (auto& r : g_recs) {
    if (r.cls != kernel_class) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) {
      set_error("event timing failed: %s", hipGetErrorString(e));
      return USP_ERR_HIP;
    }
    t += ms;
    ++n;
  }
  *total_ms = t;
  *launches = n;
  return USP_OK;
}

}  // extern "C"
