// Device facts, launch timing (HIP events) and launch-error reporting.

#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "runtime.h"

namespace pagedkv {

namespace {

std::mutex g_cu_mu;
std::vector<int> g_cu_cache;  // per device id, 0 = unknown

struct TraceStore {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> launches[PAGED_KERNEL_COUNT];
  std::vector<hipEvent_t> spare;

  hipEvent_t get_event() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

TraceStore& trace() {
  static TraceStore* t = new TraceStore();  // never destroyed: events outlive static teardown
  return *t;
}

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(g_cu_mu);
  if (static_cast<int>(g_cu_cache.size()) <= dev) g_cu_cache.resize(dev + 1, 0);
  if (g_cu_cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    g_cu_cache[dev] = cus;
  }
  return g_cu_cache[dev];
}

LaunchTrace::LaunchTrace(int kernel, hipStream_t stream) : kernel_(kernel), stream_(stream) {
  TraceStore& t = trace();
  if (!t.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(t.mu);
  start_ = t.get_event();
  if (start_ && hipEventRecord(start_, stream_) != hipSuccess) {
    t.spare.push_back(start_);
    start_ = nullptr;
  }
}

void LaunchTrace::finish() {
  if (!start_) return;
  TraceStore& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  hipEvent_t end = t.get_event();
  if (!end || hipEventRecord(end, stream_) != hipSuccess) {
    t.spare.push_back(start_);
    if (end) t.spare.push_back(end);
    start_ = nullptr;
    return;
  }
  t.launches[kernel_].emplace_back(start_, end);
  start_ = nullptr;
}

int32_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PAGED_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace pagedkv

using pagedkv::fail;
using pagedkv::ok;

extern "C" int32_t paged_trace_enable(int32_t on) {
  pagedkv::trace().on.store(on != 0);
  return ok();
}

extern "C" int32_t paged_trace_reset(void) {
  auto& t = pagedkv::trace();
  std::lock_guard<std::mutex> lk(t.mu);
  for (auto& v : t.launches) {
    for (auto& pr : v) {
      t.spare.push_back(pr.first);
      t.spare.push_back(pr.second);
    }
    v.clear();
  }
  return ok();
}

extern "C" int32_t paged_trace_query(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= PAGED_KERNEL_COUNT || !total_ms || !launches)
    return fail(PAGED_ERR_INVALID_ARG, "bad argument");
  auto& t = pagedkv::trace();
  std::lock_guard<std::mutex> lk(t.mu);
  double sum = 0.0;
  for (auto& pr : t.launches[kernel]) {
    if (hipEventSynchronize(pr.second) != hipSuccess)
      return fail(PAGED_ERR_HIP, "hipEventSynchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
      return fail(PAGED_ERR_HIP, "hipEventElapsedTime failed");
    sum += ms;
  }
  *total_ms = sum;
  *launches = static_cast<int64_t>(t.launches[kernel].size());
  return ok();
}
