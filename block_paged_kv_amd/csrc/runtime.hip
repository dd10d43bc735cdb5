// Device facts, launch timing (HIP events) and launch-error reporting.

#include <algorithm>
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

LaunchTrace::LaunchTrace(int kernel, hipStream_t stream) : kernel_(kernel) {
  TraceStore& t = trace();
  if (!t.on.load(std::memory_order_relaxed)) return;
  // Events inside a captured graph cannot be timed: record nothing there.
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  std::lock_guard<std::mutex> lk(t.mu);
  start_ = t.get_event();
  stop_ = t.get_event();
  if (!start_ || !stop_) {
    if (start_) t.spare.push_back(start_);
    if (stop_) t.spare.push_back(stop_);
    start_ = stop_ = nullptr;
  }
}

void LaunchTrace::finish() {
  if (!start_) return;
  TraceStore& t = trace();
  std::lock_guard<std::mutex> lk(t.mu);
  t.launches[kernel_].emplace_back(start_, stop_);
  start_ = stop_ = nullptr;
}

namespace {

struct DeviceSide {
  std::mutex mu;
  hipStream_t stream = nullptr;
  hipEvent_t fork_ev = nullptr;
  hipEvent_t join_ev = nullptr;
};

std::mutex g_side_mu;
std::vector<DeviceSide*> g_side;  // per device id; never destroyed (the stream outlives static teardown)

DeviceSide* side_state() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lk(g_side_mu);
  if (static_cast<int>(g_side.size()) <= dev) g_side.resize(dev + 1, nullptr);
  if (!g_side[dev]) {
    auto* d = new DeviceSide();
    if (hipStreamCreateWithFlags(&d->stream, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&d->fork_ev, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&d->join_ev, hipEventDisableTiming) != hipSuccess) {
      delete d;  // partially created handles are left to the process end
      return nullptr;
    }
    g_side[dev] = d;
  }
  return g_side[dev];
}

}  // namespace

SideStream::SideStream(hipStream_t s) : s_(s) {
  DeviceSide* d = side_state();
  if (!d) {
    status_ = fail(PAGED_ERR_HIP, "cannot create the side stream");
    return;
  }
  d->mu.lock();
  dev_ = d;
  locked_ = true;
  if (hipEventRecord(d->fork_ev, s) != hipSuccess || hipStreamWaitEvent(d->stream, d->fork_ev, 0) != hipSuccess) {
    status_ = fail(PAGED_ERR_HIP, "cannot order the side stream after the caller's stream");
    d->mu.unlock();
    locked_ = false;
    return;
  }
  status_ = PAGED_OK;
}

hipStream_t SideStream::get() const { return static_cast<DeviceSide*>(dev_)->stream; }

int32_t SideStream::join() {
  if (!locked_) return PAGED_OK;
  auto* d = static_cast<DeviceSide*>(dev_);
  int32_t rc = PAGED_OK;
  if (hipEventRecord(d->join_ev, d->stream) != hipSuccess || hipStreamWaitEvent(s_, d->join_ev, 0) != hipSuccess)
    rc = fail(PAGED_ERR_HIP, "cannot order the caller's stream after the side stream");
  d->mu.unlock();
  locked_ = false;
  return rc;
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

extern "C" int32_t paged_trace_durations(int32_t kernel, double* ms, int64_t capacity,
                                         int64_t* launches) {
  if (kernel < 0 || kernel >= PAGED_KERNEL_COUNT || !launches || capacity < 0 || (capacity > 0 && !ms))
    return fail(PAGED_ERR_INVALID_ARG, "bad argument");
  auto& t = pagedkv::trace();
  std::lock_guard<std::mutex> lk(t.mu);
  const auto& v = t.launches[kernel];
  *launches = static_cast<int64_t>(v.size());
  const int64_t n = std::min<int64_t>(capacity, static_cast<int64_t>(v.size()));
  for (int64_t i = 0; i < n; ++i) {
    if (hipEventSynchronize(v[i].second) != hipSuccess)
      return fail(PAGED_ERR_HIP, "hipEventSynchronize failed");
    float f = 0.f;
    if (hipEventElapsedTime(&f, v[i].first, v[i].second) != hipSuccess)
      return fail(PAGED_ERR_HIP, "hipEventElapsedTime failed");
    ms[i] = f;
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
