// Host-side runtime shared by the launchers: device facts, launch timing and
// argument checks.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"
#include "status.h"

namespace pagedkv {

// Compute units of the current device (cached per device); 0 on failure.
int device_cu_count();

// Timing events for one launch when tracing is on: pass start()/stop() to
// hipExtLaunchKernelGGL, which stamps them at the kernel's own start and end
// (host launch overhead is not included), then call finish().
class LaunchTrace {
 public:
  LaunchTrace(int kernel, hipStream_t stream);
  hipEvent_t start() const { return start_; }
  hipEvent_t stop() const { return stop_; }
  void finish();  // keep the pair for paged_trace_query (call right after the launch)
 private:
  int kernel_;
  hipEvent_t start_ = nullptr;
  hipEvent_t stop_ = nullptr;
};

// A second queue per device, for the part of one call that may run beside
// the part on the caller's stream. Construction makes the side stream wait
// for everything already enqueued on `s` (an event recorded on `s`); join()
// makes `s` wait for everything enqueued on the side stream since (the
// destructor joins too). The device's lock is held from construction to
// join, so calls from several host threads do not interleave their event
// records. The stream and its two events are created on the first use on a
// device (outside graph capture) and kept until the process ends; the stream
// has the default priority.
class SideStream {
 public:
  explicit SideStream(hipStream_t s);
  ~SideStream() { join(); }
  SideStream(const SideStream&) = delete;
  SideStream& operator=(const SideStream&) = delete;
  int32_t status() const { return status_; }  // PAGED_OK once forked
  hipStream_t get() const;
  int32_t join();

 private:
  hipStream_t s_;
  void* dev_ = nullptr;  // per-device state (runtime.hip)
  bool locked_ = false;
  int32_t status_ = PAGED_ERR_HIP;
};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int esize_of(int32_t dtype) {
  return dtype == PAGED_BF16 ? 2 : dtype == PAGED_F32 ? 4 : dtype == PAGED_FP8_E4M3 ? 1 : 0;
}

inline bool pow2_in(int32_t x, int32_t lo, int32_t hi) {
  return x >= lo && x <= hi && (x & (x - 1)) == 0;
}

inline int ilog2(int32_t x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Report a launch error (if any) as PAGED_ERR_HIP.
int32_t check_launch(const char* what);

}  // namespace pagedkv
