// Host-side runtime shared by the entry points: error reporting, launch checks,
// optional per-kernel event timing, workspace carving and tuning knobs.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "spec_measure.h"
#include "spec_verify.h"

namespace specv {

// Record a thread-local detail message and return `status`.
spec_status_t fail(spec_status_t status, const char* fmt, ...);

// One kernel launch under `name`.  When timing is enabled, start() and stop() are a HIP
// event pair for hipExtLaunchKernelGGL, which stamps them at the kernel's own dispatch
// and completion on `stream` (otherwise both are null and nothing is recorded); on
// destruction the launch is checked.
class LaunchScope {
 public:
  LaunchScope(const char* name, hipStream_t stream);
  ~LaunchScope();
  hipEvent_t start() const { return start_; }
  hipEvent_t stop() const { return stop_; }
  // Launches `kernel` on `stream`: with the timing events when timing is on, else as a
  // plain launch (which stream capture records like any other).
  template <typename F, typename... Args>
  void launch(F kernel, dim3 grid, dim3 block, hipStream_t stream, Args... args) {
    if (start_ && stop_) {
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start_, stop_, 0, args...);
    } else {
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
    }
  }
  // Status of the launch (checks hipGetLastError); call after the kernel launch.
  spec_status_t finish();

 private:
  const char* name_;
  hipEvent_t start_;
  hipEvent_t stop_;
  bool finished_;
};

constexpr int kMaxDevices = 64;  // per-device caches in the host code

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Current value of a knob of spec_measure.h (its default unless a caller set it).
int knob(spec_knob_t k);

// Vectors (16 B each) per lane in one chunk: the largest of 8, 4, 2, 1 that still
// gives at least `min_groups` workgroups over `rows` rows of V elements, else 1.
// SPEC_KNOB_CHUNK_VECTORS forces 1, 2, 4 or 8.
int choose_nv(long long rows, int V, int elems_per_vec, long long min_groups);

}  // namespace specv
