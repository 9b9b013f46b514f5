// Host runtime: status strings, thread-local error detail, per-kernel event timing
// and the bandwidth probes of spec_measure.h.
#include "host_runtime.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "device_common.h"
#include "spec_measure.h"

namespace specv {

static thread_local char g_last_error[512] = "";

spec_status_t fail(spec_status_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

// ---------------------------------------------------------------- knobs

namespace {

constexpr int kKnobs = 4;
constexpr int kKnobDefault[kKnobs] = {0, kPollLimit, 0, 1};
std::atomic<int> g_knobs[kKnobs] = {{kKnobDefault[0]}, {kKnobDefault[1]}, {kKnobDefault[2]}, {kKnobDefault[3]}};

}  // namespace

int knob(spec_knob_t k) {
  const int i = static_cast<int>(k);
  return i >= 0 && i < kKnobs ? g_knobs[i].load(std::memory_order_relaxed) : 0;
}

int choose_nv(long long rows, int V, int elems_per_vec, long long min_groups) {
  const int forced = knob(SPEC_KNOB_CHUNK_VECTORS);
  if (forced == 1 || forced == 2 || forced == 4 || forced == 8) return forced;
  for (int nv = 8; nv >= 1; nv >>= 1) {
    const long long chunk = static_cast<long long>(nv) * kThreads * elems_per_vec;
    const long long C = (V + chunk - 1) / chunk;
    if (rows * C >= min_groups) return nv;
  }
  return 1;
}

// ---------------------------------------------------------------- timing registry

namespace {

struct TimedRecord {
  const char* name;
  hipEvent_t start;
  hipEvent_t stop;
};

struct Aggregate {
  const char* name;
  long long launches;
  double total_ms;
};

struct TimingState {
  std::mutex mu;
  bool enabled = false;
  std::vector<TimedRecord> records;
  std::vector<hipEvent_t> pool;
  std::vector<Aggregate> aggregate;
};

TimingState& timing() {
  static TimingState* s = new TimingState();  // never destroyed: safe at process exit
  return *s;
}

hipEvent_t take_event(TimingState& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

LaunchScope::LaunchScope(const char* name, hipStream_t)
    : name_(name), start_(nullptr), stop_(nullptr), finished_(false) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  if (!t.enabled) return;
  TimedRecord r{name, take_event(t), take_event(t)};
  if (!r.start || !r.stop) return;
  t.records.push_back(r);
  start_ = r.start;
  stop_ = r.stop;
}

spec_status_t LaunchScope::finish() {
  finished_ = true;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "launch of %s failed: %s", name_, hipGetErrorString(e));
  return SPEC_OK;
}

LaunchScope::~LaunchScope() {
  if (!finished_) finish();
}

// ---------------------------------------------------------------- small kernels

// Pure read in the streaming passes' access shape: one workgroup per chunk of NV * 4 KiB,
// chunks in XCD-blocked order, each wave one contiguous quarter of its chunk, every
// non-temporal 16-byte load issued before any is used.  The words are folded with XOR and
// a never-true test on the result keeps the loads alive.
template <int NV>
__global__ __launch_bounds__(kThreads) void probe_read_kernel(const u32x4* src, uint32_t* out) {
  const int g = xcd_blocked_index();
  const u32x4* p = src + static_cast<size_t>(g) * NV * kThreads + (threadIdx.x >> 6) * NV * 64 + (threadIdx.x & 63);
  u32x4 v[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) v[j] = __builtin_nontemporal_load(p + j * 64);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < NV; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  if (wave_max_int(static_cast<int>(acc & 0x7fffffff)) == -1 && threadIdx.x == 0) *out = 1u;
}

__global__ __launch_bounds__(kThreads) void probe_copy_kernel(const u32x4* src, u32x4* dst, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

static int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  return cus;
}

}  // namespace specv

using namespace specv;

extern "C" {

const char* spec_status_string(spec_status_t status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARG: return "SPEC_ERR_INVALID_ARG";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP";
  }
  return "SPEC_ERR_UNKNOWN";
}

const char* spec_last_error(void) { return g_last_error; }

spec_status_t spec_set_knob(spec_knob_t k, int value) {
  const int i = static_cast<int>(k);
  if (i < 0 || i >= kKnobs) return fail(SPEC_ERR_INVALID_ARG, "unknown knob %d", i);
  if (value < 0) value = kKnobDefault[i];
  const bool ok = k == SPEC_KNOB_CHUNK_VECTORS
                      ? (value == 0 || value == 1 || value == 2 || value == 4 || value == 8 || value == 16)
                      : ((k != SPEC_KNOB_SINGLE_LAUNCH && k != SPEC_KNOB_XCD_LOCAL) || value == 0 || value == 1);
  if (!ok) return fail(SPEC_ERR_INVALID_ARG, "value %d is not allowed for knob %d", value, i);
  g_knobs[i].store(value, std::memory_order_relaxed);
  return SPEC_OK;
}

int spec_get_knob(spec_knob_t k) {
  const int i = static_cast<int>(k);
  return i >= 0 && i < kKnobs ? g_knobs[i].load(std::memory_order_relaxed) : -1;
}

spec_status_t spec_timing_enable(int enable) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  t.enabled = enable != 0;
  return SPEC_OK;
}

spec_status_t spec_timing_reset(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  for (auto& r : t.records) {
    hipEventSynchronize(r.stop);
    t.pool.push_back(r.start);
    t.pool.push_back(r.stop);
  }
  t.records.clear();
  t.aggregate.clear();
  return SPEC_OK;
}

int spec_timing_collect(void) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  for (auto& r : t.records) {
    float ms = 0.f;
    hipEventSynchronize(r.stop);
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) ms = 0.f;
    bool found = false;
    for (auto& a : t.aggregate) {
      if (strcmp(a.name, r.name) == 0) {
        a.launches += 1;
        a.total_ms += ms;
        found = true;
        break;
      }
    }
    if (!found) t.aggregate.push_back(Aggregate{r.name, 1, ms});
    t.pool.push_back(r.start);
    t.pool.push_back(r.stop);
  }
  t.records.clear();
  return static_cast<int>(t.aggregate.size());
}

spec_status_t spec_timing_entry(int index, const char** name, long long* launches, double* total_ms) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  if (index < 0 || index >= static_cast<int>(t.aggregate.size()))
    return fail(SPEC_ERR_INVALID_ARG, "timing entry %d out of range", index);
  if (name) *name = t.aggregate[index].name;
  if (launches) *launches = t.aggregate[index].launches;
  if (total_ms) *total_ms = t.aggregate[index].total_ms;
  return SPEC_OK;
}

spec_status_t spec_probe_read(const void* src, size_t bytes, size_t chunk_bytes, uint32_t* out,
                              spec_stream_t stream) {
  if (chunk_bytes != 16384 && chunk_bytes != 32768 && chunk_bytes != 65536)
    return fail(SPEC_ERR_INVALID_ARG, "probe_read chunk must be 16, 32 or 64 KiB");
  if (!src || !out || bytes == 0 || bytes % chunk_bytes || !aligned16(src))
    return fail(SPEC_ERR_INVALID_ARG, "probe_read needs a 16-byte aligned source of whole chunks");
  if (bytes / chunk_bytes > 2147483647u) return fail(SPEC_ERR_UNSUPPORTED, "probe_read grid too large");
  const dim3 grid(static_cast<unsigned>(bytes / chunk_bytes));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(src);
  LaunchScope scope("probe_read", s);
  if (chunk_bytes == 16384) scope.launch(probe_read_kernel<4>, grid, dim3(kThreads), s, p, out);
  else if (chunk_bytes == 32768) scope.launch(probe_read_kernel<8>, grid, dim3(kThreads), s, p, out);
  else scope.launch(probe_read_kernel<16>, grid, dim3(kThreads), s, p, out);
  return scope.finish();
}

spec_status_t spec_probe_copy(const void* src, void* dst, size_t bytes, spec_stream_t stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 || !aligned16(src) || !aligned16(dst))
    return fail(SPEC_ERR_INVALID_ARG, "probe_copy needs 16-byte aligned buffers and size");
  const unsigned grid = static_cast<unsigned>(device_cu_count() * 8);
  LaunchScope scope("probe_copy", static_cast<hipStream_t>(stream));
  scope.launch(probe_copy_kernel, dim3(grid), dim3(kThreads), static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return scope.finish();
}

}  // extern "C"
