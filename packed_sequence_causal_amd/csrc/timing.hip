// Optional kernel timing: when switched on, each main kernel launch is
// bracketed by two HIP events recorded on the launch stream; reading the
// totals waits for those events.  Off by default; costs nothing when off.
#include <mutex>
#include <vector>

#include "../../include/psc.h"
#include "psc_internal.h"

namespace psc {
namespace {

struct Record {
  int slot;
  hipEvent_t start, stop;
};

struct Timer {
  std::mutex mu;
  bool on = false;
  uint32_t mask = ~0u;  // kernels timed while on (bit k = psc_kernel k)
  std::vector<Record> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[kTimerSlots] = {};
  int64_t launches[kTimerSlots] = {};
};

Timer& timer() {
  static Timer t;
  return t;
}

hipEvent_t take_event(Timer& t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Folds finished records into the totals.  Caller holds the mutex.
int drain(Timer& t) {
  int st = PSC_OK;
  for (Record& r : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) {
      st = PSC_ERR_HIP;
    } else {
      t.total_ms[r.slot] += ms;
      t.launches[r.slot] += 1;
    }
    t.pool.push_back(r.start);
    t.pool.push_back(r.stop);
  }
  t.pending.clear();
  return st;
}

}  // namespace

ScopedKernelTimer::ScopedKernelTimer(int slot, hipStream_t stream) : slot_(slot), stream_(stream) {
  Timer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on || slot < 0 || slot >= 32 || !((t.mask >> slot) & 1u)) return;
  start_ = take_event(t);
  if (start_ && hipEventRecord(static_cast<hipEvent_t>(start_), stream) != hipSuccess) start_ = nullptr;
}

ScopedKernelTimer::~ScopedKernelTimer() {
  if (!start_) return;
  Timer& t = timer();
  std::lock_guard<std::mutex> g(t.mu);
  hipEvent_t stop = take_event(t);
  if (!stop || hipEventRecord(stop, stream_) != hipSuccess) return;
  t.pending.push_back({slot_, static_cast<hipEvent_t>(start_), stop});
}

}  // namespace psc

extern "C" {

int psc_timing_enable(int enable) {
  psc::Timer& t = psc::timer();
  std::lock_guard<std::mutex> g(t.mu);
  t.on = enable != 0;
  return PSC_OK;
}

int psc_timing_select(uint32_t kernel_mask) {
  psc::Timer& t = psc::timer();
  std::lock_guard<std::mutex> g(t.mu);
  t.mask = kernel_mask;
  return PSC_OK;
}

int psc_timing_reset(void) {
  psc::Timer& t = psc::timer();
  std::lock_guard<std::mutex> g(t.mu);
  int st = psc::drain(t);
  for (int i = 0; i < psc::kTimerSlots; ++i) {
    t.total_ms[i] = 0.0;
    t.launches[i] = 0;
  }
  return st;
}

int psc_timing_read(int kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= psc::kTimerSlots || !total_ms || !launches) return PSC_ERR_INVALID;
  psc::Timer& t = psc::timer();
  std::lock_guard<std::mutex> g(t.mu);
  int st = psc::drain(t);
  *total_ms = t.total_ms[kernel];
  *launches = t.launches[kernel];
  return st;
}

const char* psc_kernel_name(int kernel) {
  static const char* names[psc::kTimerSlots] = {"pack",          "attn_schedule", "attn_fwd", "attn_bwd_pre",
                                                "attn_bwd_dkdv", "attn_bwd_dq",   "rope",     "data_steps"};
  return (kernel >= 0 && kernel < psc::kTimerSlots) ? names[kernel] : "unknown";
}

}  // extern "C"
