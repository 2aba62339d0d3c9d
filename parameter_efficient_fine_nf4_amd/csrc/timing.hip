// timing.hip -- optional per-kernel timing of libqlora's launches.
//
// While enabled, every kernel the library launches carries two HIP events
// that its dispatch stamps with the kernel's start and end time
// (hipExtLaunchKernel).  qlora_timing_collect() waits for the events and adds
// each pair's elapsed time to the kernel's running total.  A profiling aid: the state is process-wide and
// guarded by a mutex; events are created on demand and reused.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"
#include "qlora.h"

namespace qlora {

namespace {
struct Bracket {
  const char* name;
  hipEvent_t start, stop;
};
struct TimingState {
  std::mutex mu;
  bool on = false;
  bool failed = false;
  std::vector<hipEvent_t> pool;     // free events
  std::vector<Bracket> pending;     // recorded, not yet collected
  std::map<std::string, std::pair<double, int64_t>> totals;
};
TimingState& state() {
  static TimingState s;
  return s;
}
hipEvent_t take_event(TimingState& s) {
  if (!s.pool.empty()) {
    hipEvent_t e = s.pool.back();
    s.pool.pop_back();
    return e;
  }
  // timing only: no system-scope fence (no cache writeback/invalidate of
  // its own around the kernel it stamps)
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) {
    s.failed = true;
    return nullptr;
  }
  return e;
}
}  // namespace

TimedLaunch::TimedLaunch(const char* name, hipStream_t)
    : active_(false), name_(name), a_(nullptr), b_(nullptr) {
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (!s.on) return;
  a_ = take_event(s);
  b_ = take_event(s);
  if (a_ == nullptr || b_ == nullptr) {
    s.failed = true;
    if (a_) s.pool.push_back(a_);
    if (b_) s.pool.push_back(b_);
    return;
  }
  active_ = true;
}

TimedLaunch::~TimedLaunch() {
  if (!active_) return;
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  if (hipPeekAtLastError() != hipSuccess) s.failed = true;
  s.pending.push_back(Bracket{name_, a_, b_});
}

}  // namespace qlora

using namespace qlora;

extern "C" {

int qlora_timing_enable(int on) {
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  s.on = on != 0;
  return QLORA_OK;
}

int qlora_timing_collect(void) {
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  int status = s.failed ? QLORA_ERR_HIP : QLORA_OK;
  s.failed = false;
  for (const Bracket& b : s.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(b.stop) != hipSuccess || hipEventElapsedTime(&ms, b.start, b.stop) != hipSuccess) {
      status = QLORA_ERR_HIP;
    } else {
      auto& t = s.totals[b.name];
      t.first += ms;
      t.second += 1;
    }
    s.pool.push_back(b.start);
    s.pool.push_back(b.stop);
  }
  s.pending.clear();
  return status;
}

int qlora_timing_query(const char* kernel, double* total_ms, int64_t* launches) {
  if (kernel == nullptr || total_ms == nullptr || launches == nullptr) return QLORA_ERR_NULL;
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  auto it = s.totals.find(kernel);
  *total_ms = it == s.totals.end() ? 0.0 : it->second.first;
  *launches = it == s.totals.end() ? 0 : it->second.second;
  return QLORA_OK;
}

int qlora_timing_reset(void) {
  TimingState& s = state();
  std::lock_guard<std::mutex> g(s.mu);
  s.totals.clear();
  return QLORA_OK;
}

}  // extern "C"
