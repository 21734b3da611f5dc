// Per-kernel HIP-event timing (include/pa_profile.h). Records are appended
// under a mutex while profiling is on; reading them waits on the events.
#include <atomic>
#include <mutex>
#include <vector>

#include "pa_profile.h"
#include "pa_internal.h"

namespace pa {
namespace {

struct Record {
  int id;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_done;
std::vector<hipEvent_t> g_free;
thread_local hipEvent_t t_open[PA_PROFILE_KERNELS] = {};

const char* const kNames[PA_PROFILE_KERNELS] = {"kv_write", "decode", "partition_reduce", "prefill_plan",
                                                "prefill", "kv_write_plan", "decode_order"};

hipEvent_t take_event() {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_free.empty()) {
      hipEvent_t e = g_free.back();
      g_free.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle_all() {
  for (auto& r : g_done) {
    g_free.push_back(r.start);
    g_free.push_back(r.stop);
  }
  g_done.clear();
}

}  // namespace

bool profiling() { return g_on.load(std::memory_order_relaxed); }

void profile_mark(int id, bool end, hipStream_t stream) {
  if (!profiling() || id < 0 || id >= PA_PROFILE_KERNELS) return;
  if (!end) {
    hipEvent_t e = take_event();
    if (e && hipEventRecord(e, stream) == hipSuccess) t_open[id] = e;
    return;
  }
  hipEvent_t start = t_open[id];
  t_open[id] = nullptr;
  if (!start) return;
  hipEvent_t stop = take_event();
  if (!stop || hipEventRecord(stop, stream) != hipSuccess) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_done.push_back({id, start, stop});
}

}  // namespace pa

extern "C" {

int pa_profile_start(void) {
  std::lock_guard<std::mutex> lk(pa::g_mu);
  for (auto& r : pa::g_done) {
    (void)hipEventSynchronize(r.stop);
  }
  pa::recycle_all();
  pa::g_on.store(true);
  return 0;
}

int pa_profile_stop(void) {
  pa::g_on.store(false);
  return 0;
}

int pa_profile_kernel(int id, double* total_ms, int64_t* launches) {
  if (id < 0 || id >= PA_PROFILE_KERNELS) return 3;
  std::lock_guard<std::mutex> lk(pa::g_mu);
  double sum = 0;
  int64_t n = 0;
  for (auto& r : pa::g_done) {
    if (r.id != id) continue;
    float ms = 0;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      return 7;
    sum += ms;
    ++n;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = n;
  return 0;
}

const char* pa_profile_kernel_name(int id) {
  return (id >= 0 && id < PA_PROFILE_KERNELS) ? pa::kNames[id] : "";
}

}  // extern "C"
