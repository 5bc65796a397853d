// Kernel timing for benchmarks (bsmm_timing_enable / bsmm_timing_read): while
// enabled, the main launch of every call is bracketed by HIP events recorded
// on the call's stream.  Events are pooled and reused across enables.

#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "bsmm.h"
#include "bsmm_internal.h"

namespace bsmm {
namespace {

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> start, stop;   // pool; the first `used` pairs are live
  size_t used = 0;
  std::string name;
};
Timing& timing_state() {
  static Timing t;
  return t;
}

}  // namespace

bool timing_on() {
  Timing& t = timing_state();
  std::lock_guard<std::mutex> g(t.mu);
  return t.on;
}

void timing_mark(void* stream, const char* name, bool begin) {
  Timing& t = timing_state();
  std::lock_guard<std::mutex> g(t.mu);
  if (!t.on) return;
  if (begin) {
    if (t.used == t.start.size()) {
      hipEvent_t a, b;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&b) != hipSuccess) { (void)hipEventDestroy(a); return; }
      t.start.push_back(a);
      t.stop.push_back(b);
    }
    (void)hipEventRecord(t.start[t.used], (hipStream_t)stream);
    t.name = name;
  } else if (t.used < t.start.size()) {
    (void)hipEventRecord(t.stop[t.used], (hipStream_t)stream);
    ++t.used;
  }
}

}  // namespace bsmm

using namespace bsmm;

extern "C" {

bsmm_status bsmm_timing_enable(int enable) {
  Timing& t = timing_state();
  std::lock_guard<std::mutex> g(t.mu);
  t.on = enable != 0;
  t.used = 0;
  t.name.clear();
  return BSMM_OK;
}

bsmm_status bsmm_timing_read(double* mean_ms, int64_t* count, char* name, size_t name_len) {
  if (!mean_ms || !count) return BSMM_ERR_NULL;
  Timing& t = timing_state();
  std::lock_guard<std::mutex> g(t.mu);
  double sum = 0.0;
  for (size_t i = 0; i < t.used; ++i) {
    if (hipEventSynchronize(t.stop[i]) != hipSuccess) return BSMM_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.start[i], t.stop[i]) != hipSuccess) return BSMM_ERR_HIP;
    sum += ms;
  }
  *count = (int64_t)t.used;
  *mean_ms = t.used ? sum / (double)t.used : 0.0;
  if (name && name_len) snprintf(name, name_len, "%s", t.name.c_str());
  return BSMM_OK;
}

}  // extern "C"
