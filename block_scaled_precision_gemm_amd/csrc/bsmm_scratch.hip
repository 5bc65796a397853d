// The library's static device scratch: the workspace of the allocation-free
// entry point (bsmm_fp8_blockwise_scratch), for callers that cannot
// allocate device memory.  Every GPU the library runs on holds its own copy
// of the array until the process ends; every call on a GPU uses that GPU's
// copy, so calls that overlap on one GPU race.  Nothing in it has to start
// at zero: each call overwrites the packed scales and split-K partials it
// reads, and stream-K counters carry a per-launch tag.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "bsmm_internal.h"

namespace bsmm {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// The address of the current device's copy of `scratch`, looked up once per
// device with that device current.  The array's name in host code is a
// host-side stand-in, never a device address: kernels and copies take the
// pointer returned here.  Null (with *err set to the HIP error) on failure.
void* scratch_device_ptr(int* err) {
  *err = 0;
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? (int)e : -1;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (r != hipSuccess || p == nullptr) {
      *err = r != hipSuccess ? (int)r : -1;
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace bsmm
