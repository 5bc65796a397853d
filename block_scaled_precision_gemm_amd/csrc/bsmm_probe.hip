// Matrix-core throughput probe: a measurement aid for the roofline, not part
// of any matmul.  Every wave issues chains of independent matrix
// instructions on register operands (no memory traffic in the loop), so the
// launch runs at the rate the matrix cores sustain on this device, at the
// clock it holds under that load.  Four instructions: those of the
// library's K loops, the fp8 16 x 16 x 128 instruction with unit e8m0 scales
// and the int8 16 x 16 x 64 one, and their 32 x 32 forms (int8 32 x 32 x 32,
// fp8 32 x 32 x 64).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsmm.h"

namespace bsmm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;   // independent accumulators per wave

// Operand bytes that vary by lane and word (finite E4M3 codes: bit 3 cleared
// keeps every byte off the NaN patterns), so the data is not a constant.
__device__ __forceinline__ int lane_bytes(int lane, int word) {
  uint32_t h = (uint32_t)(lane * 2654435761u) ^ (uint32_t)(word * 40503u + 0x9E3779B9u);
  h ^= h >> 13;
  h *= 0x5bd1e995u;
  h ^= h >> 15;
  return (int)(h & 0xF7F7F7F7u);
}

template <int KIND>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  i32x8 a, b;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    a[w] = lane_bytes(lane, w);
    b[w] = lane_bytes(lane + 64, w);
  }
  f32x4 acc[kChains];
  i32x4 iacc[kChains];
  i32x16 wacc[KIND == 2 ? kChains : 1];
  f32x16 facc[KIND == 3 ? kChains : 1];
#pragma unroll
  for (int t = 0; t < kChains; ++t) {
    acc[t] = f32x4{0, 0, 0, 0};
    iacc[t] = i32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int t = 0; t < (KIND == 2 ? kChains : 1); ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) wacc[t][r] = 0;
#pragma unroll
  for (int t = 0; t < (KIND == 3 ? kChains : 1); ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) facc[t][r] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int t = 0; t < kChains; ++t) {
      if constexpr (KIND == 0) {
        acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[t], 0, 0, 0, 127,
                                                                  0, 127);
      } else if constexpr (KIND == 1) {
        iacc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{a[0], a[1], a[2], a[3]},
                                                        i32x4{b[0], b[1], b[2], b[3]},
                                                        iacc[t], 0, 0, 0);
      } else if constexpr (KIND == 2) {
        wacc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(i32x4{a[0], a[1], a[2], a[3]},
                                                        i32x4{b[0], b[1], b[2], b[3]},
                                                        wacc[t], 0, 0, 0);
      } else {
        facc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, facc[t], 0, 0, 0, 127,
                                                                  0, 127);
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < kChains; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += KIND == 0 ? acc[t][r] : (float)iacc[t][r];
  if constexpr (KIND == 2)
#pragma unroll
    for (int t = 0; t < kChains; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += (float)wacc[t][r];
  if constexpr (KIND == 3)
#pragma unroll
    for (int t = 0; t < kChains; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += facc[t][r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace bsmm

extern "C" bsmm_status bsmm_mfma_probe(int kind, int workgroups, int iters, float* out,
                                       void* stream) {
  if (kind < 0 || kind > 3 || workgroups <= 0 || iters <= 0) return BSMM_ERR_ARG;
  if (out == nullptr) return BSMM_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (kind == 0)
    hipLaunchKernelGGL(bsmm::mfma_probe_kernel<0>, dim3((unsigned)workgroups), dim3(256), 0, s,
                       iters, out);
  else if (kind == 1)
    hipLaunchKernelGGL(bsmm::mfma_probe_kernel<1>, dim3((unsigned)workgroups), dim3(256), 0, s,
                       iters, out);
  else if (kind == 2)
    hipLaunchKernelGGL(bsmm::mfma_probe_kernel<2>, dim3((unsigned)workgroups), dim3(256), 0, s,
                       iters, out);
  else
    hipLaunchKernelGGL(bsmm::mfma_probe_kernel<3>, dim3((unsigned)workgroups), dim3(256), 0, s,
                       iters, out);
  return hipGetLastError() == hipSuccess ? BSMM_OK : BSMM_ERR_HIP;
}
