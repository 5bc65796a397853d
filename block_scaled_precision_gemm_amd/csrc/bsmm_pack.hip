// Packed scale_a for the fp8 kernels (layout described in bsmm_internal.h).
//
// One workgroup per 64 rows x 32 K blocks (x G), transposed through LDS so
// that both the reads (along K blocks, the contiguous direction of the
// pages' [M, K/128] scale tensor) and the writes (along rows) are
// contiguous.  Rows past M repeat row M-1; the GEMM kernels never store the
// results of those rows.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsmm_internal.h"

namespace bsmm {
namespace {

template <int OP>
__global__ void __launch_bounds__(256)
pack_kernel(const Problem p, void* dst, int64_t ld) {
  __shared__ uint32_t t[32][65];
  const int KB = p.K / kBlockK;
  const int q = blockIdx.x, kb0 = blockIdx.y * 32, g = blockIdx.z;
  const int tid = threadIdx.x;
  const int kl = tid & 31;
  for (int rl = tid >> 5; rl < 64; rl += 8) {
    const int m = min(q * 64 + rl, p.M - 1);
    const int kb = kb0 + kl;
    uint32_t v = 0;
    if (kb < KB) {
      if constexpr (OP == BSMM_OP_FP8_MX_BMM)
        v = ((const uint8_t*)p.sa)[(int64_t)g * p.sa_sg + (int64_t)m * p.sa_m + kb];
      else
        v = __float_as_uint(((const float*)p.sa)[(int64_t)m * p.sa_m + (int64_t)kb * p.sa_kb]);
    }
    t[kl][rl] = v;
  }
  __syncthreads();
  const int pl = tid & 63;
  const int rl = 16 * (pl & 3) + (pl >> 2);     // position 4f + i <- row 16i + f
  for (int kl2 = tid >> 6; kl2 < 32; kl2 += 4) {
    const int kb = kb0 + kl2;
    if (kb >= KB) break;
    const int64_t o = ((int64_t)g * KB + kb) * ld + (int64_t)q * 64 + pl;
    if constexpr (OP == BSMM_OP_FP8_MX_BMM) ((uint8_t*)dst)[o] = (uint8_t)t[kl2][rl];
    else ((uint32_t*)dst)[o] = t[kl2][rl];
  }
}

}  // namespace

int pack_scale_a(const Problem& p, void* dst, void* stream) {
  if (p.op == BSMM_OP_INT8_ROWWISE || dst == nullptr || ((uintptr_t)dst & 15u) || p.M <= 0)
    return 1;
  const int KB = p.K / kBlockK;
  if (KB == 0) return 0;
  const int64_t ld = packed_rows(p.M);
  const dim3 grid((unsigned)(ld / 64), (unsigned)((KB + 31) / 32),
                  (unsigned)(p.op == BSMM_OP_FP8_MX_BMM ? p.G : 1));
  hipStream_t s = (hipStream_t)stream;
  if (p.op == BSMM_OP_FP8_MX_BMM)
    hipLaunchKernelGGL(pack_kernel<BSMM_OP_FP8_MX_BMM>, grid, dim3(256), 0, s, p, dst, ld);
  else
    hipLaunchKernelGGL(pack_kernel<BSMM_OP_FP8_BLOCKWISE>, grid, dim3(256), 0, s, p, dst, ld);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace bsmm
