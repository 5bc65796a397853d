// Packed scale_a for the fp8 kernels (layout described in bsmm_internal.h).
//
// Rows past M repeat row M-1; the GEMM kernels never store the results of
// those rows.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsmm_internal.h"

namespace bsmm {
namespace {

// One thread per packed group: rows 64q + f + 16i, i = 0..3, of K block kb,
// which sit at positions 64q + 4f .. 64q + 4f + 3 of the block's row; four
// loads and one 16-byte (fp32) or 4-byte (e8m0) store.  A workgroup covers
// 16 K blocks x 16 groups (one 64-row block), so consecutive threads store
// consecutive groups and the 16 K blocks of a row share its cache line.
template <int OP>
__global__ void __launch_bounds__(256)
pack_kernel(const Problem p, void* dst, int64_t ld) {
  const int KB = p.K / kBlockK;
  const int q = blockIdx.x, g = blockIdx.z;
  const int f = threadIdx.x & 15;
  const int kb = blockIdx.y * 16 + (threadIdx.x >> 4);
  if (kb >= KB) return;
  const int64_t o = ((int64_t)g * KB + kb) * ld + (int64_t)q * 64 + 4 * f;
  if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
    const uint8_t* src = (const uint8_t*)p.sa + (int64_t)g * p.sa_sg + kb;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = min(q * 64 + 16 * i + f, p.M - 1);
      v |= (uint32_t)src[(int64_t)m * p.sa_m] << (8 * i);
    }
    *(uint32_t*)((uint8_t*)dst + o) = v;
  } else {
    const float* src = (const float*)p.sa + (int64_t)kb * p.sa_kb;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = min(q * 64 + 16 * i + f, p.M - 1);
      v[i] = src[(int64_t)m * p.sa_m];
    }
    typedef float f4 __attribute__((ext_vector_type(4)));
    *(f4*)((float*)dst + o) = f4{v[0], v[1], v[2], v[3]};
  }
}

// mx32: one thread per packed group of one 32-K chunk c.  A: rows 64q + f
// + 16i, i = 0..3, into one 4-byte word at c*Mp + 64q + 4f.  B: columns
// 128q + f + 16j, j = 0..7, into one 8-byte word at c*Np + 128q + 8f.  Rows
// past M / columns past N repeat the last one.  A workgroup covers 16
// chunks x 16 groups.
template <bool B_SIDE>
__global__ void __launch_bounds__(256)
pack_mx32_kernel(const Problem p, uint8_t* dst, int64_t ld) {
  const int KC = p.K / 32;
  const int q = blockIdx.x;
  const int f = threadIdx.x & 15;
  const int c = blockIdx.y * 16 + (threadIdx.x >> 4);
  if (c >= KC) return;
  if constexpr (!B_SIDE) {
    const uint8_t* src = (const uint8_t*)p.sa + c;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v |= (uint32_t)src[(int64_t)min(q * 64 + 16 * i + f, p.M - 1) * p.sa_m] << (8 * i);
    *(uint32_t*)(dst + (int64_t)c * ld + (int64_t)q * 64 + 4 * f) = v;
  } else {
    const uint8_t* src = (const uint8_t*)p.sb + c;
    uint32_t v[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j >> 2] |= (uint32_t)src[(int64_t)min(q * 128 + 16 * j + f, p.N - 1) * p.sb_n]
                   << (8 * (j & 3));
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    *(u2*)(dst + (int64_t)c * ld + (int64_t)q * 128 + 8 * f) = u2{v[0], v[1]};
  }
}

// groupwise scale_b: one thread per packed column n of K block kb, plain
// column order, columns past N repeating column N-1.
__global__ void __launch_bounds__(256)
pack_cols_kernel(const Problem p, float* dst, int64_t ld) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int kb = blockIdx.y;
  if (n >= ld) return;
  const float* src = (const float*)p.sb + (int64_t)kb * p.sb_kb;
  dst[(int64_t)kb * ld + n] = src[(int64_t)min((int)n, p.N - 1) * p.sb_n];
}

}  // namespace

int pack_scale_a(const Problem& p, void* dst, void* stream) {
  if (!packable_scales(p.op) || dst == nullptr || ((uintptr_t)dst & 15u) || p.M <= 0)
    return 1;
  hipStream_t s = (hipStream_t)stream;
  if (p.op == BSMM_OP_FP8_MX32_MM) {
    const int KC = p.K / 32;
    if (KC == 0) return 0;
    const int64_t mp = packed_rows(p.M), np = packed_rows(p.N);
    uint8_t* d = (uint8_t*)dst;
    hipLaunchKernelGGL(pack_mx32_kernel<false>, dim3((unsigned)(mp / 64), (unsigned)((KC + 15) / 16)),
                       dim3(256), 0, s, p, d, mp);
    hipLaunchKernelGGL(pack_mx32_kernel<true>, dim3((unsigned)(np / 128), (unsigned)((KC + 15) / 16)),
                       dim3(256), 0, s, p, d + packed_mx32_a_bytes(p.M, p.K), np);
    return hipGetLastError() == hipSuccess ? 0 : 1;
  }
  const int KB = p.K / kBlockK;
  if (KB == 0) return 0;
  if (p.op == BSMM_OP_FP8_GROUPWISE) {
    const int64_t mp = packed_rows(p.M), np = packed_rows(p.N);
    hipLaunchKernelGGL(pack_kernel<BSMM_OP_FP8_BLOCKWISE>,
                       dim3((unsigned)(mp / 64), (unsigned)((KB + 15) / 16), 1u), dim3(256), 0, s,
                       p, dst, mp);
    hipLaunchKernelGGL(pack_cols_kernel, dim3((unsigned)(np / 256), (unsigned)KB), dim3(256), 0, s,
                       p, (float*)((uint8_t*)dst + packed_gw_a_bytes(p.M, p.K)), np);
    return hipGetLastError() == hipSuccess ? 0 : 1;
  }
  const int64_t ld = packed_rows(p.M);
  const dim3 grid((unsigned)(ld / 64), (unsigned)((KB + 15) / 16),
                  (unsigned)(p.op == BSMM_OP_FP8_MX_BMM ? p.G : 1));
  if (p.op == BSMM_OP_FP8_MX_BMM)
    hipLaunchKernelGGL(pack_kernel<BSMM_OP_FP8_MX_BMM>, grid, dim3(256), 0, s, p, dst, ld);
  else
    hipLaunchKernelGGL(pack_kernel<BSMM_OP_FP8_BLOCKWISE>, grid, dim3(256), 0, s, p, dst, ld);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace bsmm
