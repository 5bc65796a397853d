// Dynamic quantisation of bf16 / fp32 activations into the codes and scales
// the scaled matmuls consume (gfx950).
//
//   int8, one scale per row: scale = amax / 127, code = clamp(rne(x / scale),
//     +-127) -- the symmetric per-row activation quantisation of the torchao
//     issue "Unify scaled INT8 matmul";
//   fp8 E4M3FN, one fp32 scale per 1 x 128 block: scale = amax / 448, code =
//     rne_e4m3(x / scale) -- the [M, K/128] activation scales of the PyTorch
//     issue "torch._scaled_mm with blockwise scaling doesn't work with
//     torch.compile";
//   fp8 E4M3FN, one e8m0 scale per 1 x 128 block: scale = 2^e with
//     e = ceil(log2(amax / 448)), code = rne_e4m3(x * 2^-e) -- the mxscale
//     activations of the ROCm aiter PR "Add opus fp8 mxscale BMM kernels for
//     gfx950" (Motivation); the same per 1 x 32 block for the 32-element MX
//     blocks of the MX matmul;
//   for the backward pass of the blockwise fp8 linear layer the PyTorch issue
//     benchmarks: fp8 E4M3FN with one fp32 scale amax / 448 per group of 128
//     consecutive rows of one column (the weight gradient contracts over
//     tokens), and per 128 x 128 block of a weight; both write the codes
//     transposed (the layout in which the GEMM that consumes them reads its
//     contraction contiguously), the weight optionally also as it is.
//
// Every quotient is the correctly rounded binary32 quotient; rounding is to
// nearest, ties to even; e4m3 saturates at +-448.  A row or block whose
// fp32 scale is 0 (amax 0, or amax so small that amax / 127 or amax / 448
// underflows) stores scale 1 (e8m0: byte 127, amax 0) and +0 codes.  The
// e8m0 exponent is clamped below at -127.
//
// All three kernels move each input byte once and each output byte once, so
// they are bound by HBM bandwidth: loads are 16 bytes per lane and
// coalesced, the arithmetic per element is a handful of VALU operations.
// Input loads and code stores are non-temporal: nothing is reused, and on
// MI355X streaming them past the caches measured 10-15% faster; the matmul
// that reads the codes next ran no slower.
//
// Division: x / s with one correctly rounded reciprocal r = 1 / s per row or
// block and, per element, q0 = x * r, e = fma(-q0, s, x), q = fma(e, r, q0).
// With r within half an ulp of 1/s and q0 within one ulp of x/s, e is exact
// and q is the correctly rounded quotient as long as nothing underflows
// (Markstein, "Computation of elementary functions on the IBM RISC
// System/6000 processor", 1990).  That holds for every element whose
// quotient can reach a rounding boundary of the int8 or e4m3 grid when
// s >= 2^-80; below that the kernels divide each element with the IEEE
// division instead.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bsmm.h"
#include "bsmm_internal.h"

namespace bsmm {
namespace {

constexpr float kFastDivMin = 0x1p-80f;
constexpr int kIters = 3;              // fp8: blocks per lane group per workgroup

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ inline uint4 load16_nt(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline void store8_nt(void* p, uint2 w) {
  const u32x2 v = {w.x, w.y};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

// ---- 8 consecutive input elements -------------------------------------------

template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> { uint4 v; };            // bf16 bits
template <> struct Raw8<float> { uint4 lo, hi; };          // fp32 bits

__device__ inline void load8(Raw8<uint16_t>& r, const uint16_t* p) { r.v = load16_nt(p); }
__device__ inline void load8(Raw8<float>& r, const float* p) {
  r.lo = load16_nt(p);
  r.hi = load16_nt(p + 4);
}

// Widen to fp32 (bf16 -> fp32 is exact: the bf16 bits are the top half).
__device__ inline void widen(const Raw8<uint16_t>& r, float f[8]) {
  const uint32_t w[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ inline void widen(const Raw8<float>& r, float f[8]) {
  const uint32_t w[8] = {r.lo.x, r.lo.y, r.lo.z, r.lo.w, r.hi.x, r.hi.y, r.hi.z, r.hi.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(w[i]);
}

// max |x| of the 8 elements, as the bits of a non-negative float (integer
// order equals float order for non-negative finite values)
template <typename T>
__device__ inline uint32_t absmax_bits(const Raw8<T>& r) {
  float f[8];
  widen(r, f);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(f[i]) & 0x7FFFFFFFu);
  return m;
}

// ---- cross-lane maxima -------------------------------------------------------

// DPP row operations act on 16-lane rows: xor 1 and xor 2 inside each quad,
// then rotations by 4 and 8 inside the row.
__device__ inline uint32_t row16_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
  return v;
}
// the same within groups of LPB = 4 or 16 consecutive lanes
template <int LPB>
__device__ inline uint32_t group_max(uint32_t v) {
  if constexpr (LPB == 16) return row16_max(v);
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  return v;
}
__device__ inline uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// ---- division and rounding ---------------------------------------------------

// s > 0, so the quotient has the sign of x; the correction step alone would
// turn x = -0 into +0 (fma(+0, r, -0) = +0).
__device__ inline float div_fast(float x, float s, float r) {
  const float q0 = __fmul_rn(x, r);
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
}

// Four e4m3 codes (nearest, ties to even) of values already within +-448,
// packed little-endian.  The gfx950 conversion writes OCP E4M3FN in the
// current rounding mode (round to nearest even).
__device__ inline uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ inline float clamp448(float t) {
  return __builtin_amdgcn_fmed3f(t, -448.0f, 448.0f);
}

// int8 codes of four values already rounded to integers in [-127, 127]
__device__ inline uint32_t i8x4(float a, float b, float c, float d) {
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)(int)b, (uint32_t)(int)a, 0x0C0C0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)(int)d, (uint32_t)(int)c, 0x0C0C0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

__device__ inline float round_i8(float t) {
  return __builtin_amdgcn_fmed3f(__builtin_rintf(t), -127.0f, 127.0f);
}

// ---- int8, one scale per row ---------------------------------------------------

// WPR waves per row (1: four rows per workgroup; 4: one row per workgroup,
// the four wave maxima combined through LDS).  A pass covers 64 * WPR * 8 *
// NV elements, held in registers; a longer row is read twice (amax, then
// codes).
template <typename T, int WPR, int NV>
__global__ void __launch_bounds__(256)
quant_int8_rows(const T* __restrict__ x, int64_t ldx, int8_t* __restrict__ q, int64_t ldq,
                float* __restrict__ scale, int64_t s_m, int M, int K) {
  static_assert(WPR == 1 || WPR == 4, "one or four waves per row");
  constexpr int kLanes = 64 * WPR;
  constexpr int kPass = kLanes * 8 * NV;
  const int lane = threadIdx.x & 63;
  const int t = WPR == 1 ? lane : (int)threadIdx.x;      // lane index within the row
  const int row = WPR == 1 ? blockIdx.x * 4 + (threadIdx.x >> 6) : blockIdx.x;
  if (WPR == 1 && row >= M) return;   // whole waves only (no barrier below for WPR 1)
  const T* xr = x + (int64_t)row * ldx;
  int8_t* qr = q + (int64_t)row * ldq;
  Raw8<T> buf[NV];
  uint32_t amax = 0;
  // Lanes past the end of the row load the row's last 8 elements (always in
  // bounds, K >= 8 here) and leave them out of the maximum; loads are never
  // branched around, so the buffers stay in registers.
  for (int base = 0; base < K; base += kPass) {
#pragma unroll
    for (int v = 0; v < NV; ++v) load8(buf[v], xr + min(base + (v * kLanes + t) * 8, K - 8));
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const uint32_t m = absmax_bits(buf[v]);
      amax = max(amax, base + (v * kLanes + t) * 8 < K ? m : 0u);
    }
  }
  amax = wave_max(amax);
  if (WPR > 1) {
    __shared__ uint32_t part[WPR];
    if (lane == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WPR; ++w) amax = max(amax, part[w]);
  }
  float s = __uint_as_float(amax) / 127.0f;
  if (!(s > 0.0f)) s = 1.0f;   // amax 0 or an underflowing scale: codes are 0 anyway
  if (t == 0) scale[(int64_t)row * s_m] = s;
  const bool fast = s >= kFastDivMin;
  const float r = 1.0f / s;
  for (int base = 0; base < K; base += kPass) {
    if (K > kPass) {
#pragma unroll
      for (int v = 0; v < NV; ++v) load8(buf[v], xr + min(base + (v * kLanes + t) * 8, K - 8));
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int k = base + (v * kLanes + t) * 8;
      if (k >= K) continue;
      float f[8];
      widen(buf[v], f);
      if (fast) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = round_i8(div_fast(f[i], s, r));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = round_i8(f[i] / s);
      }
      uint2 w;
      w.x = i8x4(f[0], f[1], f[2], f[3]);
      w.y = i8x4(f[4], f[5], f[6], f[7]);
      store8_nt(qr + k, w);
    }
  }
}

// ---- fp8, one scale per 1 x 128 block ------------------------------------------

// e8m0 exponent ceil(log2(amax / 448)) from the bits of amax, clamped to
// [-127, 127].  448 = 1.75 * 2^8: for amax = m * 2^E (m in [1, 2)) the
// exponent is E - 8 when m <= 1.75, else E - 7.  A subnormal amax is below
// 448 * 2^-127 and takes the clamp; amax 0 gives 0.
__device__ inline int e8m0_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return 0;
  const int field = (int)(amax_bits >> 23);
  if (field == 0) return -127;
  const int e = field - 127 - 8 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(e, -127);
}

// MX = false: fp32 scale amax / 448; MX = true: e8m0 scale.  LPB lanes of
// 8 elements per block: 16 (128-element blocks) or 4 (32-element MX blocks).
template <typename T, bool MX, int LPB>
__global__ void __launch_bounds__(256)
quant_fp8_blocks(const T* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                 void* __restrict__ scale, int64_t s_m, int64_t s_kb, uint32_t nblocks,
                 uint32_t KB) {
  constexpr int BLOCK = 8 * LPB;
  constexpr int PER_ITER = 256 / LPB;          // blocks per iteration of the workgroup
  const int l = threadIdx.x % LPB;
  const uint32_t b0 = blockIdx.x * (PER_ITER * kIters) + threadIdx.x / LPB;
  Raw8<T> buf[kIters];
  uint32_t row[kIters], kb[kIters];
  // a block past the end loads the last block (in bounds, nblocks >= 1) and
  // stores nothing
#pragma unroll
  for (int u = 0; u < kIters; ++u) {
    const uint32_t b = min(b0 + u * PER_ITER, nblocks - 1);
    row[u] = b / KB;
    kb[u] = b - row[u] * KB;
    load8(buf[u], x + (int64_t)row[u] * ldx + (int64_t)kb[u] * BLOCK + l * 8);
  }
#pragma unroll
  for (int u = 0; u < kIters; ++u) {
    // the lanes of a block share a DPP row (or quad), which is live or dead as a whole
    const uint32_t amax = group_max<LPB>(absmax_bits(buf[u]));
    if (b0 + u * PER_ITER >= nblocks) continue;
    float f[8];
    widen(buf[u], f);
    uint2 w;
    if (MX) {
      const int e = e8m0_exponent(amax);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = __builtin_amdgcn_ldexpf(f[i], -e);
      w.x = e4m3x4(f[0], f[1], f[2], f[3]);
      w.y = e4m3x4(f[4], f[5], f[6], f[7]);
      if (amax == 0) w = make_uint2(0, 0);
      if (l == 0)
        static_cast<uint8_t*>(scale)[(int64_t)row[u] * s_m + (int64_t)kb[u] * s_kb] =
            (uint8_t)(e + 127);
    } else {
      float s = __uint_as_float(amax) / 448.0f;
      const bool zero = !(s > 0.0f);
      if (zero) s = 1.0f;
      if (s >= kFastDivMin) {
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = clamp448(div_fast(f[i], s, r));
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = clamp448(f[i] / s);
      }
      w.x = e4m3x4(f[0], f[1], f[2], f[3]);
      w.y = e4m3x4(f[4], f[5], f[6], f[7]);
      if (zero) w = make_uint2(0, 0);
      if (l == 0)
        static_cast<float*>(scale)[(int64_t)row[u] * s_m + (int64_t)kb[u] * s_kb] = s;
    }
    store8_nt(q + (int64_t)row[u] * ldq + (int64_t)kb[u] * BLOCK + l * 8, w);
  }
}

// ---- fp8 down the columns / 128 x 128 blocks, transposed codes ---------------

// A workgroup quantises a tile of 128 rows x CW columns: one scale per
// column (groups of 128 rows down the columns; CW = 64 or 128), or, with
// BLOCK2D and CW = 128, one scale for the 128 x 128 block.  Work item it = threadIdx.x +
// 256 * ii holds rows 4a .. 4a + 3 of the 8 columns 8c .. 8c + 7 of the tile
// (c = it % (CW / 8), a = it / (CW / 8)), so 8 consecutive items read one
// 128-byte row segment (bf16).  Column chunks past C (C a multiple of 8) load
// the last chunk and store nothing.  The codes of one column's four rows
// make a dword, written to LDS at byte (8c + j) * kPitch + 4a (row pitch 132:
// at most two lanes of a wave per bank); each column's 128 codes then leave
// as 16-byte segments of row c0 + 8c + j of the transposed output.  BLOCK2D
// also stores the codes untransposed when q is not null.  ROWQ (column
// groups, CW = 128) also quantises each row's 128 columns of the tile as a
// 1 x 128 block, the forward quantisation of the same input: the 16 lanes
// that hold one row form a DPP row, so the block maximum is a row16_max;
// codes go to q untransposed and the row scale to srow.
template <typename T, int CW, bool BLOCK2D, bool ROWQ = false>
__global__ void __launch_bounds__(256)
quant_fp8_tiles(const T* __restrict__ x, int64_t ldx, uint8_t* __restrict__ q, int64_t ldq,
                uint8_t* __restrict__ qt, int64_t ldqt, float* __restrict__ scale, int64_t s_g,
                int64_t s_c, int C, float* __restrict__ srow = nullptr, int64_t sr_m = 0,
                int64_t sr_kb = 0) {
  static_assert(!ROWQ || (CW == 128 && !BLOCK2D), "row blocks span the 128-column tile");
  constexpr int NI = CW / 64;          // work items per thread
  constexpr int QW = CW / 8;           // 8-column chunks per tile row
  constexpr int kPitch = 132;
  constexpr int NS = BLOCK2D ? 1 : CW; // scales per tile
  __shared__ uint32_t part[4][NS];
  __shared__ float sc[NS];
  __shared__ __attribute__((aligned(16))) uint8_t tt[CW * kPitch];
  const int g = blockIdx.y;
  const int c0 = blockIdx.x * CW;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row0 = (int64_t)g * 128;
  Raw8<T> buf[NI][4];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int it = threadIdx.x + 256 * ii;
    const int col = min(c0 + 8 * (it % QW), C - 8);
    const int a = it / QW;
#pragma unroll
    for (int i = 0; i < 4; ++i) load8(buf[ii][i], x + (row0 + 4 * a + i) * ldx + col);
  }
  // maxima: per column (groups down the columns) or over the tile (blocks)
  if constexpr (BLOCK2D) {
    uint32_t m = 0;
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, absmax_bits(buf[ii][i]));
    m = wave_max(m);
    if (lane == 0) part[wave][0] = m;
  } else {
    // lanes QW k + c of a wave hold column chunk c in every item (256 is a
    // multiple of QW): reduce over the items, then over k
    static_assert(QW == 8 || QW == 16, "column chunks per tile row");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t m = 0;
#pragma unroll
      for (int ii = 0; ii < NI; ++ii)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float f[8];
          widen(buf[ii][i], f);
          m = max(m, __float_as_uint(f[j]) & 0x7FFFFFFFu);
        }
      if (QW == 8)
        m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xF, 0xF, false));
      m = max(m, (uint32_t)__shfl_xor((int)m, 16));
      m = max(m, (uint32_t)__shfl_xor((int)m, 32));
      if (lane < QW) part[wave][8 * lane + j] = m;
    }
  }
  __syncthreads();
  if (threadIdx.x < NS) {
    const int t = threadIdx.x;
    const uint32_t amax = max(max(part[0][t], part[1][t]), max(part[2][t], part[3][t]));
    float sv = __uint_as_float(amax) / 448.0f;
    if (!(sv > 0.0f)) sv = 0.0f;       // marks a zero group: scale 1, codes +0
    sc[t] = sv;
    const int cs = BLOCK2D ? blockIdx.x : c0 + t;
    if (BLOCK2D || cs < C) scale[(int64_t)g * s_g + (int64_t)cs * s_c] = sv > 0.0f ? sv : 1.0f;
  }
  __syncthreads();
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int it = threadIdx.x + 256 * ii;
    const int cc = it % QW, a = it / QW;
    float f[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) widen(buf[ii][i], f[i]);
    if constexpr (ROWQ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = max(m, __float_as_uint(f[i][j]) & 0x7FFFFFFFu);
        m = row16_max(m);
        float sv = __uint_as_float(m) / 448.0f;
        const bool zero = !(sv > 0.0f);
        if (zero) sv = 1.0f;
        float g[8];
        if (sv >= kFastDivMin) {
          const float r = 1.0f / sv;
#pragma unroll
          for (int j = 0; j < 8; ++j) g[j] = clamp448(div_fast(f[i][j], sv, r));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) g[j] = clamp448(f[i][j] / sv);
        }
        uint2 w;
        w.x = e4m3x4(g[0], g[1], g[2], g[3]);
        w.y = e4m3x4(g[4], g[5], g[6], g[7]);
        if (zero) w = make_uint2(0, 0);
        store8_nt(q + (row0 + 4 * a + i) * ldq + c0 + 8 * cc, w);
        if (cc == 0) srow[(row0 + 4 * a + i) * sr_m + (int64_t)blockIdx.x * sr_kb] = sv;
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float sv = sc[BLOCK2D ? 0 : 8 * cc + j];
      const float s = sv > 0.0f ? sv : 1.0f;
      if (s >= kFastDivMin) {
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i][j] = clamp448(div_fast(f[i][j], s, r));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i][j] = clamp448(f[i][j] / s);
      }
      if (!(sv > 0.0f))
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i][j] = 0.0f;
      *reinterpret_cast<uint32_t*>(tt + (8 * cc + j) * kPitch + 4 * a) =
          e4m3x4(f[0][j], f[1][j], f[2][j], f[3][j]);
    }
    if (BLOCK2D && q != nullptr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 w;
        w.x = e4m3x4(f[i][0], f[i][1], f[i][2], f[i][3]);
        w.y = e4m3x4(f[i][4], f[i][5], f[i][6], f[i][7]);
        store8_nt(q + (row0 + 4 * a + i) * ldq + c0 + 8 * cc, w);
      }
    }
  }
  if (qt == nullptr) return;
  __syncthreads();
  // row c of the tile's transposed codes: 8 segments of 16 bytes
#pragma unroll
  for (int n = 0; n < CW * 8 / 256; ++n) {
    const int ci = threadIdx.x + 256 * n;
    const int c = ci >> 3, k = ci & 7;
    if (c0 + c >= C) continue;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(tt + c * kPitch + 16 * k);
    const u32x4 v = {src[0], src[1], src[2], src[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(qt + (int64_t)(c0 + c) * ldqt +
                                                            row0 + 16 * k));
  }
}

// columns per workgroup tile of the column-group quantiser: 128 (eight
// 16-byte loads in flight per lane) measured 4-6% faster than 64 on MI355X
constexpr int kColTile = 128;

template <typename T, int CW, bool BLOCK2D, bool ROWQ = false>
void launch_tiles(const QuantArgs& a, hipStream_t st) {
  const dim3 grid((unsigned)((a.K + CW - 1) / CW), (unsigned)(a.M / 128));
  hipLaunchKernelGGL((quant_fp8_tiles<T, CW, BLOCK2D, ROWQ>), grid, dim3(256), 0, st,
                     static_cast<const T*>(a.x), a.ldx, static_cast<uint8_t*>(a.q), a.ldq,
                     static_cast<uint8_t*>(a.qt), a.ldqt, static_cast<float*>(a.scale), a.s_m,
                     a.s_kb, (int)a.K, static_cast<float*>(a.scale2), a.s2_m, a.s2_kb);
}

template <typename T, int WPR, int NV>
void launch_rows(const QuantArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)(WPR == 1 ? (a.M + 3) / 4 : a.M);
  hipLaunchKernelGGL((quant_int8_rows<T, WPR, NV>), dim3(grid), dim3(256), 0, st,
                     static_cast<const T*>(a.x), a.ldx, static_cast<int8_t*>(a.q), a.ldq,
                     static_cast<float*>(a.scale), a.s_m, (int)a.M, (int)a.K);
}

// Short rows: a wave per row.  Longer rows: a workgroup per row, so each
// wave carries less of the row and more waves overlap their loads with
// other waves' stores (MI355X, 8192 x 4096 bf16: 19.8 us against 20.6 for
// a wave per row).
template <typename T>
void launch_rows_nv(const QuantArgs& a, hipStream_t st) {
  if (a.K <= 512) launch_rows<T, 1, 1>(a, st);
  else if (a.K <= 1024) launch_rows<T, 1, 2>(a, st);
  else if (a.K <= 2048) launch_rows<T, 4, 1>(a, st);
  else if (a.K <= 4096) launch_rows<T, 4, 2>(a, st);
  else launch_rows<T, 4, 4>(a, st);
}

template <typename T, bool MX, int LPB>
void launch_blocks(const QuantArgs& a, hipStream_t st) {
  const uint32_t KB = (uint32_t)(a.K / (8 * LPB));
  const uint32_t nblocks = (uint32_t)(a.M * KB);
  const uint32_t per_wg = 256 / LPB * kIters;
  const unsigned grid = (nblocks + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((quant_fp8_blocks<T, MX, LPB>), dim3(grid), dim3(256), 0, st,
                     static_cast<const T*>(a.x), a.ldx, static_cast<uint8_t*>(a.q), a.ldq,
                     a.scale, a.s_m, a.s_kb, nblocks, KB);
}

}  // namespace

int launch_quant(const QuantArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = a.x_dtype == BSMM_BF16;
  switch (a.kind) {
    case QuantArgs::kInt8Rows:
      if (bf) launch_rows_nv<uint16_t>(a, st); else launch_rows_nv<float>(a, st);
      break;
    case QuantArgs::kFp8Blocks:
      if (bf) launch_blocks<uint16_t, false, 16>(a, st); else launch_blocks<float, false, 16>(a, st);
      break;
    case QuantArgs::kFp8Mx32:
      if (bf) launch_blocks<uint16_t, true, 4>(a, st); else launch_blocks<float, true, 4>(a, st);
      break;
    case QuantArgs::kFp8Columns:
      if (bf) launch_tiles<uint16_t, kColTile, false>(a, st);
      else launch_tiles<float, kColTile, false>(a, st);
      break;
    case QuantArgs::kFp8Weight:
      if (bf) launch_tiles<uint16_t, 128, true>(a, st); else launch_tiles<float, 128, true>(a, st);
      break;
    case QuantArgs::kFp8RowsColumns:
      if (bf) launch_tiles<uint16_t, 128, false, true>(a, st);
      else launch_tiles<float, 128, false, true>(a, st);
      break;
    default:
      if (bf) launch_blocks<uint16_t, true, 16>(a, st); else launch_blocks<float, true, 16>(a, st);
      break;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace bsmm
