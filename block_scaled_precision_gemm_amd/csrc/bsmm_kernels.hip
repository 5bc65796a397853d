// HIP kernels for the block-scaled matmul on gfx950 (CDNA4).
//
// One tile kernel template serves the three entry points:
//   * int8 rowwise     -- v_mfma_i32_16x16x64_i8, exact int32 accumulators,
//                         scales applied in the epilogue;
//   * fp8 blockwise    -- v_mfma_scale_f32_16x16x128_f8f6f4 with unit e8m0
//                         scales gives the fp32 partial of one 128-K block,
//                         which one fp32 multiply-add per element folds into
//                         the accumulator with the block's scale product;
//   * fp8 mx (e8m0)    -- the same instruction with the blocks' e8m0 scale
//                         bytes as its hardware scale operands, accumulating
//                         in place.
// The K extent of one 16x16x128 fp8 instruction is exactly one scale block.
//
// Data movement: A and B tiles (both K-contiguous, 128 bytes of K per step)
// go global -> LDS with direct-to-LDS buffer loads (no staging registers),
// double-buffered; rows past the end of the matrix fall outside the buffer
// resource's range and load as zeros, so partial tiles need no masks on the
// load side.  LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled so
// that the fragment reads (16 consecutive rows per lane group) hit distinct
// banks.  Fragments are read with ds_read_b128.
//
// Lane layouts (gfx950, checked on hardware against a host reference):
//   16x16 operand: lane l holds row (l % 16); its 32 bytes cover K bytes
//     [32*(l/16), +32) of the 128-byte block (the hardware's internal K order
//     within those bytes is irrelevant because A and B use the same order and
//     one scale covers the whole block);
//   16x16 result: lane l, register r -> row 4*(l/16) + r, column l % 16.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsmm_internal.h"

namespace bsmm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWave = 64;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, dword format
constexpr uint32_t kOob = 0xFFFFFFF0u;         // a voffset past any range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                           uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)n, (int)kRsrcWord3);
}

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row; depends only on
// row % 16, so rows 16 apart share a pattern and fragment addresses of
// different 16-row tiles differ by constants.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int lds_off(int r, int c) {
  return (r << 7) + ((c ^ swz(r)) << 4);
}

__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
    return (uint16_t)((u >> 16) | 0x0040u);          // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Kernel arguments: the validated problem plus the launch's row range and
// split.
// ---------------------------------------------------------------------------
struct KArgs {
  Problem p;
  int row_begin, row_end;
  int tiles_m, tiles_n;
  int splits, kb_per_split;
  void* ws;           // split-K partials [splits][G][rows][N] (fp32 / int32)
};

template <int OP> struct OpT;
template <> struct OpT<BSMM_OP_INT8_ROWWISE> { typedef i32x4 acc_t; typedef int elem_t; };
template <> struct OpT<BSMM_OP_FP8_BLOCKWISE> { typedef f32x4 acc_t; typedef float elem_t; };
template <> struct OpT<BSMM_OP_FP8_MX_BMM> { typedef f32x4 acc_t; typedef float elem_t; };

// Map the flat workgroup id to (split, group, tile_m, tile_n).
//  1. XCD-aware remap: consecutive hardware ids land on different XCDs
//     (round robin over 8), so contiguous runs of logical ids are given to
//     one XCD and share its L2.
//  2. GROUP_M rasterisation over the tiles (the grouped program-id order of
//     the Triton mm template in Inductor's mm.py) for L2 reuse.
struct TileId { int s, g, tm, tn; };
__device__ __forceinline__ TileId decode_tile(const KArgs& k) {
  const int total = gridDim.x;
  const int hw = blockIdx.x;
  const int per = total >> 3, rem = total & 7;
  const int xcd = hw & 7, local = hw >> 3;
  int pid = (xcd < rem) ? xcd * (per + 1) + local
                        : rem * (per + 1) + (xcd - rem) * per + local;
  const int tiles = k.tiles_m * k.tiles_n;
  TileId t;
  int tile = pid % tiles;
  int rest = pid / tiles;
  t.g = rest % k.p.G;
  t.s = rest / k.p.G;
  constexpr int GROUP_M = 8;
  const int width = GROUP_M * k.tiles_n;
  const int gid = tile / width;
  const int first_m = gid * GROUP_M;
  const int gsize = min(k.tiles_m - first_m, GROUP_M);
  const int in = tile - gid * width;
  t.tm = first_m + in % gsize;
  t.tn = in / gsize;
  return t;
}

// ---------------------------------------------------------------------------
// The tile kernel.  Workgroup tile BM x BN, waves arranged WM x WN, each wave
// a 64 x 128 sub-tile = 4 x 8 MFMA tiles of 16 x 16.
// ---------------------------------------------------------------------------
template <int OP, int WM, int WN>
struct Tile {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * kWave;
  static constexpr int WTM = 64, WTN = 128;
  static constexpr int TI = WTM / 16, TJ = WTN / 16;
  static constexpr int BM = WM * WTM, BN = WN * WTN;
  static constexpr int A_BYTES = BM * kBlockK;
  static constexpr int B_BYTES = BN * kBlockK;
  // blockwise: BM fp32 row scales + up to 64 fp32 column-block scales
  static constexpr int S_BYTES = (OP == BSMM_OP_FP8_BLOCKWISE) ? (BM * 4 + 256) : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int LDS = 2 * STAGE;
  static_assert((BM / 8) % NW == 0 || NW % (BM / 8) == 0, "A loader split");
};

template <int R, int NW>
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t rs,
                                          uint8_t* dst, uint32_t ld,
                                          uint32_t kbyte, int wave, int lane) {
  // R rows x 128 bytes; one wave instruction moves 8 rows (64 x 16 bytes)
  // to LDS bytes [q*1024, q*1024+1024) of the tile, lane l -> slot l.
  constexpr int Q = R / 8;
  if constexpr (Q >= NW) {
#pragma unroll
    for (int t = 0; t < Q / NW; ++t) {
      const int q = t * NW + wave;
      const int r = q * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const uint32_t vo = (uint32_t)r * ld + kbyte + ((uint32_t)c << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + q * 1024),
                                               16, vo, 0, 0, 0);
    }
  } else {
    if (wave < Q) {
      const int q = wave;
      const int r = q * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const uint32_t vo = (uint32_t)r * ld + kbyte + ((uint32_t)c << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + q * 1024),
                                               16, vo, 0, 0, 0);
    }
  }
}

template <int OP, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
tile_kernel(const KArgs k) {
  using T = Tile<OP, WM, WN>;
  using acc_t = typename OpT<OP>::acc_t;
  constexpr int BM = T::BM, BN = T::BN, TI = T::TI, TJ = T::TJ;
  constexpr int NW = T::NW;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS];

  const Problem& p = k.p;
  const TileId t = decode_tile(k);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const int row0 = k.row_begin + t.tm * BM;
  const int col0 = t.tn * BN;
  const int KB = p.K / kBlockK;
  const int kb0 = t.s * k.kb_per_split;
  const int kb1 = min(KB, kb0 + k.kb_per_split);

  // Buffer resources: rows past the launch's end / past N are out of range.
  const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(
      p.a + (int64_t)t.g * p.a_sg + (int64_t)row0 * p.lda,
      (uint64_t)(k.row_end - row0) * p.lda);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(
      p.b + (int64_t)t.g * p.b_sg + (int64_t)col0 * p.ldb,
      (uint64_t)(p.N - col0) * p.ldb);

  // Blockwise scale resources (fp32): rows of this tile, column blocks.
  __amdgpu_buffer_rsrc_t rsa, rsb;
  if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
    const float* sa = (const float*)p.sa + (int64_t)row0 * p.sa_m;
    const int64_t last = (int64_t)(k.row_end - 1 - row0) * p.sa_m +
                         (int64_t)(KB - 1) * p.sa_kb + 1;
    rsa = make_rsrc(sa, (uint64_t)last * 4);
    const int NB = p.N / kBlockK;
    const int64_t lastb = (int64_t)(KB - 1) * p.sb_kb + (int64_t)(NB - 1) * p.sb_n + 1;
    rsb = make_rsrc(p.sb, (uint64_t)lastb * 4);
  }

  auto issue = [&](int kb, int st) {
    uint8_t* base = smem + st * T::STAGE;
    const uint32_t kbyte = (uint32_t)kb * kBlockK;
    load_rows<BM, NW>(ra, base, lda, kbyte, wave, lane);
    load_rows<BN, NW>(rb, base + T::A_BYTES, ldb, kbyte, wave, lane);
    if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
      uint8_t* sdst = base + T::A_BYTES + T::B_BYTES;
      constexpr int QA = BM / 64;             // 64 row scales per instruction
#pragma unroll
      for (int q = 0; q <= QA; ++q) {
        if (wave == q % NW) {
          uint32_t vo;
          if (q < QA) {
            vo = (uint32_t)(((int64_t)(q * 64 + lane) * p.sa_m +
                             (int64_t)kb * p.sa_kb) * 4);
            if (row0 + q * 64 + lane >= k.row_end) vo = kOob;
          } else {
            const int nb = col0 / kBlockK + lane;
            vo = (lane < BN / kBlockK)
                     ? (uint32_t)(((int64_t)kb * p.sb_kb + (int64_t)nb * p.sb_n) * 4)
                     : kOob;
          }
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              q < QA ? rsa : rsb, (lds_ptr_t)(sdst + q * 256), 4, vo, 0, 0, 0);
        }
      }
    }
  };

  acc_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = acc_t{0, 0, 0, 0};

  // Per-lane fragment addresses (bytes within a stage): row / column
  // (lane % 16) of the wave's first 16-row tile, chunks 2*(lane/16) + h.
  const int fr = lane & 15;
  const int fc = (lane >> 4) * 2;
  const int a_r = wm * T::WTM + fr;
  const int b_r = wn * T::WTN + fr;
  const int a_off0 = lds_off(a_r, fc), a_off1 = lds_off(a_r, fc + 1);
  const int b_off0 = T::A_BYTES + lds_off(b_r, fc);
  const int b_off1 = T::A_BYTES + lds_off(b_r, fc + 1);

  // mx scale bytes: x_scale rows of this lane's 4 row tiles, w_scale block.
  const uint8_t* xs_row[TI];
  const uint8_t* ws_blk = nullptr;
  if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      int m = row0 + wm * T::WTM + i * 16 + fr;
      m = min(m, k.row_end - 1);   // rows past the end: any valid row
      xs_row[i] = (const uint8_t*)p.sa + (int64_t)t.g * p.sa_sg + (int64_t)m * p.sa_m;
    }
    // waves whose columns lie past N (N tail) read the last block's scale;
    // their results are never stored
    const int nb = min((col0 + wn * T::WTN) / kBlockK, p.N / kBlockK - 1);
    ws_blk = (const uint8_t*)p.sb + (int64_t)t.g * p.sb_sg + (int64_t)nb * p.sb_n;
  }

  // mx scale bytes of the current K block; the next block's are loaded one
  // step ahead, together with its tiles.
  int xsc[TI];
  int wsc = 127;
  if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
    if (kb0 < kb1) {
#pragma unroll
      for (int i = 0; i < TI; ++i) xsc[i] = xs_row[i][kb0];
      wsc = ws_blk[kb0];
    }
  }

  if (kb0 < kb1) issue(kb0, 0);
  for (int kb = kb0; kb < kb1; ++kb) {
    const int st = (kb - kb0) & 1;
    wait_vmem();
    __syncthreads();
    int xsn[TI];
    int wsn = 127;
    if (kb + 1 < kb1) {
      issue(kb + 1, st ^ 1);
      if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
#pragma unroll
        for (int i = 0; i < TI; ++i) xsn[i] = xs_row[i][kb + 1];
        wsn = ws_blk[kb + 1];
      }
    }
    const uint8_t* S = smem + st * T::STAGE;

    i32x8 af[TI];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const i32x4 lo = *(const i32x4*)(S + a_off0 + i * 2048);
      const i32x4 hi = *(const i32x4*)(S + a_off1 + i * 2048);
      af[i] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }

    f32x4 sc[TI];
    if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
      const float* sa_s = (const float*)(S + T::A_BYTES + T::B_BYTES);
      const float sbv = sa_s[BM + wn];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const f32x4 v = *(const f32x4*)(sa_s + wm * T::WTM + i * 16 + 4 * (lane >> 4));
        sc[i] = v * sbv;
      }
    }

#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const i32x4 blo = *(const i32x4*)(S + b_off0 + j * 2048);
      const i32x4 bhi = *(const i32x4*)(S + b_off1 + j * 2048);
      const i32x8 bf = i32x8{blo.x, blo.y, blo.z, blo.w, bhi.x, bhi.y, bhi.z, bhi.w};
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
          const i32x4 alo = i32x4{af[i][0], af[i][1], af[i][2], af[i][3]};
          const i32x4 ahi = i32x4{af[i][4], af[i][5], af[i][6], af[i][7]};
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi, acc[i][j], 0, 0, 0);
        } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bf, f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[i][j][r] = __builtin_fmaf(sc[i][r], part[r], acc[i][j][r]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[i], bf, acc[i][j], 0, 0, 0, xsc[i], 0, wsc);
        }
      }
    }
    if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
#pragma unroll
      for (int i = 0; i < TI; ++i) xsc[i] = xsn[i];
      wsc = wsn;
    }
  }

  // ------------------------------------------------------------- epilogue --
  const int mbase = row0 + wm * T::WTM + 4 * (lane >> 4);
  const int nbase = col0 + wn * T::WTN + fr;
  if (k.splits > 1) {
    // fp32 / int32 partials, reduced in split order by splitk_reduce.
    const int rows = k.row_end - k.row_begin;
    typedef typename OpT<OP>::elem_t E;
    E* ws = (E*)k.ws + ((int64_t)t.s * p.G + t.g) * (int64_t)rows * p.N;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = mbase + i * 16 + r, n = nbase + j * 16;
          if (m < k.row_end && n < p.N)
            ws[(int64_t)(m - k.row_begin) * p.N + n] = acc[i][j][r];
        }
    return;
  }

  uint8_t* obase = (uint8_t*)p.out;
  const int osz = p.out_dtype == BSMM_BF16 ? 2 : 4;
  const int64_t og = (int64_t)t.g * p.o_sg;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    float sa_r[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
      if (p.out_dtype != BSMM_I32) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = min(mbase + i * 16 + r, k.row_end - 1);
          sa_r[r] = ((const float*)p.sa)[(int64_t)m * p.sa_m];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = nbase + j * 16;
      float sb_c = 1.f;
      if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
        if (p.out_dtype != BSMM_I32)
          sb_c = ((const float*)p.sb)[(int64_t)min(n, p.N - 1) * p.sb_n];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mbase + i * 16 + r;
        if (m >= k.row_end || n >= p.N) continue;
        const int64_t e = og + (int64_t)m * p.ldo + n;
        if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
          if (p.out_dtype == BSMM_I32) {
            ((int*)obase)[e] = acc[i][j][r];
            continue;
          }
          // (f32(acc) * sa) * sb, two separately rounded binary32 products
          const float y = __fmul_rn(__fmul_rn((float)acc[i][j][r], sa_r[r]), sb_c);
          if (osz == 2) ((uint16_t*)obase)[e] = f32_to_bf16_rne(y);
          else ((float*)obase)[e] = y;
        } else {
          const float y = acc[i][j][r];
          if (osz == 2) ((uint16_t*)obase)[e] = f32_to_bf16_rne(y);
          else ((float*)obase)[e] = y;
        }
      }
    }
  }
}

// Split-K reduction: out = epilogue(sum over s of partial[s]) in ascending s.
template <int OP>
__global__ void __launch_bounds__(256)
splitk_reduce(const KArgs k) {
  const Problem& p = k.p;
  const int rows = k.row_end - k.row_begin;
  const int64_t per_g = (int64_t)rows * p.N;
  const int64_t total = per_g * p.G;
  typedef typename OpT<OP>::elem_t E;
  const E* ws = (const E*)k.ws;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(e / per_g);
    const int64_t rem = e - (int64_t)g * per_g;
    const int mr = (int)(rem / p.N);
    const int n = (int)(rem - (int64_t)mr * p.N);
    E s = 0;
    for (int q = 0; q < k.splits; ++q) s += ws[(int64_t)q * total + e];
    const int m = k.row_begin + mr;
    const int64_t o = (int64_t)g * p.o_sg + (int64_t)m * p.ldo + n;
    float y;
    if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
      if (p.out_dtype == BSMM_I32) { ((int*)p.out)[o] = (int)s; continue; }
      y = __fmul_rn(__fmul_rn((float)s, ((const float*)p.sa)[(int64_t)m * p.sa_m]),
                    ((const float*)p.sb)[(int64_t)n * p.sb_n]);
    } else {
      y = (float)s;
    }
    if (p.out_dtype == BSMM_BF16) ((uint16_t*)p.out)[o] = f32_to_bf16_rne(y);
    else ((float*)p.out)[o] = y;
  }
}

// Output for K == 0: zeros.
__global__ void zero_out(const KArgs k) {
  const Problem& p = k.p;
  const int64_t per_g = (int64_t)p.M * p.N;
  const int64_t total = per_g * p.G;
  const int osz = p.out_dtype == BSMM_BF16 ? 2 : 4;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(e / per_g);
    const int64_t rem = e - (int64_t)g * per_g;
    const int m = (int)(rem / p.N);
    const int n = (int)(rem - (int64_t)m * p.N);
    const int64_t o = (int64_t)g * p.o_sg + (int64_t)m * p.ldo + n;
    if (osz == 2) ((uint16_t*)p.out)[o] = 0;
    else ((uint32_t*)p.out)[o] = 0;
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int check_launch() {
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

template <int OP, int WM, int WN>
int launch_tile(const Problem& p, int row_begin, int row_end, int split,
                void* ws, void* stream) {
  using T = Tile<OP, WM, WN>;
  KArgs k;
  k.p = p;
  k.row_begin = row_begin;
  k.row_end = row_end;
  const int rows = row_end - row_begin;
  k.tiles_m = (rows + T::BM - 1) / T::BM;
  k.tiles_n = (p.N + T::BN - 1) / T::BN;
  const int KB = p.K / kBlockK;
  k.ws = ws;
  hipStream_t s = (hipStream_t)stream;
  if (KB == 0) {              // empty sum: the output is zero
    k.splits = 1;
    k.kb_per_split = 0;
    hipLaunchKernelGGL(zero_out, dim3(1024), dim3(256), 0, s, k);
    return check_launch();
  }
  if (split < 1) split = 1;
  if (split > KB) split = KB;
  k.kb_per_split = (KB + split - 1) / split;
  k.splits = (KB + k.kb_per_split - 1) / k.kb_per_split;
  const int64_t grid = (int64_t)k.tiles_m * k.tiles_n * p.G * k.splits;
  hipLaunchKernelGGL((tile_kernel<OP, WM, WN>), dim3((unsigned)grid), dim3(T::NT), 0, s, k);
  if (check_launch()) return 1;
  if (k.splits > 1) {
    const int64_t total = (int64_t)rows * p.N * p.G;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(splitk_reduce<OP>, dim3((unsigned)blocks), dim3(256), 0, s, k);
    return check_launch();
  }
  return 0;
}

constexpr unsigned kAllOps = 7u;

#define BSMM_VARIANT(NAME, WM, WN)                                              \
  static int NAME##_launch(const Problem& p, int rb, int re, int sp, void* ws,  \
                           void* st) {                                          \
    switch (p.op) {                                                             \
      case BSMM_OP_INT8_ROWWISE:                                                \
        return launch_tile<BSMM_OP_INT8_ROWWISE, WM, WN>(p, rb, re, sp, ws, st); \
      case BSMM_OP_FP8_BLOCKWISE:                                               \
        return launch_tile<BSMM_OP_FP8_BLOCKWISE, WM, WN>(p, rb, re, sp, ws, st); \
      default:                                                                  \
        return launch_tile<BSMM_OP_FP8_MX_BMM, WM, WN>(p, rb, re, sp, ws, st);  \
    }                                                                           \
  }

BSMM_VARIANT(t256x256, 4, 2)
BSMM_VARIANT(t256x128, 4, 1)
BSMM_VARIANT(t128x256, 2, 2)
BSMM_VARIANT(t128x128, 2, 1)
BSMM_VARIANT(t64x256, 1, 2)
BSMM_VARIANT(t64x128, 1, 1)

const Variant kVariants[] = {
    {"t256x256", 256, 256, kAllOps, true, t256x256_launch},
    {"t256x128", 256, 128, kAllOps, true, t256x128_launch},
    {"t128x256", 128, 256, kAllOps, true, t128x256_launch},
    {"t128x128", 128, 128, kAllOps, true, t128x128_launch},
    {"t64x256", 64, 256, kAllOps, true, t64x256_launch},
    {"t64x128", 64, 128, kAllOps, true, t64x128_launch},
};

}  // namespace

const Variant* variants(int* count) {
  *count = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
  return kVariants;
}

}  // namespace bsmm
