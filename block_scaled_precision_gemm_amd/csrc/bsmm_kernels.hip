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
// go global -> LDS with direct-to-LDS buffer loads (no staging registers)
// into a ring of LDS slots; rows past the end of the matrix fall outside the buffer
// resource's range and load as zeros, so partial tiles need no masks on the
// load side.  LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled so
// that the fragment reads (16 consecutive rows per lane group) hit distinct
// banks.  Fragments are read with ds_read_b128.
//
// Lane layouts (gfx950, checked on hardware against a host reference):
//   16x16 operand: lane l holds row (l % 16); its 32 bytes cover K bytes
//     [32*(l/16), +32) of the 128-byte block (the hardware's internal K order
//     within those bytes is irrelevant because A and B use the same order and
//     one scale covers the whole block; the 32-element MX blocks need the
//     instruction's own order -- see kChunk);
//   16x16 result D = X * Y: lane l, register r -> D[4*(l/16) + r][l % 16].
// The kernels compute the transposed product (X = B fragment, Y = A
// fragment), so lane l holds output row (l % 16) and the four consecutive
// output columns 4*(l/16) .. +3: the epilogue stores 8 or 16 contiguous bytes
// per lane and each lane needs one row scale per 16-row tile.

#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdint>
#include <type_traits>

#include "bsmm_internal.h"

namespace bsmm {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kWave = 64;
constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw buffer, dword format
constexpr uint32_t kOob = 0xFFFFFFF0u;         // a voffset past any range
constexpr int kSc0 = 1;                        // buffer cache policy bit sc0

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

// Workgroup barrier for the K loop.  Each wave has already waited for its
// own direct-to-LDS loads and consumed every LDS read of the stage being
// recycled, so a bare s_barrier suffices (no release fence); the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Two fp32 values to a packed pair of bf16 (a in the low half) with the
// hardware conversion (v_cvt_pk_bf16_f32): round to nearest even, as the
// kernels' float mode (round to nearest even, denormals kept) sets it; a NaN
// input is unsupported.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
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
  int vec_out;        // output (or workspace) rows allow 8/16-byte stores
  void* ws;           // split-K partials [splits][G][rows][N] (fp32 / int32)
  const void* psa;    // packed scale_a [G][KB][psa_ld] (packed-scale kernels)
  int64_t psa_ld;
  int units;          // tiles_m * tiles_n * G * splits work units of the launch
  uint64_t epoch;     // narrow split-K: distinct per launch (tags its counters)
};

template <int OP> struct OpT;
template <> struct OpT<BSMM_OP_INT8_ROWWISE> { typedef i32x4 acc_t; typedef int elem_t; };
template <> struct OpT<BSMM_OP_FP8_BLOCKWISE> { typedef f32x4 acc_t; typedef float elem_t; };
template <> struct OpT<BSMM_OP_FP8_MX_BMM> { typedef f32x4 acc_t; typedef float elem_t; };
template <> struct OpT<BSMM_OP_FP8_SCALED_MM> { typedef f32x4 acc_t; typedef float elem_t; };
template <> struct OpT<BSMM_OP_FP8_MX32_MM> { typedef f32x4 acc_t; typedef float elem_t; };
template <> struct OpT<BSMM_OP_FP8_GROUPWISE> { typedef f32x4 acc_t; typedef float elem_t; };

// fp8 scaled_mm epilogue: Inductor's apply_scaling (acc * (sa * sb)), then
// the bias, then the result scale; each step one binary32 rounding.
struct ScaledEpi {
  float sr;
  bool has_bias, bias_bf16;
  const void* bias;
  __device__ __forceinline__ explicit ScaledEpi(const Problem& p)
      : sr(p.sr ? *p.sr : 1.0f), has_bias(p.bias != nullptr), bias_bf16(p.bias_bf16 != 0),
        bias(p.bias) {}
  __device__ __forceinline__ float bias_at(int n) const {
    return bias_bf16 ? __uint_as_float((uint32_t)((const uint16_t*)bias)[n] << 16)
                     : ((const float*)bias)[n];
  }
  __device__ __forceinline__ float operator()(float acc, float sa, float sb, int n) const {
    float y = __fmul_rn(acc, __fmul_rn(sa, sb));
    if (has_bias) y = __fadd_rn(y, bias_at(n));   // absent: no +0, which would turn -0 into +0
    return __fmul_rn(y, sr);
  }
};

// Map a work unit (flat workgroup id) to (split, group, tile_m, tile_n).
//  1. XCD-aware remap: consecutive hardware ids land on different XCDs
//     (round robin over 8), so contiguous runs of logical ids are given to
//     one XCD and share its L2.
//  2. GROUP_M rasterisation over the tiles (the grouped program-id order of
//     the Triton mm template in Inductor's mm.py) for L2 reuse.
//  3. A grid smaller than the number of units (one workgroup per slot of the
//     device) is persistent: workgroup slot w takes units w, w + grid, ...,
//     so while a tile's stores drain the workgroup already loads its next
//     tile, and the CUs drift out of step instead of all storing at once.
struct TileId { int s, g, tm, tn; };
__device__ __forceinline__ int first_unit() {
  const int total = gridDim.x;
  const int hw = blockIdx.x;
  const int per = total >> 3, rem = total & 7;
  const int xcd = hw & 7, local = hw >> 3;
  return (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}
__device__ __forceinline__ TileId decode_tile(const KArgs& k, int pid) {
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
//
// LDS is a ring of NSLOT slots; K block c of the workgroup occupies two
// "half-stages": h = 2c (its A tile) and h = 2c + 1 (its B tile), in slot
// h % NSLOT.  While K block c computes from its two slots, the other
// NSLOT - 2 half-stages are in flight (for 256 x 256 tiles: five 32 KB slots,
// the whole 160 KB, so 1.5 K blocks stay in flight).  The two slots of block
// c - 1 are refilled with half-stages 2c + NSLOT - 2 and 2c + NSLOT - 1 as
// soon as every wave has passed the barrier at the top of block c.  Scales
// do not go through LDS (groupwise aside): each lane loads the ones it needs
// into registers one K block ahead.
//
// Groupwise (a column scale per lane column, 32 per lane and K block, more
// than the registers hold): each K block's packed scale_a slice (BM rows)
// and scale_b slice (BN columns) ride with its A half-stage into a 1 KB
// region each beside the slot, and the K loop reads them from LDS when it
// folds.  The ring then has four slots (the regions take the fifth's room).
// ---------------------------------------------------------------------------
template <int OP, int WM, int WN, int RING>
struct Tile {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * kWave;
  static constexpr int WTM = 64, WTN = 128;
  static constexpr int TI = WTM / 16, TJ = WTN / 16;
  static constexpr int BM = WM * WTM, BN = WN * WTN;
  static constexpr int A_BYTES = BM * kBlockK;
  static constexpr int B_BYTES = BN * kBlockK;
  static constexpr int SLOT = A_BYTES > B_BYTES ? A_BYTES : B_BYTES;
  static constexpr bool GW = OP == BSMM_OP_FP8_GROUPWISE;
  static constexpr int NSLOT = GW ? 4 : RING;
#ifndef BSMM_LOADER_SPLIT
#define BSMM_LOADER_SPLIT 1
#endif
  // Waves that issue the tile loads: the first half, one per SIMD, so that
  // while a loading wave waits to issue a load its SIMD sibling keeps the
  // matrix core busy.
  static constexpr int NLD = BSMM_LOADER_SPLIT && NW >= 8 ? NW / 2 : NW;
  // groupwise: scale loads per loading wave and A half-stage (instruction
  // q = t * NLD + wave moves 1 KB: q = 0 scale_a, q = 1 scale_b, others no
  // memory), and the LDS bytes of one slot's scale regions
  static constexpr int SCL_LOADS = GW ? (NLD >= 2 ? 1 : 2) : 0;
  static constexpr int SCL = NLD * SCL_LOADS * 1024;
  static constexpr int LDS = NSLOT * (SLOT + SCL);
  // direct-to-LDS loads per loading wave for one A (tile rows, then the
  // scale loads) / one B half-stage
  static constexpr int LA_ROWS = BM / 8 / NLD;
  static constexpr int LA = LA_ROWS + SCL_LOADS, LB = BN / 8 / NLD;
  // loads of the half-stages after block c's pair that may still be in
  // flight when block c starts: h = 2c+2 .. 2c+NSLOT-3 (A, B, A, ...)
  static constexpr int WAIT = ((NSLOT - 3) / 2) * LA + ((NSLOT - 4) / 2) * LB;
  static_assert(NSLOT >= 4, "the ring needs at least four slots");
  static_assert((BM / 8) % NLD == 0 && (BN / 8) % NLD == 0, "loader split");
  static_assert(WAIT < 64, "vmcnt range");
  static_assert(TI == 4, "packed scales hold four rows per lane");
  static_assert(!GW || (BM * 4 <= 1024 && BN * 4 <= 1024), "one scale load per slice");
};

// R rows x 128 bytes; one wave instruction moves 8 rows (64 x 16 bytes) to
// LDS bytes [q*1024, q*1024+1024) of the slot, lane l -> slot byte 16 l.
// Wave `wave` of NW issues instructions t = 0 .. R/8/NW - 1, q = t*NW + wave.
// The lane's part of the offset (its row and swizzled chunk) is the same for
// every K block, so it stays in a register; the block's byte offset goes in
// the instruction's scalar offset, and the load costs no VALU work.  A dead
// half-stage (past the last K block) is issued through `dead`, a resource
// of zero bytes: it keeps the per-wave load count uniform and touches no
// memory.  Rows past the end of the matrix are out of range through their
// lane offset alone, and a valid row's access stays inside that row, so the
// result does not depend on whether the range check counts the scalar
// offset.
template <int NW>
__device__ __forceinline__ void load_row_group(__amdgpu_buffer_rsrc_t rs,
                                               __amdgpu_buffer_rsrc_t dead, uint8_t* dst,
                                               uint32_t ld, uint32_t kbyte, int wave,
                                               int lane, bool live, int t) {
  const int q = t * NW + wave;
  const int r = q * 8 + (lane >> 3);
  const int c = (lane & 7) ^ swz(r);
  const uint32_t vo = (uint32_t)r * ld + ((uint32_t)c << 4);
  // the LDS address is the low word of the generic one; formed as an
  // integer it needs no null check of the generic pointer
  const lds_ptr_t l = (lds_ptr_t)(uintptr_t)(uint32_t)(uintptr_t)(dst + q * 1024);
  // sc0: the loads miss in the CU's L1 instead of allocating there -- every
  // byte goes to LDS once, and the tiles' re-use is in L2 (mx 8 x 8192 x
  // 1024 x 4096: 1.7% faster; the other workloads unchanged)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rs : dead, l, 16, vo, (int)kbyte, 0, kSc0);
}

// mx MFMA: scale byte-select `sel` (0..3, a constant after unrolling) picks the
// B-side (A-fragment) e8m0 scale from the lane's packed four row scales.
__device__ __forceinline__ f32x4 mfma_mx(i32x8 x, i32x8 y, f32x4 c, int sx, int sel,
                                         uint32_t sy) {
  switch (sel) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, sx, 0, (int)sy);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, sx, 1, (int)sy);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, sx, 2, (int)sy);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, sx, 3, (int)sy);
  }
}

// Which 16-byte chunks of a row's 128-byte K block a lane (group g = lane
// / 16) gives the 16 x 16 x 128 fp8 instruction.  The instruction reads a
// lane's 32 bytes as K [16 g, 16 g + 16) and then K [64 + 16 g, 64 + 16 g +
// 16), and multiplies its 32-K block b (K [32 b, 32 b + 32) in that order)
// by the scale byte of lane group b -- measured on gfx950 by doubling one
// scale byte at a time against data in one 16-K chunk at a time.  With one
// scale per 128-K block any assignment used alike for both operands works,
// and the lane reads chunks 2g and 2g + 1; with 32-element blocks (mx32) it
// reads chunks g and g + 4, so that the instruction's K order is the true
// one and scale byte b covers true K [32 b, 32 b + 32).
template <int OP> struct kChunk {
  __device__ __forceinline__ static int first(int g) {
    return OP == BSMM_OP_FP8_MX32_MM ? g : 2 * g;
  }
  __device__ __forceinline__ static int second(int g) {
    return OP == BSMM_OP_FP8_MX32_MM ? g + 4 : 2 * g + 1;
  }
};

// MX with 32-element K blocks: every lane brings the e8m0 scale of its own
// 32 K values (its row or column, K chunk lane / 16), for the B fragment
// byte `selx` of sx and for the A fragment byte `sely` of sy (both constants
// after unrolling).
template <int SY>
__device__ __forceinline__ f32x4 mfma_mx32_x(i32x8 x, i32x8 y, f32x4 c, uint32_t sx, int selx,
                                             uint32_t sy) {
  switch (selx) {
    case 0: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 0, (int)sx, SY, (int)sy);
    case 1: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 1, (int)sx, SY, (int)sy);
    case 2: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 2, (int)sx, SY, (int)sy);
    default: return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, c, 0, 0, 3, (int)sx, SY, (int)sy);
  }
}
__device__ __forceinline__ f32x4 mfma_mx32(i32x8 x, i32x8 y, f32x4 c, uint32_t sx, int selx,
                                           uint32_t sy, int sely) {
  switch (sely) {
    case 0: return mfma_mx32_x<0>(x, y, c, sx, selx, sy);
    case 1: return mfma_mx32_x<1>(x, y, c, sx, selx, sy);
    case 2: return mfma_mx32_x<2>(x, y, c, sx, selx, sy);
    default: return mfma_mx32_x<3>(x, y, c, sx, selx, sy);
  }
}

// Lane part of a tile load's offset, (8 wave + l/8) * ld + 16 * chunk, for
// rows 8q + l/8 with q of parity qpar (see load_row_group); the rest of the
// offset, 8 t NW ld + the K-block byte offset, is wave-uniform.
__device__ __forceinline__ uint32_t lane_base(uint32_t ld, int wave, int lane, int qpar) {
  const int c = (lane & 7) ^ (lane >> 3) ^ qpar;
  return (uint32_t)(wave * 8 + (lane >> 3)) * ld + ((uint32_t)c << 4);
}

__device__ __forceinline__ void load_tile_rows(__amdgpu_buffer_rsrc_t rs, uint8_t* dst,
                                               uint32_t base, uint32_t uniform_off,
                                               bool live) {
  // opaque to the optimiser, which would otherwise keep one loop-invariant
  // base + offset sum per load in a VGPR for the whole K loop
  asm volatile("" : "+s"(uniform_off));
  const uint32_t vo = live ? base + uniform_off : kOob;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, vo, 0, 0, 0);
}

__device__ __forceinline__ void wait_lgkm0() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Store 4 consecutive output values of one row.  The vector stores are
// non-temporal: a round of tile epilogues writes as much as an XCD's L2
// holds, and would otherwise evict the A and B slices the next tiles read.
// E4M3 codes of values clamped to +-448 (the gfx950 conversion rounds to
// nearest even in the default mode); a NaN input is unsupported.
__device__ __forceinline__ uint32_t e4m3x4(const float* y) {
  float c[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = __builtin_amdgcn_fmed3f(y[r], -448.0f, 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return (uint32_t)w;
}

template <int OUT>
__device__ __forceinline__ void store4(uint8_t* base, int64_t e, const float* y,
                                       const int* yi, bool vec, int nvalid) {
  if (OUT == BSMM_E4M3) {
    uint8_t* o = base + e;
    const uint32_t w = e4m3x4(y);
    if (vec && nvalid == 4) __builtin_nontemporal_store(w, (uint32_t*)o);
    else for (int r = 0; r < nvalid; ++r) o[r] = (uint8_t)(w >> (8 * r));
  } else if (OUT == BSMM_BF16) {
    uint16_t* o = (uint16_t*)base + e;
    if (vec && nvalid == 4) {
      u32x2 v;
      v.x = bf16x2(y[0], y[1]);
      v.y = bf16x2(y[2], y[3]);
      __builtin_nontemporal_store(v, (u32x2*)o);
    } else {
      for (int r = 0; r < nvalid; ++r) o[r] = (uint16_t)bf16x2(y[r], 0.f);
    }
  } else if (OUT == BSMM_F32) {
    float* o = (float*)base + e;
    if (vec && nvalid == 4) __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]}, (f32x4*)o);
    else for (int r = 0; r < nvalid; ++r) o[r] = y[r];
  } else {
    int* o = (int*)base + e;
    if (vec && nvalid == 4) __builtin_nontemporal_store(i32x4{yi[0], yi[1], yi[2], yi[3]}, (i32x4*)o);
    else for (int r = 0; r < nvalid; ++r) o[r] = yi[r];
  }
}

// The K loop: acc += the products of K blocks [kb0, kb0 + nkb) of tile
// (g, row0, col0).  Shared by the one-tile-per-workgroup kernel and the
// persistent stream-K kernel.  Every wave of the workgroup must call it with
// the same arguments; it starts with a barrier (a previous call's LDS reads
// must be finished before its loads overwrite the ring) and leaves no loads
// in flight.
template <int OP, int WM, int WN, int RING, bool PK>
struct Mainloop {
  using T = Tile<OP, WM, WN, RING>;
  // int8 with at most four waves per workgroup (one wave per SIMD) runs
  // 32 x 32 x 32 matrix instructions (1.4 times the 16 x 16 x 64 one's rate
  // on gfx950): a wave's 64 x 128 sub-tile is 2 x 4 blocks of 32 x 32 with
  // 16 int32 accumulators per lane each (17-37% faster than 16 x 16 x 64 on
  // int8 8192 x 4096 x 4096 with those kernels).  The eight-wave kernels keep
  // 16 x 16 x 64, which measured 12% faster there than 32 x 32 x 32 with two
  // waves per SIMD.  The fp8 operations run 16 x 16 x 128 tiles (4 x 8 of
  // them, 4 accumulators per lane each).
  static constexpr bool W32 = OP == BSMM_OP_INT8_ROWWISE && WM * WN <= 4;
  using acc_t = std::conditional_t<W32, i32x16, typename OpT<OP>::acc_t>;
  static constexpr int TI = W32 ? 2 : T::TI, TJ = W32 ? 4 : T::TJ;
  // refill slots per wave and K block: one after each 16 x 16 tile's
  // instructions, or after each 32 x 32 x 32 instruction
  static constexpr int NQ = 32;
  static_assert(W32 || T::TI * T::TJ == NQ, "one refill slot per 16 x 16 tile");
  static constexpr int kLoadsPerBlock = T::LA + T::LB;   // per wave
  // shared memory: the ring, or the epilogue's 32-row strips of every wave
  // if those need more (a four-slot ring of 256 x 256 tiles does)
  static constexpr int STAGE = T::NW * 32 * (16 * T::TJ * 4 + 16);
  static constexpr int SMEM = T::LDS > STAGE ? T::LDS : STAGE;

  __device__ __forceinline__ static void run(const KArgs& k, uint8_t* smem, int g,
                                             int row0, int col0, int kb0, int nkb,
                                             acc_t (&acc)[TI][TJ]) {
    constexpr int NSLOT = T::NSLOT, SLOT = T::SLOT;
    const Problem& p = k.p;
    const int lane = threadIdx.x & 63;
    // wave-uniform values live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave / WN, wn = wave % WN;

    // Buffer resources: rows past the launch's end / past N are out of range.
    const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(
        p.a + (int64_t)g * p.a_sg + (int64_t)row0 * p.lda,
        (uint64_t)(k.row_end - row0) * p.lda);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(
        p.b + (int64_t)g * p.b_sg + (int64_t)col0 * p.ldb,
        (uint64_t)(p.N - col0) * p.ldb);
    const __amdgpu_buffer_rsrc_t rdead = make_rsrc(p.b, 0);    // every access out of range

    // Groupwise scale loads (see Tile): per scale load t of this wave, the
    // lane's byte offset into the packed scales at K block 0, the per-block
    // step, and a floor that sends lanes past the slice (and waves with
    // nothing to load) out of range.  Offsets fit 32 bits (checked on the
    // host).
    __amdgpu_buffer_rsrc_t rsc = make_rsrc(k.psa, 0);
    uint32_t gw_base[2] = {0, 0}, gw_step[2] = {0, 0}, gw_floor[2] = {kOob, kOob};
    if constexpr (T::GW) {
      const int KBt = p.K / kBlockK;
      const uint32_t mp = (uint32_t)k.psa_ld, np = (uint32_t)((p.N + 255) / 256 * 256);
      const uint32_t b_region = ((uint32_t)KBt * mp * 4u + 255u) & ~255u;
      rsc = make_rsrc(k.psa, (uint64_t)b_region + (uint64_t)KBt * np * 4u);
  #pragma unroll
      for (int t = 0; t < T::SCL_LOADS; ++t) {
        const int q = t * T::NLD + wave;
        if (q == 0) {
          gw_base[t] = (uint32_t)row0 * 4u + 16u * lane;
          gw_step[t] = mp * 4u;
          gw_floor[t] = lane < T::BM / 4 ? 0u : kOob;
        } else if (q == 1) {
          gw_base[t] = b_region + (uint32_t)col0 * 4u + 16u * lane;
          gw_step[t] = np * 4u;
          gw_floor[t] = lane < T::BN / 4 ? 0u : kOob;
        }
      }
    }
    uint8_t* const scl_base = smem + T::NSLOT * SLOT;

    // Load t of half-stage h (relative to kb0): its K block's A tile (h
    // even, LA loads per wave, the groupwise scale loads last) or B tile (h
    // odd, LB loads), into `slot`.
    auto issue_load = [&](int h, int slot, int t) {
      uint8_t* dst = smem + slot * SLOT;
      const bool live = h < 2 * nkb;
      const uint32_t kbyte = (uint32_t)(kb0 + (h >> 1)) * kBlockK;
      if (h & 1) {
        load_row_group<T::NLD>(rb, rdead, dst, ldb, kbyte, wave, lane, live, t);
      } else if (T::GW && t >= T::LA_ROWS) {
        const int ts = t - T::LA_ROWS;
        const uint32_t floor = live ? gw_floor[ts] : kOob;
        const uint32_t vo = max(gw_base[ts] + (uint32_t)(kb0 + (h >> 1)) * gw_step[ts], floor);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsc, (lds_ptr_t)(scl_base + slot * T::SCL + (ts * T::NLD + wave) * 1024), 16, vo, 0,
            0, 0);
      } else {
        load_row_group<T::NLD>(ra, rdead, dst, lda, kbyte, wave, lane, live, t);
      }
    };
    auto issue_half = [&](int h, int slot) {
      const int n = (h & 1) ? T::LB : T::LA;
      for (int t = 0; t < n; ++t) issue_load(h, slot, t);
    };

    // Per-lane fragment addresses (bytes within a slot): row / column
    // (lane % 16) of the wave's first 16-row tile, chunks 2*(lane/16) + h.
    const int fr = lane & 15;
    // the lane's two 16-byte chunks of its row's 128 K bytes (mx32: the
    // matrix instruction's own K order, see kChunk)
    const int fc0 = kChunk<OP>::first(lane >> 4), fc1 = kChunk<OP>::second(lane >> 4);
    const int a_r = wm * T::WTM + fr;
    const int b_r = wn * T::WTN + fr;
    const int a_off0 = lds_off(a_r, fc0), a_off1 = lds_off(a_r, fc1);
    const int b_off0 = lds_off(b_r, fc0), b_off1 = lds_off(b_r, fc1);

    lds_barrier();     // LDS reads of a previous call are finished
    // Scale pointers.  mx: x_scale bytes of this lane's row in each 16-row
    // tile and the wave's w_scale block.  blockwise: scale_a of the same rows
    // and the wave's scale_b column block.  Rows past the end read a valid row
    // (their results are never stored); so do waves whose columns lie past N.
    const uint8_t* xs_row[TI];
    const uint8_t* ws_blk = nullptr;
    const float* sa_row[TI];
    const float* sb_blk = nullptr;
    // packed scale_a: this lane's four rows are at one 4-byte (mx) or 16-byte
    // (blockwise) position of each K block's row
    const int64_t pk_lane = (int64_t)(row0 + wm * T::WTM) + 4 * fr;
    const int64_t pk_g = PK && OP == BSMM_OP_FP8_MX_BMM ? (int64_t)g * (p.K / kBlockK) : 0;
    if constexpr (OP == BSMM_OP_FP8_BLOCKWISE || OP == BSMM_OP_FP8_MX_BMM) {
      const int nb = min((col0 + wn * T::WTN) / kBlockK, p.N / kBlockK - 1);
      if constexpr (!PK) {
  #pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int m = min(row0 + wm * T::WTM + i * 16 + fr, k.row_end - 1);
          if constexpr (OP == BSMM_OP_FP8_MX_BMM)
            xs_row[i] = (const uint8_t*)p.sa + (int64_t)g * p.sa_sg + (int64_t)m * p.sa_m;
          else
            sa_row[i] = (const float*)p.sa + (int64_t)m * p.sa_m;
        }
      }
      if constexpr (OP == BSMM_OP_FP8_MX_BMM)
        ws_blk = (const uint8_t*)p.sb + (int64_t)g * p.sb_sg + (int64_t)nb * p.sb_n;
      else
        sb_blk = (const float*)p.sb + (int64_t)nb * p.sb_n;
    }

    // mx32: byte offsets (below 2^31, checked on the host) of the lane's K
    // chunk (lane / 16) in the scale rows of its A rows and of its column in
    // each B tile j; rows past M / columns past N read a valid one.  32-bit
    // offsets from the uniform bases take half the registers of pointers.
    uint32_t xs_off[TI], ws_off[TJ];
    // packed (PK): the lane's A word at chunk c sits at c*Mp + a_lane, its
    // B word at c*Np + b_lane of the B region
    const uint8_t* pk_a = (const uint8_t*)k.psa;
    const uint8_t* pk_b = nullptr;
    int64_t a_lane = 0, b_lane = 0, mp = 0, np = 0;
    if constexpr (OP == BSMM_OP_FP8_MX32_MM && PK) {
      const int fq = lane >> 4;
      mp = k.psa_ld;
      np = (p.N + 255) / 256 * 256;    // the pre-pass's column padding
      pk_b = pk_a + (((int64_t)(p.K / 32) * mp + 255) & ~(int64_t)255);
      a_lane = fq * mp + (row0 + wm * T::WTM) + 4 * fr;
      b_lane = fq * np + (col0 + wn * T::WTN) + 8 * fr;
    } else if constexpr (OP == BSMM_OP_FP8_MX32_MM) {
      const int fq = lane >> 4;
  #pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int m = min(row0 + wm * T::WTM + i * 16 + fr, k.row_end - 1);
        xs_off[i] = (uint32_t)((int64_t)m * p.sa_m + fq);
      }
  #pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int n = min(col0 + wn * T::WTN + j * 16 + fr, p.N - 1);
        ws_off[j] = (uint32_t)((int64_t)n * p.sb_n + fq);
      }
    }
    uint32_t wc_cur[TJ / 4], wc_nxt[TJ / 4];     // mx32: B scale bytes, byte j % 4 of word j / 4
  #pragma unroll
    for (int q = 0; q < TJ / 4; ++q) wc_cur[q] = wc_nxt[q] = 0x7F7F7F7Fu;

    // Scale registers of the current K block (cur) and the next one (nxt),
    // loaded at least half a K block before they are used.
    // mx: the four row scale bytes of a lane, byte i for 16-row tile i (the
    // MFMA's scale byte-select picks it)
    uint32_t xs_cur = 0x7F7F7F7Fu, xs_nxt = 0x7F7F7F7Fu;
    int ws_cur = 127, ws_nxt = 127;
    float sa_nxt[TI];
    float sb_nxt = 1.f;
    float sc[TI];     // blockwise: scale product of this lane's row in each 16-row tile;
                      // groupwise: that row's scale
    auto load_scales = [&](int kb) {
      if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
        if constexpr (PK) {
          xs_nxt = *(const uint32_t*)((const uint8_t*)k.psa + (pk_g + kb) * k.psa_ld + pk_lane);
        } else {
          uint32_t v = 0;
  #pragma unroll
          for (int i = 0; i < TI; ++i) v |= (uint32_t)xs_row[i][kb] << (8 * i);
          xs_nxt = v;
        }
        ws_nxt = ws_blk[kb];
      } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
        if constexpr (PK) {
          const f32x4 v = *(const f32x4*)((const float*)k.psa + (int64_t)kb * k.psa_ld + pk_lane);
  #pragma unroll
          for (int i = 0; i < TI; ++i) sa_nxt[i] = v[i];
        } else {
  #pragma unroll
          for (int i = 0; i < TI; ++i) sa_nxt[i] = sa_row[i][(int64_t)kb * p.sa_kb];
        }
        sb_nxt = sb_blk[(int64_t)kb * p.sb_kb];
      } else if constexpr (OP == BSMM_OP_FP8_MX32_MM && PK) {
        xs_nxt = *(const uint32_t*)(pk_a + a_lane + 4 * kb * mp);
        const u32x2 w = *(const u32x2*)(pk_b + b_lane + 4 * kb * np);
        wc_nxt[0] = w.x;
        wc_nxt[1] = w.y;
      } else if constexpr (OP == BSMM_OP_FP8_MX32_MM) {
        const uint8_t* xsb = (const uint8_t*)p.sa + 4 * kb;
        const uint8_t* wsb = (const uint8_t*)p.sb + 4 * kb;
        uint32_t v = 0;
  #pragma unroll
        for (int i = 0; i < TI; ++i) v |= (uint32_t)xsb[xs_off[i]] << (8 * i);
        xs_nxt = v;
  #pragma unroll
        for (int q = 0; q < TJ / 4; ++q) {
          uint32_t w = 0;
  #pragma unroll
          for (int t = 0; t < 4; ++t) w |= (uint32_t)wsb[ws_off[4 * q + t]] << (8 * t);
          wc_nxt[q] = w;
        }
      }
    };
    auto use_scales = [&]() {
      if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
        xs_cur = xs_nxt;
        ws_cur = __builtin_amdgcn_readfirstlane(ws_nxt);   // wave-uniform; taken here, not sunk into the next iteration
      } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
  #pragma unroll
        for (int i = 0; i < TI; ++i) sc[i] = sa_nxt[i] * sb_nxt;
      } else if constexpr (OP == BSMM_OP_FP8_MX32_MM) {
        xs_cur = xs_nxt;
  #pragma unroll
        for (int q = 0; q < TJ / 4; ++q) wc_cur[q] = wc_nxt[q];
      }
    };

    // Fragments of the current K block: all A tiles, and the B tile of the
    // column being computed (bcur); the B tile of column j+1 is read while
    // column j computes.
    const uint8_t* SA = smem;
    const uint8_t* SB = smem;
    i32x8 af[T::TI];
    i32x8 bcur;          // B tile of the current column
    // int8 (32 x 32 x 32): lane l holds row l % 32 of a block and, of each
    // 32-byte K step s, the 16 bytes of LDS chunk 2 s + l / 32 (the K order
    // is the same for both operands, which is all an exact integer sum needs)
    const int r32 = lane & 31, h32 = lane >> 5;
    const int a32 = (wm * T::WTM + r32) << 7, b32 = (wn * T::WTN + r32) << 7;
    int c32[4];
  #pragma unroll
    for (int q = 0; q < 4; ++q) c32[q] = ((2 * q + h32) ^ swz(r32)) << 4;
    i32x4 af32[2][4];    // A blocks 0, 1 of the K block, by K step
    i32x4 bc32[4];       // B block of the current column block, by K step
    auto read_b32 = [&](int bj, i32x4 (&f)[4]) {
  #pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = *(const i32x4*)(SB + b32 + bj * 4096 + c32[q]);
    };
    auto read_b = [&](int j) {
      const i32x4 lo = *(const i32x4*)(SB + b_off0 + j * 2048);
      const i32x4 hi = *(const i32x4*)(SB + b_off1 + j * 2048);
      return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    // groupwise: the current K block's staged scales; this lane's four row
    // scales (packed, one 16-byte read) and the four columns it holds in
    // 16-column tile j (16 bytes at 64 j of the scale_b region)
    const uint8_t* scl = scl_base;
    const int gw_sa = (wm * T::WTM + 4 * fr) * 4;
    const int gw_sb = 1024 + (wn * T::WTN + 4 * (lane >> 4)) * 4;
    auto read_frags = [&](int slot_a, int slot_b) {
      SA = smem + slot_a * SLOT;
      SB = smem + slot_b * SLOT;
      if constexpr (T::GW) {
        scl = scl_base + slot_a * T::SCL;
        const f32x4 v = *(const f32x4*)(scl + gw_sa);
  #pragma unroll
        for (int i = 0; i < TI; ++i) sc[i] = v[i];
      }
      if constexpr (W32) {
        read_b32(0, bc32);
  #pragma unroll
        for (int bi = 0; bi < 2; ++bi)
  #pragma unroll
          for (int q = 0; q < 4; ++q)
            af32[bi][q] = *(const i32x4*)(SA + a32 + bi * 4096 + c32[q]);
      } else {
        bcur = read_b(0);
  #pragma unroll
        for (int i = 0; i < T::TI; ++i) {
          const i32x4 lo = *(const i32x4*)(SA + a_off0 + i * 2048);
          const i32x4 hi = *(const i32x4*)(SA + a_off1 + i * 2048);
          af[i] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
      }
    };

    // Columns [J0, J1) of the current K block.  Blockwise: the fp32 partial
    // of MFMA tile t is folded into its accumulator D steps later, so the
    // multiply-adds never wait on the MFMA that was just issued; the ring is
    // drained at the end of the block.
    constexpr int D = 4;
    static_assert(!T::GW || D == TI, "groupwise folds the previous column's tiles");
    f32x4 ring[D];
    auto columns = [&](auto refill, auto is_loader) {
      constexpr bool LOADER = decltype(is_loader)::value;
      (void)LOADER;
      // groupwise: column scales of the column whose tiles are being folded
      // (the previous one) and of the current one
      f32x4 sbp = f32x4{0, 0, 0, 0}, sbn = sbp;
      // The order is fixed by hard scheduling fences: per column j, its first
      // MFMA, then the reads of B tile j+1 and the column's refill loads, then
      // its other MFMAs, each preceded (blockwise) by the four multiply-adds
      // that fold tile tt-D out of the ring slot the MFMA is about to refill.
      // Left to itself the scheduler hoists the reads and folds each partial
      // right behind its own MFMA, which serialises MFMA and VALU.
      auto tile = [&](int i, int j) {
        const int tt = j * TI + i;
        if constexpr (OP == BSMM_OP_INT8_ROWWISE && !W32) {
          const i32x4 alo = i32x4{af[i][0], af[i][1], af[i][2], af[i][3]};
          const i32x4 ahi = i32x4{af[i][4], af[i][5], af[i][6], af[i][7]};
          const i32x4 blo = i32x4{bcur[0], bcur[1], bcur[2], bcur[3]};
          const i32x4 bhi = i32x4{bcur[4], bcur[5], bcur[6], bcur[7]};
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(blo, alo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bhi, ahi, acc[i][j], 0, 0, 0);
        } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
          if (tt >= D) {
            const int u = tt - D, ui = u % TI, uj = u / TI;
  #pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[ui][uj][r] = __builtin_fmaf(sc[ui], ring[u % D][r], acc[ui][uj][r]);
          }
          ring[tt % D] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bcur, af[i], f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
        } else if constexpr (OP == BSMM_OP_FP8_GROUPWISE) {
          if (tt >= D) {
            const int u = tt - D, ui = u % TI, uj = u / TI;   // uj = j - 1
  #pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[ui][uj][r] = __builtin_fmaf(__fmul_rn(sc[ui], sbp[r]), ring[u % D][r],
                                              acc[ui][uj][r]);
          }
          ring[tt % D] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bcur, af[i], f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
        } else if constexpr (OP == BSMM_OP_FP8_MX32_MM) {
          acc[i][j] = mfma_mx32(bcur, af[i], acc[i][j], wc_cur[j >> 2], j & 3, xs_cur, i);
        } else if constexpr (OP != BSMM_OP_INT8_ROWWISE) {    // mx; scaled_mm with unit scales
          acc[i][j] = mfma_mx(bcur, af[i], acc[i][j], ws_cur, i, xs_cur);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      if constexpr (W32) {
        // int8: per column block bj, its first instruction, then the next
        // column block's B reads and the refills, then the other seven;
        // consecutive instructions alternate between the two accumulators
  #pragma unroll
        for (int bj = 0; bj < TJ; ++bj) {
          i32x4 bn32[4];
  #pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int q = t >> 1, bi = t & 1;
            acc[bi][bj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bc32[q], af32[bi][q],
                                                                acc[bi][bj], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (t == 0) {
              if (bj + 1 < TJ) read_b32(bj + 1, bn32);
              else {
  #pragma unroll
                for (int q2 = 0; q2 < 4; ++q2) bn32[q2] = bc32[q2];
              }
            }
            refill(bj * 8 + t);
            __builtin_amdgcn_sched_barrier(0);
          }
  #pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) bc32[q2] = bn32[q2];
        }
      } else {
  #pragma unroll
      for (int j = 0; j < TJ; ++j) {
        tile(0, j);
        // B tile of column j+1, read while column j computes; the refill
        // loads spread one after every few MFMAs (in bursts they queue in the
        // texture unit and hold up the issuing wave)
        i32x8 bnext = bcur;
        if (j + 1 < TJ) bnext = read_b(j + 1);
        if constexpr (T::GW) sbn = *(const f32x4*)(scl + gw_sb + 64 * j);
        refill(j * TI);
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int i = 1; i < TI; ++i) {
          tile(i, j);
          refill(j * TI + i);
          __builtin_amdgcn_sched_barrier(0);
        }
        bcur = bnext;
        sbp = sbn;
      }
      if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
  #pragma unroll
        for (int u = TI * TJ - D; u < TI * TJ; ++u) {
          const int ui = u % TI, uj = u / TI;
  #pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[ui][uj][r] = __builtin_fmaf(sc[ui], ring[u % D][r], acc[ui][uj][r]);
        }
      } else if constexpr (OP == BSMM_OP_FP8_GROUPWISE) {
  #pragma unroll
        for (int u = TI * TJ - D; u < TI * TJ; ++u) {
          const int ui = u % TI, uj = u / TI;
  #pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[ui][uj][r] = __builtin_fmaf(__fmul_rn(sc[ui], sbp[r]), ring[u % D][r],
                                            acc[ui][uj][r]);
        }
      }
      }
    };

    if (nkb <= 0) return;
    // The loading waves and the others run the same K loop; only the
    // former issue tile loads (the others' vmcnt waits are then trivially
    // met: they have at most their scale loads in flight).
    auto body = [&](auto is_loader) {
      constexpr bool LOADER = decltype(is_loader)::value;
      // Ring schedule.  K block c occupies half-stages 2c (A) and 2c+1 (B) in
      // slots h % NSLOT.  At the top of block c (after the barrier that frees
      // block c-1's two slots) those slots start to be refilled with the next
      // two half-stages, h1 = 2c+NSLOT-2 and h2 = 2c+NSLOT-1, whose loads are
      // spread over the block's columns (h1 first, it is needed first): issued
      // in one burst they would queue in the texture unit and stall the
      // issuing waves' MFMAs.  At the top of block c+1 only h2's loads may
      // still be in flight.
      load_scales(kb0);
      if constexpr (LOADER) {
    #pragma unroll
        for (int h = 0; h < NSLOT - 2; ++h) issue_half(h, h);
      }
      // Scale registers are always consumed in the iteration that loaded them
      // (block c+1's at the end of block c): a loaded value read across the
      // loop's back edge makes the compiler wait for nearly every load in
      // flight, this block's refills included.
      use_scales();
      for (int c = 0; c < nkb; ++c) {
        const int slot_a = (2 * c) % NSLOT;
        const int slot_b = slot_a + 1 == NSLOT ? 0 : slot_a + 1;
        const int h1 = 2 * c + NSLOT - 2, h2 = h1 + 1;
        const int slot1 = h1 % NSLOT;
        const int slot2 = slot1 + 1 == NSLOT ? 0 : slot1 + 1;
        constexpr int L1 = (NSLOT % 2) ? T::LB : T::LA;    // h1 is odd iff NSLOT is odd
        // block c's two half-stages have landed (a wave that issues no tile
        // loads has only its scale loads to wait for, which the compiler does)
        if constexpr (LOADER) wait_vmcnt<T::WAIT>();
        lds_barrier();           // ... for every wave; block c-1's slots are free
        read_frags(slot_a, slot_b);
        // Next block's scales (clamped), issued before this block's refills,
        // taken into use after its last MFMA.
        load_scales(kb0 + min(c + 1, nkb - 1));
        __builtin_amdgcn_sched_barrier(0);
        columns([&](int q) {   // at the block's refill slot q of NQ
          if constexpr (LOADER) {
    #pragma unroll
            for (int u = kLoadsPerBlock * q / NQ; u < kLoadsPerBlock * (q + 1) / NQ; ++u) {
              if (u < L1) issue_load(h1, slot1, u);
              else issue_load(h2, slot2, u - L1);
            }
          }
        }, is_loader);
        use_scales();
      }
      // the last refills were out-of-range loads; let them drain
      if constexpr (LOADER) wait_vmcnt<0>();
    };
    if (wave < T::NLD) body(std::true_type());
    else body(std::false_type());
  }
};

// ---------------------------------------------------------------------------
// Skinny kernel for M <= 16 (decode-sized calls, bound by reading B once).
// One workgroup per 16 output columns of one batch; its four waves split
// the K blocks four ways.  Each wave streams its B fragments (16 rows x 32
// bytes per lane-group, 2 KB per K block) and the A fragment (the <= 16 rows
// of A, zero-filled past M by the buffer range) straight from memory into
// registers, SPF K blocks ahead (a template argument) -- no LDS staging, every B byte is used once
// -- and does one 16 x 16 x 128 MFMA step per K block with the operation's
// scale handling.  The four partial tiles are added in wave order in LDS and
// wave 0 runs the epilogue.
// ---------------------------------------------------------------------------
template <int OP, int OUT, int SPF>
__global__ void __launch_bounds__(256)
skinny_kernel(const KArgs k) {
  using acc_t = typename OpT<OP>::acc_t;
  __shared__ acc_t red[4][kWave];
  const Problem& p = k.p;
  // the kernel arguments in one batch of loads (see the narrow kernel)
  asm volatile("" ::"s"(k.vec_out), "s"(p.M), "s"(p.N), "s"(p.K), "s"(p.a), "s"(p.a_sg),
               "s"(p.lda), "s"(p.b), "s"(p.b_sg), "s"(p.ldb), "s"(p.sa), "s"(p.sa_sg),
               "s"(p.sa_m), "s"(p.sa_kb), "s"(p.sb), "s"(p.sb_sg), "s"(p.sb_n), "s"(p.sb_kb),
               "s"(p.out), "s"(p.o_sg), "s"(p.ldo));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ntiles = (p.N + 15) / 16;
  const int g = blockIdx.x / ntiles;
  const int n0 = (blockIdx.x - g * ntiles) * 16;
  const int KB = p.K / kBlockK;
  const int kbA = wave * KB / 4, kbB = (wave + 1) * KB / 4;
  const int r16 = lane & 15;             // B row n0 + r16, A row r16
  // byte offsets of the lane's two 16-byte chunks within a K block
  const uint32_t co = (uint32_t)kChunk<OP>::first(lane >> 4) * 16;
  const uint32_t co2 = (uint32_t)(kChunk<OP>::second(lane >> 4) - kChunk<OP>::first(lane >> 4)) * 16;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(
      p.b + (int64_t)g * p.b_sg + (int64_t)n0 * p.ldb, (uint64_t)(p.N - n0) * p.ldb);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(
      p.a + (int64_t)g * p.a_sg, (uint64_t)(p.M - 1) * p.lda + (uint64_t)p.K);
  const uint32_t wrow = (uint32_t)r16 * (uint32_t)p.ldb + co;
  const bool xlive = r16 < p.M;
  const uint32_t xrow = (uint32_t)r16 * (uint32_t)p.lda + co;
  const int m_s = min(r16, p.M - 1);     // scale row (rows past M: any valid one)
  const int nb = n0 / kBlockK;

  i32x8 wf[SPF], xf[SPF];
  float s_blk[SPF];                      // blockwise: sa * sb
  int xs_blk[SPF], ws_blk[SPF];          // mx: e8m0 bytes
  auto load = [&](int kb, int slot) {
    const uint32_t kbyte = (uint32_t)kb * kBlockK;
    const i32x4 wl = __builtin_amdgcn_raw_buffer_load_b128(rw, wrow + kbyte, 0, 0);
    const i32x4 wh = __builtin_amdgcn_raw_buffer_load_b128(rw, wrow + kbyte + co2, 0, 0);
    const uint32_t xo = xlive ? xrow + kbyte : kOob;   // rows past M read as zero
    const i32x4 xl = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
    const i32x4 xh = __builtin_amdgcn_raw_buffer_load_b128(rx, xlive ? xo + co2 : kOob, 0, 0);
    wf[slot] = i32x8{wl.x, wl.y, wl.z, wl.w, wh.x, wh.y, wh.z, wh.w};
    xf[slot] = i32x8{xl.x, xl.y, xl.z, xl.w, xh.x, xh.y, xh.z, xh.w};
    if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
      xs_blk[slot] = ((const uint8_t*)p.sa)[(int64_t)g * p.sa_sg + (int64_t)m_s * p.sa_m + kb];
      ws_blk[slot] = ((const uint8_t*)p.sb)[(int64_t)g * p.sb_sg + (int64_t)nb * p.sb_n + kb];
    } else if constexpr (OP == BSMM_OP_FP8_MX32_MM) {
      // the lane's own K chunk: row / column r16, chunk 4 kb + lane / 16
      const int c = 4 * kb + (lane >> 4);
      xs_blk[slot] = ((const uint8_t*)p.sa)[(int64_t)m_s * p.sa_m + c];
      ws_blk[slot] = ((const uint8_t*)p.sb)[(int64_t)min(n0 + r16, p.N - 1) * p.sb_n + c];
    } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
      s_blk[slot] = ((const float*)p.sa)[(int64_t)m_s * p.sa_m + (int64_t)kb * p.sa_kb] *
                    ((const float*)p.sb)[(int64_t)kb * p.sb_kb + (int64_t)nb * p.sb_n];
    }
  };
  acc_t acc = acc_t{0, 0, 0, 0};
  auto step = [&](int slot) {
    const i32x8 w = wf[slot], x = xf[slot];
    if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{w[0], w[1], w[2], w[3]},
                                                   i32x4{x[0], x[1], x[2], x[3]}, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(i32x4{w[4], w[5], w[6], w[7]},
                                                   i32x4{x[4], x[5], x[6], x[7]}, acc, 0, 0, 0);
    } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
      const f32x4 pp = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          w, x, f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(s_blk[slot], pp[r], acc[r]);
    } else if constexpr (OP == BSMM_OP_FP8_MX_BMM || OP == BSMM_OP_FP8_MX32_MM) {
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, acc, 0, 0, 0, ws_blk[slot], 0,
                                                             xs_blk[slot]);
    } else {   // scaled_mm: unit hardware scales, the scales come in the epilogue
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, x, acc, 0, 0, 0, 127, 0, 127);
    }
  };
#pragma unroll
  for (int s0 = 0; s0 < SPF; ++s0)
    if (kbA + s0 < kbB) load(kbA + s0, s0);
  for (int b = kbA; b < kbB; b += SPF) {
#pragma unroll
    for (int s0 = 0; s0 < SPF; ++s0) {
      if (b + s0 < kbB) {
        step(s0);
        if (b + s0 + SPF < kbB) load(b + s0 + SPF, s0);
      }
    }
  }
  // the four waves' partial tiles, added in wave order
  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  acc_t sum = red[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const acc_t v = red[w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) sum[r] += v[r];
  }
  // lane: output row r16, columns n0 + 4 (lane / 16) .. +3
  const int m = r16;
  const int n = n0 + 4 * (lane >> 4);
  const int nvalid = min(4, p.N - n);
  if (m >= p.M || nvalid <= 0) return;
  float y[4];
  int yi[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
      yi[r] = sum[r];
      if constexpr (OUT != BSMM_I32)
        y[r] = __fmul_rn(__fmul_rn((float)sum[r], ((const float*)p.sa)[(int64_t)m * p.sa_m]),
                         ((const float*)p.sb)[(int64_t)min(n + r, p.N - 1) * p.sb_n]);
    } else if constexpr (OP == BSMM_OP_FP8_SCALED_MM) {
      const ScaledEpi epi(p);
      const int nc = min(n + r, p.N - 1);
      y[r] = epi(sum[r], ((const float*)p.sa)[(int64_t)m * p.sa_m],
                 ((const float*)p.sb)[(int64_t)nc * p.sb_n], nc);
    } else {
      y[r] = sum[r];
    }
  }
  store4<OUT>((uint8_t*)p.out, (int64_t)g * p.o_sg + (int64_t)m * p.ldo + n, y, yi,
              k.vec_out != 0, nvalid);
}

// ---------------------------------------------------------------------------
// Narrow kernel for 16 < M <= 128 (decode batches: bound by reading B once).
// One workgroup computes a 128-row x BN-column output tile (BN = 32 or 64)
// over its share of K: the whole of K, or one of S contiguous K ranges whose
// partial tiles the last-arriving workgroup adds (below).  Its four waves
// each own 32 rows (two 16-row MFMA tiles) and all BN / 16 column tiles.
//
// A rows are used by one wave only, so each wave loads its own straight
// into registers in the matrix instruction's operand layout (a lane's 32
// bytes of its row per K block: two 16-byte loads per tile), NS K blocks
// ahead: a ring of NS register sets, indexed by a constant in the loop,
// which is unrolled NS times.  The BN x 128-byte B tile of a K block is
// shared by the four waves: it goes global -> LDS (each wave a quarter, by
// direct-to-LDS loads) into a ring of NS slots.  At block c a wave waits for
// its own loads of block c + 1, the barrier makes every wave's quarter of
// block c + 1 visible and frees block c - 1's slot, block c + NS - 1 is
// requested into the registers and slot block c - 1 used, the B fragments
// of block c + 1 are read, and block c's matrix instructions run on the
// fragments read one step earlier.  (Direct-to-LDS loads alone kept too few
// bytes in flight: A is two thirds or more of each block.)  Steps past the
// end run dead loads (zeros) with neutral scales.
//
// The per-block scales of the workgroup's K range are staged in LDS once,
// before the K loop: mx: the e8m0 byte of each of the 128 rows per K block
// and the tile's B block byte per K block; blockwise: the fp32 row scales
// and the B block scale.
//
// Split K (S > 1): every workgroup stores its fp32 / int32 partial tile in
// a slot of the workspace and then counts itself in the tile's counter with
// a global atomic; the one that brings the count to S adds the S partials in
// ascending K order and runs the epilogue.  No
// workgroup waits for another.  A counter holds the launch's 40-bit tag
// above a 24-bit count; a value with another tag counts as zero, so the
// counters need no clearing between launches.
//
// The grid is G x (N / BN) x S workgroups in the XCD-aware order, so the
// workgroups of one batch share an XCD and read that batch's A from its L2.
// ---------------------------------------------------------------------------
// f(integral_constant<int, i>) for i = B .. E - 1, unrolled
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    static_for<B + 1, E>(f);
  }
}

// Count one arrival in a tile's counter and return the count it makes.  A
// counter holds a launch's 40-bit tag above a 24-bit count; a value with
// another tag (an earlier launch, or whatever the workspace held) counts as
// zero.  The first exchange guesses that this is the last of n arrivals,
// so the last one, whose adds follow, needs a single atomic round trip; a
// wrong guess costs one more, and every failure after it means another
// arrival's exchange succeeded, so at most n + 1 attempts.
__device__ __forceinline__ int count_arrival(uint64_t* ctr, uint64_t tag, int n) {
  uint64_t old = (tag << 24) | (uint64_t)(n - 1);
  uint64_t now;
  do {
    now = (old >> 24) == tag ? old + 1 : ((tag << 24) | 1u);
  } while (!__hip_atomic_compare_exchange_strong(ctr, &old, now, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return (int)(now & 0xFFFFFFu);
}

namespace narrow {
constexpr int BM = 128;
constexpr int SCL = 20480;                       // scale region
template <int BN> struct Cfg {
  static_assert(BN == 32 || BN == 64, "tile widths");
  static constexpr int NS = BN == 32 ? 8 : 6;    // K blocks in the ring
  static constexpr int WB = BN * kBlockK;        // B tile bytes per K block
  static constexpr int BL = BN / 32;             // B loads per wave and K block
  static constexpr int LOADS = 4 + BL;           // per wave and K block: 4 A + B
  static constexpr int TJ = BN / 16;             // 16-column MFMA tiles
  static constexpr int LDS = NS * WB + SCL;
};
// Staged scale rows: KB elements padded to an odd number of 4-byte words.
template <class S> __host__ __device__ constexpr int scale_pitch(int KB) {
  return sizeof(S) == 1 ? ((((KB + 3) >> 2) | 1) << 2) : (KB | 1);
}
// scale region: BM staged rows + the B scale of every K block
template <class S> __host__ __device__ constexpr bool scales_fit(int KB) {
  return (BM * scale_pitch<S>(KB) + KB) * (int)sizeof(S) <= SCL && KB <= 256;
}
template <int OP> constexpr bool supported() {
  return OP == BSMM_OP_FP8_MX_BMM || OP == BSMM_OP_FP8_BLOCKWISE ||
         OP == BSMM_OP_INT8_ROWWISE || OP == BSMM_OP_FP8_SCALED_MM;
}
}  // namespace narrow
constexpr int kNarrowLds = narrow::Cfg<32>::LDS > narrow::Cfg<64>::LDS ? narrow::Cfg<32>::LDS
                                                                        : narrow::Cfg<64>::LDS;

template <int OP, int OUT, int BN>
__global__ void __launch_bounds__(256)
narrow_kernel(const KArgs k) {
  using namespace narrow;
  using C = Cfg<BN>;
  constexpr int NS = C::NS, WB = C::WB, BL = C::BL, LOADS = C::LOADS, TJ = C::TJ;
  using acc_t = typename OpT<OP>::acc_t;
  typedef typename OpT<OP>::elem_t E;
  // LDS sized for the wider tile (one workgroup per CU either way)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNarrowLds];
  static_assert(C::LDS <= kNarrowLds, "LDS");
  const Problem& p = k.p;
  // Every kernel argument read below, loaded in one batch before anything
  // else: left to the compiler, each load waits for the branch or address
  // that first needs it, and the workgroup pays several dependent round
  // trips to the argument buffer before its first tile load.
  asm volatile("" ::"s"(gridDim.x), "s"(k.units), "s"(k.row_begin), "s"(k.row_end),
               "s"(k.vec_out), "s"(k.splits), "s"(k.kb_per_split), "s"(p.N), "s"(p.K), "s"(p.a), "s"(p.a_sg),
               "s"(p.lda), "s"(p.b), "s"(p.b_sg), "s"(p.ldb), "s"(p.sa), "s"(p.sa_sg),
               "s"(p.sa_m), "s"(p.sa_kb), "s"(p.sb), "s"(p.sb_sg), "s"(p.sb_n), "s"(p.sb_kb),
               "s"(p.out), "s"(p.o_sg), "s"(p.ldo));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int KB = p.K / kBlockK;
  const int nblk = p.N / BN;
  const int S = k.splits;
  const int u = first_unit();
  if (u >= k.units) return;
  const int g = u / (nblk * S);
  const int rem = u - g * nblk * S;
  const int jt = rem / S;                      // column tile
  const int ks = rem - jt * S;                 // K range
  const int col0 = jt * BN;
  // K ranges of kb_per_split blocks, the last one shorter (the launch
  // picks S so that none is empty)
  const int kb0 = ks * k.kb_per_split;
  const int nk = min(k.kb_per_split, KB - kb0);
  const int row0 = k.row_begin;
  const int rows = k.row_end - row0;          // <= BM

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(
      p.a + (int64_t)g * p.a_sg + (int64_t)row0 * p.lda, (uint64_t)rows * p.lda);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(
      p.b + (int64_t)g * p.b_sg + (int64_t)col0 * p.ldb, (uint64_t)BN * p.ldb);
  // The workgroup's walk over its K range starts at local block rot and
  // wraps: the tiles of one batch (which share an XCD) spread their requests
  // over K at any moment instead of all asking for the same K block -- with
  // row strides that are multiples of 4 KB those would all land on the same
  // few L2 and HBM channels.  Step c works on local block kbo(c), global
  // block kb0 + kbo(c).
  const int rot = (int)((uint32_t)jt % (uint32_t)nk);
  auto kbo = [&](int c) { const int t = c + rot; return t >= nk ? t - nk : t; };
  const __amdgpu_buffer_rsrc_t rdead = make_rsrc(p.b, 0);
  const int fr = lane & 15, fq = lane >> 4;
  const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb;
  // A: lane's row 32 wave + 16 i + f, bytes [32 fq, 32 fq + 32) of the block
  // (rows past the launch fall outside the resource: zeros)
  uint32_t a_vo[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_vo[i] = (uint32_t)(32 * wave + 16 * i + fr) * lda + 32u * fq;
  // B: this wave's quarter, BL groups of 8 rows; group q = BL wave + t holds
  // rows 8 q + lane / 8, chunk (lane % 8) ^ swz, at slot bytes 1024 q
  // (a fixed size: with a BN-dependent one the host-side pass drops the
  // kernel template, with no stub and no error, where a lambda hands an
  // element to the buffer builtin)
  uint32_t b_vo[2];
#pragma unroll
  for (int t = 0; t < BL; ++t) {
    const int b_row = (BL * wave + t) * 8 + (lane >> 3);
    b_vo[t] = (uint32_t)b_row * ldb + ((uint32_t)((lane & 7) ^ swz(b_row)) << 4);
  }
  i32x4 xr[NS][2][2];            // A fragments of the NS blocks in flight
  // step b's loads into register set / B slot s (a constant)
  auto issue = [&](int b, auto s_c) {
    constexpr int s = decltype(s_c)::value;
    const bool live = b < nk;
    const __amdgpu_buffer_rsrc_t rA = live ? ra : rdead;
    const int kbyte = (live ? kb0 + kbo(b) : 0) * kBlockK;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      xr[s][i][0] = __builtin_amdgcn_raw_buffer_load_b128(rA, a_vo[i], kbyte, 0);
      xr[s][i][1] = __builtin_amdgcn_raw_buffer_load_b128(rA, a_vo[i] + 16, kbyte, 0);
    }
#pragma unroll
    for (int t = 0; t < BL; ++t) {
      const lds_ptr_t l = (lds_ptr_t)(uintptr_t)(uint32_t)(uintptr_t)(
          smem + s * WB + (BL * wave + t) * 1024);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rb : rdead, l, 16, b_vo[t], kbyte, 0, 0);
    }
  };

  // The scales of the K range go to the scale region once: A's as [row]
  // [local K block] with a row pitch of an odd number of 4-byte words (the
  // loop's reads of 16 rows then fall in 16 different banks), followed by
  // the tile's B scale of every local K block.  Each wave stages its own 32
  // rows (only it reads them); element e of a wave is row e >> lkb, local
  // K block e & (KBP - 1) for KBP = 2^lkb >= nk, so a load instruction
  // covers whole runs of a row's contiguous bytes, and a row past the launch
  // reads the last valid row.  Rounds of CH loads per lane; the last round's
  // loads and the B scales' are issued ahead of the prologue's tile loads
  // (the empty asm keeps them there) and written after them.
  uint8_t* const scl = smem + NS * WB;
  constexpr int CH = 16;
  using SC = typename std::conditional<OP == BSMM_OP_FP8_BLOCKWISE, float, uint8_t>::type;
  constexpr bool SCALES = OP == BSMM_OP_FP8_MX_BMM || OP == BSMM_OP_FP8_BLOCKWISE;
  const int pitch = scale_pitch<SC>(nk);         // elements per staged row
  const int lkb = nk <= 1 ? 0 : 32 - __builtin_clz(nk - 1);
  const int n_e = SCALES ? 32 << lkb : 0;        // elements per wave, padding included
  auto x_load = [&](int e) -> SC {
    const int r = e >> lkb, kb = e & ((1 << lkb) - 1);
    if (e >= n_e || kb >= nk) return SC(0);
    const int64_t mm = row0 + min(32 * wave + r, rows - 1);
    if constexpr (OP == BSMM_OP_FP8_MX_BMM)
      return ((const uint8_t*)p.sa)[(int64_t)g * p.sa_sg + mm * p.sa_m + kb0 + kb];
    else
      return ((const float*)p.sa)[mm * p.sa_m + (int64_t)(kb0 + kb) * p.sa_kb];
  };
  auto x_store = [&](int e, SC v) {
    const int r = e >> lkb, kb = e & ((1 << lkb) - 1);
    if (e < n_e && kb < nk) ((SC*)scl)[(32 * wave + r) * pitch + kb] = v;
  };
  SC sv[CH];
  SC wv = SC(0);
  int e_last = 0;
  if constexpr (SCALES) {
    for (; e_last + 64 * CH < n_e; e_last += 64 * CH) {
#pragma unroll
      for (int i = 0; i < CH; ++i) sv[i] = x_load(e_last + 64 * i + lane);
#pragma unroll
      for (int i = 0; i < CH; ++i) x_store(e_last + 64 * i + lane, sv[i]);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) sv[i] = x_load(e_last + 64 * i + lane);
    const int kb = threadIdx.x;
    if (kb < nk) {
      if constexpr (OP == BSMM_OP_FP8_MX_BMM)
        wv = ((const uint8_t*)p.sb)[(int64_t)g * p.sb_sg + (int64_t)(col0 / kBlockK) * p.sb_n +
                                    kb0 + kb];
      else
        wv = ((const float*)p.sb)[(int64_t)(kb0 + kb) * p.sb_kb + (int64_t)(col0 / kBlockK) * p.sb_n];
    }
    asm volatile("" ::: "memory");
  }

  // prologue: steps 0 .. NS-1 into every register set and slot
  static_for<0, NS>([&](auto i) { issue(decltype(i)::value, i); });

  if constexpr (SCALES) {
#pragma unroll
    for (int i = 0; i < CH; ++i) x_store(e_last + 64 * i + lane, sv[i]);
    if ((int)threadIdx.x < nk) ((SC*)scl)[BM * pitch + threadIdx.x] = wv;
  }
  wait_lgkm0();                            // this wave's scale writes

  acc_t acc[2][TJ];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = acc_t{0, 0, 0, 0};
  // B fragments: rows 16 j + f, chunks 2 fq and 2 fq + 1
  int b_off[TJ][2];
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    b_off[j][0] = lds_off(16 * j + fr, 2 * fq);
    b_off[j][1] = lds_off(16 * j + fr, 2 * fq + 1);
  }
  // B fragments and scales of a step, into the set of the step's parity
  struct BFrags {
    i32x8 b[TJ];
    uint32_t xs;       // mx: the lane's two row scale bytes (byte i: A tile i)
    int ws;            // mx: the B block's scale byte
    float sa[2], sb;   // blockwise
  };
  BFrags bq[2];
  auto read_b = [&](int c, auto s_c, BFrags& f) {
    constexpr int s = decltype(s_c)::value;
    const uint8_t* sb_ = smem + s * WB;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const i32x4 lo = *(const i32x4*)(sb_ + b_off[j][0]);
      const i32x4 hi = *(const i32x4*)(sb_ + b_off[j][1]);
      f.b[j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    // steps past the end: neutral scales (their products are zeros); the
    // reads go to the last block and are selected away, so the step stays
    // one straight-line block that the fences can pin
    const bool live = c < nk;
    const int cl = kbo(min(c, nk - 1));
    f.xs = 0x7F7Fu;
    f.ws = 127;
    f.sa[0] = f.sa[1] = f.sb = 0.f;
    if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
      const uint8_t* xr0 = scl + (32 * wave + fr) * pitch + cl;
      const uint32_t xs = (uint32_t)xr0[0] | ((uint32_t)xr0[16 * pitch] << 8);
      const int ws = scl[BM * pitch + cl];
      f.xs = live ? xs : 0x7F7Fu;
      f.ws = live ? ws : 127;
    } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
      const float* sf = (const float*)scl;
      const float* xr0 = sf + (32 * wave + fr) * pitch + cl;
      const float v0 = xr0[0], v1 = xr0[16 * pitch];
      const float sb = sf[BM * pitch + cl];
      f.sa[0] = live ? v0 : 0.f;
      f.sa[1] = live ? v1 : 0.f;
      f.sb = live ? sb : 0.f;
    }
  };
  auto compute = [&](auto s_c, const BFrags& f) {
    constexpr int s = decltype(s_c)::value;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const i32x4 lo = xr[s][i][0], hi = xr[s][i][1];
      const i32x8 af = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              i32x4{f.b[j][0], f.b[j][1], f.b[j][2], f.b[j][3]}, lo, acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
              i32x4{f.b[j][4], f.b[j][5], f.b[j][6], f.b[j][7]}, hi, acc[i][j], 0, 0, 0);
        } else if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
          acc[i][j] = mfma_mx(f.b[j], af, acc[i][j], __builtin_amdgcn_readfirstlane(f.ws), i,
                              f.xs);
        } else if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) {
          const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              f.b[j], af, f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
          const float sc = f.sa[i] * f.sb;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(sc, part[r], acc[i][j][r]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              f.b[j], af, acc[i][j], 0, 0, 0, 127, 0, 127);
        }
      }
    }
  };
  // Step 0's B fragments before the loop: every wave's loads of step 0
  // landed, its scale writes done, then the barrier.
  wait_vmcnt<(NS - 1) * LOADS>();
  wait_lgkm0();
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  read_b(0, std::integral_constant<int, 0>(), bq[0]);
  // Step c: wait for this wave's loads of step c + 1 (the later steps in
  // flight may stay outstanding: NS - 2 at c = 0, then NS - 3), the barrier
  // (every wave's B quarter of step c + 1 visible; step c - 1's slot no
  // longer read, its fragments were read in step c - 2), the refill of step
  // c - 1's register set and slot with step c + NS - 1, the B fragments of
  // step c + 1, and step c's matrix instructions on fragments read in step
  // c - 1.  The fences keep every LDS read after its barrier.
  auto step = [&](int c, auto s_c, auto first_c) {
    constexpr int s = decltype(s_c)::value;
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr int sp = (s + NS - 1) % NS, sn = (s + 1) % NS;
    if constexpr (FIRST) wait_vmcnt<(NS - 2) * LOADS>();
    else wait_vmcnt<(NS - 3) * LOADS>();
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!FIRST) issue(c + NS - 1, std::integral_constant<int, sp>());
    read_b(c + 1, std::integral_constant<int, sn>(), bq[(s + 1) & 1]);
    compute(s_c, bq[s & 1]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // steps in groups of NS (register set s = c % NS); the last group's steps
  // past nk are zeros (dead loads) with neutral scales
  static_assert(NS % 2 == 0, "B fragment sets alternate with the step's parity");
  step(0, std::integral_constant<int, 0>(), std::true_type());
  static_for<1, NS>([&](auto i) { step(decltype(i)::value, i, std::false_type()); });
  for (int c0 = NS; c0 < nk; c0 += NS)
    static_for<0, NS>([&](auto i) { step(c0 + decltype(i)::value, i, std::false_type()); });
  wait_vmcnt<0>();                       // the last refills were out-of-range loads

  if (S > 1) {
    // Publish this K range's partial in slot (tile, ks): the lane's 16
    // bytes of MFMA tile (wave, i, j) at ((wave * 2 + i) * TJ + j) * 1024 +
    // 16 lane, so each store instruction writes 1 KB of whole lines, and
    // the last arriver's lanes read the same positions of every slot.  The
    // partials and the counter are touched only through agent-scope
    // (sc1) accesses: those stores write through to the device's coherence
    // point and those loads read from it, and a store has reached it once
    // the wave's vmcnt wait covers it.  So the waits below order the
    // partials before the count (and the count before the reads) without a
    // fence's L2 write-back and invalidate, which serialise across an
    // XCD's workgroups and cost more than the K loop.
    constexpr int SLOT = BM * BN * 4;
    constexpr int SC1 = 16;                    // buffer cache policy: agent scope
    const int tile = g * nblk + jt;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc((uint8_t*)k.ws + (size_t)tile * S * SLOT,
                                                (uint64_t)S * SLOT);
    uint64_t* const counters = (uint64_t*)((uint8_t*)k.ws + (size_t)k.units * SLOT);
    auto pos = [&](int i, int j) { return (uint32_t)(((wave * 2 + i) * TJ + j) * 1024 + 16 * lane); };
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, acc[i][j]), rw, pos(i, j),
                                               ks * SLOT, SC1);
    wait_vmcnt<0>();     // this wave's partial has reached the coherence point
    __syncthreads();     // ... every wave's; the ring is idle
    int* const last_arrival = (int*)smem;
    if (threadIdx.x == 0)
      *last_arrival = count_arrival(counters + tile, k.epoch & ((1ull << 40) - 1), S) == S;
    __syncthreads();
    if (!*last_arrival) return;
    if (S == 2) {
      // two partials: this workgroup's, in registers, plus the other one
      // (the sum of two does not depend on which of them adds)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          const acc_t v = __builtin_bit_cast(
              acc_t, __builtin_amdgcn_raw_buffer_load_b128(rw, pos(i, j), (1 - ks) * SLOT, SC1));
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] + v[r];
        }
    } else {
    // the S partials in ascending K order, this workgroup's own read back
    // like the others (choosing between it and a load would put the
    // accumulators in scratch memory)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        acc_t sum = __builtin_bit_cast(acc_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rw, pos(i, j), 0, SC1));
        for (int s2 = 1; s2 < S; ++s2) {
          const acc_t v = __builtin_bit_cast(
              acc_t, __builtin_amdgcn_raw_buffer_load_b128(rw, pos(i, j), s2 * SLOT, SC1));
#pragma unroll
          for (int r = 0; r < 4; ++r) sum[r] += v[r];
        }
        acc[i][j] = sum;
      }
    }
  }

  // epilogue: lane holds row 32 wave + 16 i + f, columns 16 j + 4 fq .. + 3
  const bool vec = k.vec_out != 0;
  [[maybe_unused]] const ScaledEpi epi(p);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int mr = 32 * wave + 16 * i + fr;
    if (mr >= rows) continue;
    const int m = row0 + mr;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int n = col0 + 16 * j + 4 * fq;
      float y[4];
      int yi[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
          yi[r] = acc[i][j][r];
          if constexpr (OUT != BSMM_I32)
            y[r] = __fmul_rn(__fmul_rn((float)acc[i][j][r], ((const float*)p.sa)[(int64_t)m * p.sa_m]),
                             ((const float*)p.sb)[(int64_t)(n + r) * p.sb_n]);
        } else if constexpr (OP == BSMM_OP_FP8_SCALED_MM) {
          y[r] = epi(acc[i][j][r], ((const float*)p.sa)[(int64_t)m * p.sa_m],
                     ((const float*)p.sb)[(int64_t)(n + r) * p.sb_n], n + r);
        } else {
          y[r] = acc[i][j][r];
        }
      }
      store4<OUT>((uint8_t*)p.out, (int64_t)g * p.o_sg + (int64_t)m * p.ldo + n, y, yi, vec, 4);
    }
  }
}

// Epilogue through LDS.  Stored straight from the MFMA layout, a wave's
// store instruction writes 16 rows x 32 or 64 bytes -- sixteen partial cache
// lines -- and a round of 256 tiles took ~13 us of pure write time.  Here
// each wave stages 32 rows x (16 TJ) columns of 4-byte values in LDS (idle
// after the K loop; rows padded by 16 bytes), reads them back as contiguous
// 4-element groups and stores whole row segments.  int8: the row scale is
// applied while staging, the column scale after reading back (the order
// (f32(acc) * sa) * sb is unchanged).  PARTIAL: split-K partials (int32 /
// fp32) into the workspace [splits][G][rows][N] instead of the output.
// Epilogue destinations (MODE):
//   kOut     the output (int8: both scales applied);
//   kSplitK  split-K partials (int32 / fp32) into the workspace
//            [splits][G][rows][N];
//   kSlot    a stream-K partial: the whole BM x BN tile, row-major, into
//            the slot `sl.base` (int32 / fp32);
//   kOutAdd  the output of a stream-K tile whose `sl.count` K segments sit
//            in slots sl.slot(0) .. sl.slot(count - 1), in K order; segment
//            sl.own is this workgroup's, taken from its registers.  The sum
//            runs in K order whichever segment this is, so the result does
//            not depend on which workgroup adds (int8: the raw sums are
//            staged and both scales applied after the adds, so the
//            operations are those of kOut).
enum { kOut = 0, kSplitK = 1, kSlot = 2, kOutAdd = 3 };
struct SlotRef {
  void* base = nullptr;       // slot 0
  int64_t stride = 0;         // elements per slot
  // kOutAdd: the tile's segments are those of workgroups first .. first +
  // count - 1.  A workgroup's slot 2w holds the first segment of its K
  // range, slot 2w + 1 the segment that starts a tile at the end of its
  // range; only the tile's first segment can be of the second kind.
  int first = 0, count = 0, own = 0, first_odd = 0;
  __device__ __forceinline__ int64_t slot(int j) const {
    return 2 * (int64_t)(first + j) + (j == 0 ? first_odd : 0);
  }
};

template <int OP, int OUT, int NW, int WN, int MODE, int BM, int BN, int TI, int TJ,
          class acc_t>
__device__ __forceinline__ void store_staged(const KArgs& k, int s, int g, int row0, int col0,
                                             const acc_t (&acc)[TI][TJ], uint8_t* smem,
                                             const SlotRef& sl = SlotRef()) {
  // accumulator blocks: 16 x 16 (4 values per lane: row l % 16, columns
  // 4 (l / 16) .. + 3) or, for int8, 32 x 32 (16 values per lane: row l % 32,
  // columns 8 q + 4 (l / 32) .. + 3 for q = 0 .. 3)
  constexpr bool W32 = sizeof(acc_t) == 64;
  constexpr int TW = W32 ? 32 : 16;              // rows and columns of a block
  constexpr int ROWS = 32;                       // staged rows per pass
  constexpr int WCOLS = TW * TJ;                 // the wave's columns
  constexpr int PITCH = WCOLS * 4 + 16;          // bytes per staged row
  constexpr int PER_ROW = WCOLS / 4;             // 4-element groups per row
  constexpr int GROUPS = ROWS * PER_ROW;         // per pass
  constexpr int NPASS = TW * TI / ROWS;
  constexpr bool PARTIAL = MODE == kSplitK || MODE == kSlot;
  static_assert((TW * TI) % ROWS == 0 && GROUPS % kWave == 0, "staging layout");
  typedef typename OpT<OP>::elem_t E;
  const Problem& p = k.p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int wm = wave / WN, wn = wave % WN;
  uint8_t* st = smem + wave * (ROWS * PITCH);
  const int fr = lane & 15, fq = lane >> 4;
  const int wrow0 = row0 + wm * TW * TI, wcol0 = col0 + wn * WCOLS;
  const bool vec = k.vec_out != 0;
  uint8_t* obase;
  int64_t og, ldo;
  if constexpr (MODE == kSplitK) {
    const int rows = k.row_end - k.row_begin;
    obase = (uint8_t*)((E*)k.ws + ((int64_t)s * p.G + g) * (int64_t)rows * p.N);
    og = -(int64_t)k.row_begin * p.N;
    ldo = p.N;
  } else if constexpr (MODE == kSlot) {
    obase = (uint8_t*)sl.base;
    og = -(int64_t)row0 * BN - col0;
    ldo = BN;
  } else {
    obase = (uint8_t*)p.out;
    og = (int64_t)g * p.o_sg;
    ldo = p.ldo;
  }
  // int8 scales: the row scale while staging (kOut), or both after the
  // slot adds (kOutAdd)
  constexpr bool SCALE = OP == BSMM_OP_INT8_ROWWISE && OUT != BSMM_I32 && !PARTIAL;
  constexpr bool SCALE_A_STAGED = SCALE && MODE == kOut;
  // fp8 scaled_mm: both scales, the bias and the result scale after the
  // (stream-K) adds
  constexpr bool SCALED = OP == BSMM_OP_FP8_SCALED_MM && !PARTIAL;
  const bool sb_vec = (SCALE || SCALED) && p.sb_n == 1 && (((uintptr_t)p.sb) & 15u) == 0;
  // the column scales of the lane's four columns, the same in every group
  // the lane stores (group q of a pass covers row q kWave / PER_ROW + lane /
  // PER_ROW and columns 4 (lane % PER_ROW) ..), loaded once per tile
  static_assert(kWave % PER_ROW == 0, "a lane's groups share their columns");
  float sb_l[4] = {1.f, 1.f, 1.f, 1.f};
  if constexpr (SCALE || SCALED) {
    const int n_l = wcol0 + 4 * (lane % PER_ROW);
    if (sb_vec && p.N - n_l >= 4) {
      const f32x4 t = *(const f32x4*)((const float*)p.sb + n_l);
      sb_l[0] = t[0]; sb_l[1] = t[1]; sb_l[2] = t[2]; sb_l[3] = t[3];
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sb_l[c] = ((const float*)p.sb)[(int64_t)max(0, min(n_l + c, p.N - 1)) * p.sb_n];
    }
  }
  [[maybe_unused]] const ScaledEpi epi(p);
  lds_barrier();     // every wave's K-loop reads of LDS are done
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    if constexpr (W32) {
      // block row `pass`: the lane's row l % 32, four runs of four columns
      // per 32-column block
      const int r32 = lane & 31, h32 = lane >> 5;
      float sa_m = 1.f;
      if constexpr (SCALE_A_STAGED)
        sa_m = ((const float*)p.sa)[(int64_t)min(wrow0 + 32 * pass + r32, k.row_end - 1) * p.sa_m];
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          i32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (SCALE_A_STAGED)
              v[r] = __float_as_int(__fmul_rn((float)acc[pass][j][4 * q + r], sa_m));
            else
              v[r] = acc[pass][j][4 * q + r];
          }
          *(i32x4*)(st + r32 * PITCH + (32 * j + 8 * q + 4 * h32) * 4) = v;
        }
    } else {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * pass + ii;
      float sa_m = 1.f;
      if constexpr (SCALE_A_STAGED)
        sa_m = ((const float*)p.sa)[(int64_t)min(wrow0 + 16 * i + fr, k.row_end - 1) * p.sa_m];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        i32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (SCALE_A_STAGED)
            v[r] = __float_as_int(__fmul_rn((float)acc[i][j][r], sa_m));
          else if constexpr (OP == BSMM_OP_INT8_ROWWISE)
            v[r] = acc[i][j][r];
          else
            v[r] = __float_as_int(acc[i][j][r]);
        }
        *(i32x4*)(st + (16 * ii + fr) * PITCH + (16 * j + 4 * fq) * 4) = v;
      }
    }
    }
#pragma unroll
    for (int q = 0; q < GROUPS / kWave; ++q) {
      const int gi = q * kWave + lane;
      const int r = gi / PER_ROW, cg = gi % PER_ROW;
      i32x4 v = *(const i32x4*)(st + r * PITCH + cg * 16);
      const int m = wrow0 + ROWS * pass + r;
      const int n = wcol0 + 4 * cg;
      // a slot holds the whole tile: every group is stored
      const int nvalid = MODE == kSlot ? 4 : min(4, p.N - n);
      if (MODE != kSlot && (m >= k.row_end || nvalid <= 0)) continue;
      const int64_t e = og + (int64_t)m * ldo + n;
      if constexpr (MODE == kOutAdd) {
        const int64_t off = (int64_t)(m - row0) * BN + (n - col0);
        const i32x4 mine = v;
        for (int q2 = 0; q2 < sl.count; ++q2) {
          i32x4 t = mine;
          if (q2 != sl.own) {
            // agent-scope (sc1) loads: they read the partials from the
            // device's coherence point, where their agent-scope stores put
            // them (every slot lies within 4 GB of slot 0)
            t = __builtin_amdgcn_raw_buffer_load_b128(
                make_rsrc(sl.base, 0xFFFFFFF0ull),
                (uint32_t)((sl.slot(q2) * sl.stride + off) * (int64_t)sizeof(E)), 0, 16);
          }
          if (q2 == 0) {
            v = t;
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if constexpr (OP == BSMM_OP_INT8_ROWWISE) v[c] += t[c];
              else v[c] = __float_as_int(__int_as_float(v[c]) + __int_as_float(t[c]));
            }
          }
        }
      }
      float y[4];
      int yi[4];
      if constexpr (SCALED) {
        const float* sb = sb_l;
        const float sa_m = ((const float*)p.sa)[(int64_t)m * p.sa_m];
#pragma unroll
        for (int c = 0; c < 4; ++c) y[c] = epi(__int_as_float(v[c]), sa_m, sb[c], min(n + c, p.N - 1));
      } else if constexpr (SCALE) {
        const float* sb = sb_l;
        if constexpr (SCALE_A_STAGED) {
#pragma unroll
          for (int c = 0; c < 4; ++c) y[c] = __fmul_rn(__int_as_float(v[c]), sb[c]);
        } else {
          const float sa_m = ((const float*)p.sa)[(int64_t)m * p.sa_m];
#pragma unroll
          for (int c = 0; c < 4; ++c) y[c] = __fmul_rn(__fmul_rn((float)v[c], sa_m), sb[c]);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          y[c] = __int_as_float(v[c]);
          yi[c] = v[c];
        }
      }
      if constexpr (MODE == kSlot) {
        // agent-scope (sc1) stores: written through to the device's
        // coherence point (the stream-K protocol orders them with vmcnt
        // waits alone); the staged values are the partial's bits
        __builtin_amdgcn_raw_buffer_store_b128(v, make_rsrc(obase, (uint64_t)BM * BN * sizeof(E)),
                                               (uint32_t)(e * (int64_t)sizeof(E)), 0, 16);
      } else if constexpr (PARTIAL) {
        store4<OP == BSMM_OP_INT8_ROWWISE ? BSMM_I32 : BSMM_F32>(obase, e, y, yi, vec, nvalid);
      } else {
        store4<OUT>(obase, e, y, yi, vec, nvalid);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide-wave K loop: four waves (one per SIMD), a 256 x 256 tile, each wave a
// 128 x 128 sub-tile = 8 x 8 MFMA tiles whose 256 accumulator registers the
// compiler keeps in AGPRs.  For the paths without per-element work in the
// K loop (int8, mx).
//
// Per K block and wave: 64 MFMA tiles in row order (A tile i with B tiles
// 0..7), 16 direct-to-LDS loads and 32 fragment reads, each of them for the
// NEXT block and into the register it replaces: the next block's A tile i
// after row i (a whole block ahead of its use), its B tile j right after
// the last MFMA that uses B tile j (row 7; eight MFMAs ahead of its first
// use in row 0).  The only synchronisation is one barrier per block,
// placed after row 0.
//
// LDS ring of five 32 KB half-stages, half-stage h (2c: A of block c,
// 2c+1: B) in slot h % 5.  Barrier #c (after row 0 of block c) certifies
// that block c+1 has landed (it is read during block c) and that every
// wave has finished reading block c (read during block c-1): block c's two
// slots are refilled with half-stages 2c+5 (block c+2's B, rows 1..4) and
// 2c+6 (block c+3's A, rows 5..7).  At barrier #c only half-stage 2c+4's
// loads (block c+2's A, issued during block c-1) may still be in flight.
// ---------------------------------------------------------------------------
template <int OP, bool PK>
struct Mainloop4 {
  static constexpr int NW = 4, WN = 2, TI = 8, TJ = 8, WTM = 128, WTN = 128;
  static constexpr int BM = 256, BN = 256, NT = NW * kWave;
  static constexpr int SLOT = BM * kBlockK, NSLOT = 5, LDS = NSLOT * SLOT;
  static constexpr int LA = BM / 8 / NW, LB = BN / 8 / NW;    // loads per half-stage per wave
  using acc_t = typename OpT<OP>::acc_t;
  static_assert(OP != BSMM_OP_FP8_BLOCKWISE, "blockwise needs its accumulators in VGPRs");

  __device__ __forceinline__ static void run(const KArgs& k, uint8_t* smem, int g,
                                             int row0, int col0, int kb0, int nkb,
                                             acc_t (&acc)[TI][TJ]) {
    const Problem& p = k.p;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave / WN, wn = wave % WN;
    const uint32_t lda = (uint32_t)p.lda, ldb = (uint32_t)p.ldb;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(
        p.a + (int64_t)g * p.a_sg + (int64_t)row0 * p.lda,
        (uint64_t)(k.row_end - row0) * p.lda);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(
        p.b + (int64_t)g * p.b_sg + (int64_t)col0 * p.ldb,
        (uint64_t)(p.N - col0) * p.ldb);
    // lane part of the load offsets (the chunk swizzle of row 8q + l/8
    // depends on q's parity, which is the wave's for four waves)
    const uint32_t base_a = lane_base(lda, wave, lane, wave & 1);
    const uint32_t base_b = lane_base(ldb, wave, lane, wave & 1);
    auto issue_load = [&](int h, int t) {
      uint8_t* dst = smem + (h % NSLOT) * SLOT + (t * NW + wave) * 1024;
      const bool live = h < 2 * nkb;
      const uint32_t kbyte = (uint32_t)(kb0 + (h >> 1)) * kBlockK;
      if (h & 1) load_tile_rows(rb, dst, base_b, (uint32_t)(t * NW * 8) * ldb + kbyte, live);
      else load_tile_rows(ra, dst, base_a, (uint32_t)(t * NW * 8) * lda + kbyte, live);
    };

    const int fr = lane & 15;
    const int fc = (lane >> 4) * 2;
    const int a_r = wm * WTM + fr, b_r = wn * WTN + fr;
    const int a_off0 = lds_off(a_r, fc), a_off1 = lds_off(a_r, fc + 1);
    const int b_off0 = lds_off(b_r, fc), b_off1 = lds_off(b_r, fc + 1);
    auto frag = [&](int h, int off0, int off1, int t) {
      const uint8_t* S = smem + (h % NSLOT) * SLOT;
      const i32x4 lo = *(const i32x4*)(S + off0 + t * 2048);
      const i32x4 hi = *(const i32x4*)(S + off1 + t * 2048);
      return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };

    lds_barrier();     // LDS reads of a previous call are finished
    // mx scales: the lane's rows f + 16 i, i = 0..7, as two packed dwords
    // (byte i % 4 of word i / 4), and the wave's w_scale block
    const uint8_t* xs_row[TI];
    const uint8_t* ws_blk = nullptr;
    const int64_t pk_lane = (int64_t)(row0 + wm * WTM) + 4 * fr;
    const int64_t pk_g = PK ? (int64_t)g * (p.K / kBlockK) : 0;
    if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
      const int nb = min((col0 + wn * WTN) / kBlockK, p.N / kBlockK - 1);
      ws_blk = (const uint8_t*)p.sb + (int64_t)g * p.sb_sg + (int64_t)nb * p.sb_n;
      if constexpr (!PK) {
  #pragma unroll
        for (int i = 0; i < TI; ++i) {
          const int m = min(row0 + wm * WTM + i * 16 + fr, k.row_end - 1);
          xs_row[i] = (const uint8_t*)p.sa + (int64_t)g * p.sa_sg + (int64_t)m * p.sa_m;
        }
      }
    }
    uint32_t xs_cur[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu}, xs_nxt[2] = {0x7F7F7F7Fu, 0x7F7F7F7Fu};
    int ws_cur = 127, ws_nxt = 127;
    auto load_scales = [&](int kb) {
      if constexpr (OP == BSMM_OP_FP8_MX_BMM) {
        if constexpr (PK) {
          const uint8_t* q = (const uint8_t*)k.psa + (pk_g + kb) * k.psa_ld + pk_lane;
          xs_nxt[0] = *(const uint32_t*)q;
          xs_nxt[1] = *(const uint32_t*)(q + 64);
        } else {
  #pragma unroll
          for (int w = 0; w < 2; ++w) {
            uint32_t v = 0;
  #pragma unroll
            for (int i = 0; i < 4; ++i) v |= (uint32_t)xs_row[4 * w + i][kb] << (8 * i);
            xs_nxt[w] = v;
          }
        }
        ws_nxt = ws_blk[kb];
      }
    };
    auto use_scales = [&]() {
      xs_cur[0] = xs_nxt[0];
      xs_cur[1] = xs_nxt[1];
      ws_cur = __builtin_amdgcn_readfirstlane(ws_nxt);   // wave-uniform; taken here, not sunk into the next iteration
    };

    if (nkb <= 0) return;
    i32x8 af[TI], bf[TJ];
    // prologue: blocks 0, 1 and block 2's A in flight; block 0 read
    load_scales(kb0);
  #pragma unroll
    for (int h = 0; h < 5; ++h)
  #pragma unroll
      for (int t = 0; t < ((h & 1) ? LB : LA); ++t) issue_load(h, t);
    wait_vmcnt<LA + LB + LA>();         // block 0 landed
    lds_barrier();
  #pragma unroll
    for (int i = 0; i < TI; ++i) af[i] = frag(0, a_off0, a_off1, i);
  #pragma unroll
    for (int j = 0; j < TJ; ++j) bf[j] = frag(1, b_off0, b_off1, j);
    use_scales();     // consumed where loaded, never across the back edge

    constexpr int kMfma = 0x008, kVmemRead = 0x020, kDsRead = 0x100;
    constexpr int MF = OP == BSMM_OP_INT8_ROWWISE ? 2 : 1;
    auto mfma_tile = [&](int i, int j) {
      if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
        const i32x4 alo = i32x4{af[i][0], af[i][1], af[i][2], af[i][3]};
        const i32x4 ahi = i32x4{af[i][4], af[i][5], af[i][6], af[i][7]};
        const i32x4 blo = i32x4{bf[j][0], bf[j][1], bf[j][2], bf[j][3]};
        const i32x4 bhi = i32x4{bf[j][4], bf[j][5], bf[j][6], bf[j][7]};
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(blo, alo, acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(bhi, ahi, acc[i][j], 0, 0, 0);
      } else {
        acc[i][j] = mfma_mx(bf[j], af[i], acc[i][j], ws_cur, i & 3, xs_cur[i >> 2]);
      }
    };
    for (int c = 0; c < nkb; ++c) {
  #pragma unroll
      for (int j = 0; j < TJ; ++j) mfma_tile(0, j);
      wait_vmcnt<LA>();                 // block c+1 landed
      wait_lgkm0();                     // this wave's reads of block c are done
      lds_barrier();                    // ... every wave's: block c's slots are free
      load_scales(kb0 + min(c + 1, nkb - 1));
      af[0] = frag(2 * c + 2, a_off0, a_off1, 0);
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int i = 1; i < TI; ++i) {
  #pragma unroll
        for (int j = 0; j < TJ; ++j) {
          mfma_tile(i, j);
          // row 7: B tile j is done for this block; read the next block's
          if (i == TI - 1) bf[j] = frag(2 * c + 3, b_off0, b_off1, j);
        }
        af[i] = frag(2 * c + 2, a_off0, a_off1, i);
        // refills: block c+2's B over rows 1..4, block c+3's A over rows 5..7
        if (i <= 4) {
          issue_load(2 * c + 5, 2 * (i - 1));
          issue_load(2 * c + 5, 2 * (i - 1) + 1);
        } else {
  #pragma unroll
          for (int t = LA * (i - 5) / 3; t < LA * (i - 4) / 3; ++t) issue_load(2 * c + 6, t);
        }
        // schedule: MFMAs with the fragment reads and loads spread among them
  #pragma unroll
        for (int j = 0; j < TJ; ++j) {
          __builtin_amdgcn_sched_group_barrier(kMfma, MF, 0);
          if (i == TI - 1) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
          if (j == 1 && i < TI - 1) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
          if (j == 4) {
            constexpr int kA = LA;   // block c+3's A loads over rows 5..7
            const int nl = i <= 4 ? 2 : kA * (i - 4) / 3 - kA * (i - 5) / 3;
            if (nl == 2) __builtin_amdgcn_sched_group_barrier(kVmemRead, 2, 0);
            if (nl == 3) __builtin_amdgcn_sched_group_barrier(kVmemRead, 3, 0);
          }
        }
        if (i == TI - 1) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      use_scales();     // block c+1's, after block c's last MFMA
    }
    wait_vmcnt<0>();     // the last refills were out-of-range loads
  }
};

template <int OP, int OUT, bool PK>
__global__ void __launch_bounds__(256)
tile4_kernel(const KArgs k) {
  using M = Mainloop4<OP, PK>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[M::LDS];
  const int KB = k.p.K / kBlockK;
  for (int u = first_unit(); u < k.units; u += gridDim.x) {
    const TileId t = decode_tile(k, u);
    const int row0 = k.row_begin + t.tm * M::BM;
    const int col0 = t.tn * M::BN;
    const int kb0 = t.s * k.kb_per_split;
    const int nkb = max(0, min(KB, kb0 + k.kb_per_split) - kb0);
    typename M::acc_t acc[M::TI][M::TJ];
#pragma unroll
    for (int i = 0; i < M::TI; ++i)
#pragma unroll
      for (int j = 0; j < M::TJ; ++j) acc[i][j] = typename M::acc_t{0, 0, 0, 0};
    M::run(k, smem, t.g, row0, col0, kb0, nkb, acc);
    if (k.splits > 1)
      store_staged<OP, OUT, 4, 2, kSplitK, 256, 256>(k, t.s, t.g, row0, col0, acc, smem);
    else
      store_staged<OP, OUT, 4, 2, kOut, 256, 256>(k, t.s, t.g, row0, col0, acc, smem);
  }
}

// One output tile (or one K slice of it, with split-K) per workgroup.
template <int OP, int OUT, int WM, int WN, int RING, bool PK>
__global__ void __launch_bounds__(64 * WM * WN)
tile_kernel(const KArgs k) {
  using M = Mainloop<OP, WM, WN, RING, PK>;
  using T = typename M::T;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[M::SMEM];
  const int KB = k.p.K / kBlockK;
  for (int u = first_unit(); u < k.units; u += gridDim.x) {
    const TileId t = decode_tile(k, u);
    const int row0 = k.row_begin + t.tm * T::BM;
    const int col0 = t.tn * T::BN;
    const int kb0 = t.s * k.kb_per_split;
    const int nkb = max(0, min(KB, kb0 + k.kb_per_split) - kb0);
    typename M::acc_t acc[M::TI][M::TJ];
#pragma unroll
    for (int i = 0; i < M::TI; ++i)
#pragma unroll
      for (int j = 0; j < M::TJ; ++j) acc[i][j] = typename M::acc_t{};
    M::run(k, smem, t.g, row0, col0, kb0, nkb, acc);
    if (k.splits > 1)
      store_staged<OP, OUT, WM * WN, WN, kSplitK, T::BM, T::BN>(k, t.s, t.g, row0, col0, acc, smem);
    else
      store_staged<OP, OUT, WM * WN, WN, kOut, T::BM, T::BN>(k, t.s, t.g, row0, col0, acc, smem);
  }
}

// ---------------------------------------------------------------------------
// Persistent stream-K kernel.  The work, tiles x K blocks, is cut into equal
// contiguous ranges, one per workgroup, so every CU gets the same number of
// K blocks however the tile count divides the CU count.  A tile split between
// consecutive ranges is finished by whichever of its segments' workgroups
// arrives last: each segment stores its fp32 / int32 partial in a slot of
// its own, then counts itself in the tile's counter with a global atomic;
// the workgroup that brings the count to the number of segments adds all of
// them in K order (its own from registers) and stores the tile.  No
// workgroup ever waits for another, so the result does not depend on how
// many of the grid's workgroups the device holds at once, and the fixed K
// order makes it deterministic.
// The partials and the counters are touched only through agent-scope
// atomics, whose stores write through to the device's coherence point and
// whose loads read from it; a wave's vmcnt wait after its stores orders them
// before the count, and the adds read after the count.  That gives the
// ordering of a release and an acquire without a fence's L2 write-back and
// invalidate, which serialise across an XCD's workgroups.
// A counter holds the launch's 40-bit tag above a 24-bit count; a value with
// another tag (an earlier launch, or whatever the workspace held) counts as
// zero, so the counters need no clearing between launches.
// Workspace: two partial slots of BM x BN elements per workgroup (see
// SlotRef), then one 64-bit counter per stream-K tile (at most 2P of them).
// ---------------------------------------------------------------------------
struct SkArgs {
  int64_t units;       // K-block units of the stream-K phase: sk tiles * KB (>= P)
  uint64_t epoch;      // distinct per launch (its low 40 bits tag the counters)
  int tiles_total;     // tiles_m * tiles_n * G
  int dp_tiles;        // whole tiles before the stream-K phase
};

template <int OP, int OUT, int WM, int WN, int RING, bool PK>
__global__ void __launch_bounds__(64 * WM * WN)
sk_kernel(const KArgs k, const SkArgs sk) {
  using M = Mainloop<OP, WM, WN, RING, PK>;
  using T = typename M::T;
  using acc_t = typename M::acc_t;
  typedef typename OpT<OP>::elem_t E;
  constexpr int TI = M::TI, TJ = M::TJ;
  constexpr int SLOT_ELEMS = T::BM * T::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[M::SMEM];
  // the last-arrival flag: the ring's first word, idle between a segment's
  // stores and the next barrier (the ring fills the whole LDS)
  int* const last_arrival = (int*)smem;
  const int P = gridDim.x;
  // XCD-aware: consecutive ranges run on the same XCD
  const int hw = blockIdx.x;
  const int per = P >> 3, rem = P & 7;
  const int xcd = hw & 7, local = hw >> 3;
  const int w = (xcd < rem) ? xcd * (per + 1) + local
                            : rem * (per + 1) + (xcd - rem) * per + local;
  const int KB = k.p.K / kBlockK;
  auto range_start = [&](int wi) { return (int64_t)wi * sk.units / P; };   // units * P < 2^63
  // the range holding unit u: the last wi with range_start(wi) <= u (every
  // range is non-empty because units >= P)
  auto range_of = [&](int64_t u) { return (int)(((u + 1) * P - 1) / sk.units); };
  E* slots = (E*)k.ws;
  uint64_t* counters = (uint64_t*)((uint8_t*)k.ws + (size_t)2 * P * SLOT_ELEMS * sizeof(E));
  const uint64_t tag = sk.epoch & ((1ull << 40) - 1);
  const int tid = threadIdx.x;

  // Data-parallel phase: whole tiles dp_tiles in the persistent order
  // (workgroup w takes tiles w, w + P, ...: at any time the workgroups of an
  // XCD hold a compact block of the grouped raster).  Then the stream-K phase
  // over the remaining tiles' K blocks, contiguous ranges per workgroup.
  int dp = w;
  int64_t u = range_start(w);
  const int64_t uend = range_start(w + 1);
  while (dp < sk.dp_tiles || u < uend) {
    int tile, kb_a, kb_b;
    if (dp < sk.dp_tiles) {
      tile = dp;
      kb_a = 0;
      kb_b = KB;
    } else {
      const int st = (int)(u / KB);
      tile = sk.dp_tiles + st;
      kb_a = (int)(u - (int64_t)st * KB);
      kb_b = (int)min((int64_t)KB, (int64_t)kb_a + (uend - u));
    }
    // tile -> (g, tm, tn): grouped order within each G
    const int tiles = k.tiles_m * k.tiles_n;
    const int g = tile / tiles;
    const int tin = tile - g * tiles;
    constexpr int GROUP_M = 8;
    const int width = GROUP_M * k.tiles_n;
    const int gid = tin / width;
    const int first_m = gid * GROUP_M;
    const int gsize = min(k.tiles_m - first_m, GROUP_M);
    const int in = tin - gid * width;
    const int tm = first_m + in % gsize, tn = in / gsize;
    const int row0 = k.row_begin + tm * T::BM;
    const int col0 = tn * T::BN;

    acc_t acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j) acc[i][j] = acc_t{};
    M::run(k, smem, g, row0, col0, kb_a, kb_b - kb_a, acc);

    if (kb_a == 0 && kb_b == KB) {
      store_staged<OP, OUT, WM * WN, WN, kOut, T::BM, T::BN>(k, 0, g, row0, col0, acc, smem);
    } else {
      // a segment of a split tile (tiles of the data-parallel phase are
      // never split)
      const int64_t t0 = (int64_t)(tile - sk.dp_tiles) * KB;   // the tile's first unit
      SlotRef sl;
      sl.base = slots;
      sl.stride = SLOT_ELEMS;
      sl.first = range_of(t0);
      sl.count = range_of(t0 + KB - 1) - sl.first + 1;
      sl.first_odd = range_start(sl.first) < t0 ? 1 : 0;
      sl.own = w - sl.first;
      // publish this segment's partial, then count it in
      SlotRef mine;
      mine.base = slots + sl.slot(sl.own) * SLOT_ELEMS;
      store_staged<OP, OUT, WM * WN, WN, kSlot, T::BM, T::BN>(k, 0, g, row0, col0, acc, smem,
                                                              mine);
      wait_vmcnt<0>();     // this wave's part of the partial has reached the
      __syncthreads();     // coherence point (agent-scope stores), every wave's
      if (tid == 0)
        *last_arrival = count_arrival(counters + (tile - sk.dp_tiles), tag, sl.count) == sl.count;
      __syncthreads();
      if (*last_arrival) {   // store_staged's first barrier precedes any LDS write
        // the other partials are read with agent-scope loads (no fence)
        store_staged<OP, OUT, WM * WN, WN, kOutAdd, T::BM, T::BN>(k, 0, g, row0, col0, acc, smem,
                                                                  sl);
      }
    }
    if (dp < sk.dp_tiles) dp += P;
    else u += kb_b - kb_a;
  }
}

// Split-K reduction: out = epilogue(sum over s of partial[s]) in ascending s.
template <int OP, int OUT>
__global__ void __launch_bounds__(256)
splitk_reduce(const KArgs k) {
  // Work items (row of [G][rows], 1024-column chunk) strided over the grid,
  // 4-column groups over the workgroup's threads; one division per item.
  const Problem& p = k.p;
  const int rows = k.row_end - k.row_begin;
  const int64_t nrows = (int64_t)rows * p.G;
  const int64_t split_stride = nrows * p.N;
  typedef typename OpT<OP>::elem_t E;
  typedef E e4 __attribute__((ext_vector_type(4)));
  const E* ws = (const E*)k.ws;
  const bool v4 = (p.N & 3) == 0;     // partial rows are 16-byte aligned
  const bool vec = k.vec_out != 0;
  const int chunks = (p.N + 1023) / 1024;
  const int64_t items = nrows * chunks;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t r = it / chunks;
    const int n0 = (int)(it - r * chunks) * 1024;
    const int g = (int)(r / rows);
    const int mr = (int)(r - (int64_t)g * rows);
    const int m = k.row_begin + mr;
    const E* src = ws + r * p.N;
    float sa_m = 1.f;
    if constexpr ((OP == BSMM_OP_INT8_ROWWISE && OUT != BSMM_I32) || OP == BSMM_OP_FP8_SCALED_MM)
      sa_m = ((const float*)p.sa)[(int64_t)m * p.sa_m];
    [[maybe_unused]] const ScaledEpi epi(p);
    uint8_t* obase = (uint8_t*)p.out;
    const int64_t orow = (int64_t)g * p.o_sg + (int64_t)m * p.ldo;
    for (int n = n0 + 4 * (int)threadIdx.x; n < min(p.N, n0 + 1024); n += 4 * (int)blockDim.x) {
      const int nvalid = min(4, p.N - n);
      E s[4] = {0, 0, 0, 0};
      for (int q = 0; q < k.splits; ++q) {
        const E* sq = src + (int64_t)q * split_stride + n;
        if (v4) {
          const e4 t = *(const e4*)sq;
#pragma unroll
          for (int c = 0; c < 4; ++c) s[c] += t[c];
        } else {
          for (int c = 0; c < nvalid; ++c) s[c] += sq[c];
        }
      }
      float y[4];
      int yi[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (OP == BSMM_OP_INT8_ROWWISE) {
          yi[c] = (int)s[c];
          if constexpr (OUT != BSMM_I32)
            y[c] = __fmul_rn(__fmul_rn((float)s[c], sa_m),
                             ((const float*)p.sb)[(int64_t)min(n + c, p.N - 1) * p.sb_n]);
        } else if constexpr (OP == BSMM_OP_FP8_SCALED_MM) {
          const int nc = min(n + c, p.N - 1);
          y[c] = epi((float)s[c], sa_m, ((const float*)p.sb)[(int64_t)nc * p.sb_n], nc);
        } else {
          y[c] = (float)s[c];
        }
      }
      store4<OUT>(obase, orow + n, y, yi, vec, nvalid);
    }
  }
}

// Output for K == 0: zeros; for scaled_mm the epilogue of the empty sum
// ((0 * (sa * sb) + bias) * sr).
template <int OP, int OUT>
__global__ void zero_out(const KArgs k) {
  const Problem& p = k.p;
  const int64_t per_g = (int64_t)p.M * p.N;
  const int64_t total = per_g * p.G;
  [[maybe_unused]] const ScaledEpi epi(p);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(e / per_g);
    const int64_t rem = e - (int64_t)g * per_g;
    const int m = (int)(rem / p.N);
    const int n = (int)(rem - (int64_t)m * p.N);
    const int64_t o = (int64_t)g * p.o_sg + (int64_t)m * p.ldo + n;
    float y[4] = {0.f, 0.f, 0.f, 0.f};
    const int yi[4] = {0, 0, 0, 0};
    if constexpr (OP == BSMM_OP_FP8_SCALED_MM)
      y[0] = epi(0.f, ((const float*)p.sa)[(int64_t)m * p.sa_m],
                 ((const float*)p.sb)[(int64_t)n * p.sb_n], n);
    store4<OUT>((uint8_t*)p.out, o, y, yi, false, 1);
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
int check_launch() {
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Output rows allow 8-byte (bf16) / 16-byte (fp32, int32) vector stores.
template <int OUT>
bool out_vec_ok(const Problem& p) {
  const int osz = OUT == BSMM_E4M3 ? 1 : OUT == BSMM_BF16 ? 2 : 4;
  const int vbytes = 4 * osz;
  return ((uintptr_t)p.out % vbytes == 0) && (p.ldo * osz) % vbytes == 0 &&
         (p.o_sg * osz) % vbytes == 0;
}

// Packed-scale kernels: the launch brings scale_a already packed; rows of a
// launch must start on a multiple of 64 (packed groups).
template <bool PK>
bool set_packed(KArgs& k, const Launch& l) {
  k.psa = l.psa;
  k.psa_ld = packed_rows(k.p.M);
  // an empty K sum reads no scales (the output is zeroed)
  return !PK || k.p.K < kBlockK || (l.psa != nullptr && l.row_begin % 64 == 0);
}

// Workgroups of a kernel the current device holds at once (0 on error),
// cached per device in `cache`.
int device_slots(const void* kernel, int threads, std::atomic<int>* cache) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int cap = cache[dev].load(std::memory_order_relaxed);
  if (cap == 0) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, 0) != hipSuccess)
      return 0;
    cap = cus * (occ > 0 ? occ : 1);
    cache[dev].store(cap, std::memory_order_relaxed);
  }
  return cap;
}

// Grid of a tile launch: one workgroup per unit, or -- with more units than
// the device holds at once -- one per slot, each looping over units.
int64_t tile_grid(int64_t units, const void* kernel, int threads, std::atomic<int>* cache) {
  const int cap = device_slots(kernel, threads, cache);
  return cap > 0 && units > cap ? cap : units;
}

template <int OP, int OUT, int WM, int WN, int RING, bool PK>
int launch_tile(const Problem& p, const Launch& l) {
  using T = Tile<OP, WM, WN, RING>;
  const int row_begin = l.row_begin, row_end = l.row_end;
  int split = l.split;
  void* ws = l.ws;
  KArgs k;
  k.p = p;
  if (!set_packed<PK>(k, l)) return 1;
  k.row_begin = row_begin;
  k.row_end = row_end;
  const int rows = row_end - row_begin;
  k.tiles_m = (rows + T::BM - 1) / T::BM;
  k.tiles_n = (p.N + T::BN - 1) / T::BN;
  const int KB = p.K / kBlockK;
  hipStream_t s = (hipStream_t)l.stream;
  if (KB == 0) {              // empty sum: the output is zero
    k.ws = ws;
    k.splits = 1;
    k.kb_per_split = 0;
    k.vec_out = 0;
    hipLaunchKernelGGL((zero_out<OP, OUT>), dim3(1024), dim3(256), 0, s, k);
    return check_launch();
  }
  k.ws = ws;
  if (split < 1) split = 1;
  if (split > KB) split = KB;
  k.kb_per_split = (KB + split - 1) / split;
  k.splits = (KB + k.kb_per_split - 1) / k.kb_per_split;
  if (k.splits > 1) {
    // workspace rows are N elements of 4 bytes
    k.vec_out = aligned16(ws) && p.N % 4 == 0;
  } else {
    k.vec_out = out_vec_ok<OUT>(p);
  }
  const int64_t units = (int64_t)k.tiles_m * k.tiles_n * p.G * k.splits;
  k.units = (int)units;
  static std::atomic<int> slots[64];
  const int64_t grid = tile_grid(
      units, reinterpret_cast<const void*>(&tile_kernel<OP, OUT, WM, WN, RING, PK>), T::NT, slots);
  hipLaunchKernelGGL((tile_kernel<OP, OUT, WM, WN, RING, PK>), dim3((unsigned)grid), dim3(T::NT), 0, s, k);
  if (check_launch()) return 1;
  if (k.splits > 1) {
    int64_t blocks = (int64_t)rows * p.G * ((p.N + 1023) / 1024);   // (row, chunk) items
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((splitk_reduce<OP, OUT>), dim3((unsigned)blocks), dim3(256), 0, s, k);
    return check_launch();
  }
  return 0;
}

// The wide-wave kernel (four waves of 128 x 128, int8 / mx).
template <int OP, int OUT, bool PK>
int launch_tile4(const Problem& p, const Launch& l) {
  using T = Mainloop4<OP, PK>;
  const int row_begin = l.row_begin, row_end = l.row_end;
  int split = l.split;
  void* ws = l.ws;
  KArgs k;
  k.p = p;
  if (!set_packed<PK>(k, l)) return 1;
  k.row_begin = row_begin;
  k.row_end = row_end;
  const int rows = row_end - row_begin;
  k.tiles_m = (rows + T::BM - 1) / T::BM;
  k.tiles_n = (p.N + T::BN - 1) / T::BN;
  const int KB = p.K / kBlockK;
  hipStream_t s = (hipStream_t)l.stream;
  if (KB == 0) {              // empty sum: the output is zero
    k.ws = ws;
    k.splits = 1;
    k.kb_per_split = 0;
    k.vec_out = 0;
    hipLaunchKernelGGL((zero_out<OP, OUT>), dim3(1024), dim3(256), 0, s, k);
    return check_launch();
  }
  k.ws = ws;
  if (split < 1) split = 1;
  if (split > KB) split = KB;
  k.kb_per_split = (KB + split - 1) / split;
  k.splits = (KB + k.kb_per_split - 1) / k.kb_per_split;
  if (k.splits > 1) {
    // workspace rows are N elements of 4 bytes
    k.vec_out = aligned16(ws) && p.N % 4 == 0;
  } else {
    k.vec_out = out_vec_ok<OUT>(p);
  }
  const int64_t units = (int64_t)k.tiles_m * k.tiles_n * p.G * k.splits;
  k.units = (int)units;
  static std::atomic<int> slots[64];
  const int64_t grid = tile_grid(units, reinterpret_cast<const void*>(&tile4_kernel<OP, OUT, PK>),
                                 T::NT, slots);
  hipLaunchKernelGGL((tile4_kernel<OP, OUT, PK>), dim3((unsigned)grid), dim3(T::NT), 0, s, k);
  if (check_launch()) return 1;
  if (k.splits > 1) {
    int64_t blocks = (int64_t)rows * p.G * ((p.N + 1023) / 1024);   // (row, chunk) items
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL((splitk_reduce<OP, OUT>), dim3((unsigned)blocks), dim3(256), 0, s, k);
    return check_launch();
  }
  return 0;
}

// Distinct per launch for the stream-K flags; seeded from the clock so that
// flags left in a reused workspace by another process do not match.
uint64_t next_epoch() {
  static std::atomic<uint64_t> ctr{
      ((uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() << 16) | 1u};
  return ctr.fetch_add(1, std::memory_order_relaxed);
}

template <int OP, int OUT, int WM, int WN, int RING, bool PK>
int launch_sk(const Problem& p, const Launch& l) {
  using T = Tile<OP, WM, WN, RING>;
  const int KB = p.K / kBlockK;
  typedef typename OpT<OP>::elem_t E;
  // two partial slots and two counters per workgroup (see sk_kernel)
  const size_t per_wg = 2 * ((size_t)T::BM * T::BN * sizeof(E) + sizeof(uint64_t));
  if (KB == 0 || !aligned16(l.ws) || l.ws_bytes < per_wg)
    return launch_tile<OP, OUT, WM, WN, RING, PK>(p, l);
  // the grid: the kernel's co-resident capacity on the current device
  // (cached), or the caller's choice -- the kernel never waits, so any grid
  // is correct
  static std::atomic<int> cap_cache[64];
  const int cap = l.sk_grid > 0 ? l.sk_grid
                                : device_slots(reinterpret_cast<const void*>(
                                                   &sk_kernel<OP, OUT, WM, WN, RING, PK>),
                                               T::NT, cap_cache);
  if (cap <= 0) return 1;
  KArgs k;
  k.p = p;
  if (!set_packed<PK>(k, l)) return 1;
  k.row_begin = l.row_begin;
  k.row_end = l.row_end;
  const int rows = l.row_end - l.row_begin;
  k.tiles_m = (rows + T::BM - 1) / T::BM;
  k.tiles_n = (p.N + T::BN - 1) / T::BN;
  k.splits = 1;
  k.kb_per_split = KB;
  k.units = 0;
  k.vec_out = out_vec_ok<OUT>(p);
  hipStream_t s = (hipStream_t)l.stream;
  k.ws = l.ws;
  SkArgs sk;
  sk.tiles_total = k.tiles_m * k.tiles_n * p.G;
  int P = cap;
  if ((int64_t)P > (int64_t)sk.tiles_total * KB) P = (int)((int64_t)sk.tiles_total * KB);
  if ((size_t)P * per_wg > l.ws_bytes) P = (int)(l.ws_bytes / per_wg);
  // whole rounds of tiles run data-parallel, except that the last P or more
  // tiles (a round and the remainder) are spread as K blocks over all P
  // workgroups; a whole number of rounds runs data-parallel throughout
  const int rounds = sk.tiles_total / P;
  if (sk.tiles_total % P == 0) sk.dp_tiles = sk.tiles_total;
  else sk.dp_tiles = rounds >= 1 ? (rounds - 1) * P : 0;
  sk.units = (int64_t)(sk.tiles_total - sk.dp_tiles) * KB;
  sk.epoch = next_epoch();
  hipLaunchKernelGGL((sk_kernel<OP, OUT, WM, WN, RING, PK>), dim3((unsigned)P), dim3(T::NT), 0, s,
                     k, sk);
  return check_launch();
}

}  // namespace

// Entry used by the variant table: one kernel configuration for one
// (operation, output type).  Instantiated below for the pair this
// translation unit is compiled for.
// Skinny launch (M <= 16): one workgroup per 16 columns of each batch.
template <int OP, int OUT, int SPF>
int launch_skinny(const Problem& p, const Launch& l) {
  if (p.M > 16 || l.row_begin != 0 || l.row_end != p.M) return 1;
  KArgs k;
  k.p = p;
  k.row_begin = 0;
  k.row_end = p.M;
  k.psa = nullptr;
  k.psa_ld = 0;
  k.ws = nullptr;
  k.splits = 1;
  k.kb_per_split = p.K / kBlockK;
  k.units = 0;
  k.tiles_m = 1;
  k.tiles_n = (p.N + 15) / 16;
  k.vec_out = out_vec_ok<OUT>(p);
  hipStream_t s = (hipStream_t)l.stream;
  if (p.K / kBlockK == 0) {
    hipLaunchKernelGGL((zero_out<OP, OUT>), dim3(1024), dim3(256), 0, s, k);
    return check_launch();
  }
  const int64_t grid = (int64_t)k.tiles_n * p.G;
  hipLaunchKernelGGL((skinny_kernel<OP, OUT, SPF>), dim3((unsigned)grid), dim3(256), 0, s, k);
  return check_launch();
}

// The narrow kernel (16 < rows <= 128): one workgroup per BN columns of each
// batch and K range.  Shapes it does not take (more rows, N not a multiple
// of BN, more K blocks per range than its scale region holds, an operation
// it lacks) run the 128 x 128 tile kernel instead.  A split the workspace
// cannot hold (or more ranges than K blocks) is reduced.
template <int OP, int OUT, int BN>
int launch_narrow(const Problem& p, const Launch& l) {
  const int rows = l.row_end - l.row_begin;
  const int KB = p.K / kBlockK;
  int S = l.split < 1 ? 1 : (l.split > KB ? (KB > 0 ? KB : 1) : l.split);
  if (S > 1 && (!l.ws || l.ws_bytes < narrow_workspace(p.G, p.N, BN, S))) S = 1;
  // ranges of ceil(KB / S) blocks; as many as that leaves non-empty
  const int nk_max = KB > 0 ? (KB + S - 1) / S : 0;
  if (nk_max > 0) S = (KB + nk_max - 1) / nk_max;
  bool ok = narrow::supported<OP>() && rows <= narrow::BM && p.N % BN == 0;
  if constexpr (OP == BSMM_OP_FP8_MX_BMM) ok = ok && narrow::scales_fit<uint8_t>(nk_max);
  if constexpr (OP == BSMM_OP_FP8_BLOCKWISE) ok = ok && narrow::scales_fit<float>(nk_max);
  if (!ok) {
    Launch l2 = l;
    l2.psa = nullptr;
    return launch_tile<OP, OUT, 2, 1, 5, false>(p, l2);
  }
  if constexpr (narrow::supported<OP>()) {
    KArgs k;
    k.p = p;
    k.row_begin = l.row_begin;
    k.row_end = l.row_end;
    k.psa = nullptr;
    k.psa_ld = 0;
    k.ws = S > 1 ? l.ws : nullptr;
    k.splits = S;
    k.kb_per_split = nk_max;
    k.tiles_m = 1;
    k.tiles_n = p.N / BN;
    k.vec_out = out_vec_ok<OUT>(p);
    k.epoch = S > 1 ? next_epoch() : 0;
    hipStream_t s = (hipStream_t)l.stream;
    if (KB == 0) {
      hipLaunchKernelGGL((zero_out<OP, OUT>), dim3(1024), dim3(256), 0, s, k);
      return check_launch();
    }
    k.units = p.G * k.tiles_n * S;
    hipLaunchKernelGGL((narrow_kernel<OP, OUT, BN>), dim3((unsigned)k.units), dim3(256), 0, s, k);
    return check_launch();
  }
  return 1;
}

template <int OP, int OUT, int WM, int WN, int RING, bool SK, bool PK, int KIND>
int launch_kernel(const Problem& p, const Launch& l) {
  // the int8 and scaled_mm K loops read no scales: packed variants run the
  // plain kernel
  constexpr bool PKX = PK && (OP == BSMM_OP_FP8_BLOCKWISE || OP == BSMM_OP_FP8_MX_BMM ||
                              OP == BSMM_OP_FP8_MX32_MM || OP == BSMM_OP_FP8_GROUPWISE);
  if constexpr (OP == BSMM_OP_FP8_GROUPWISE && (!PK || KIND == 2)) {
    // groupwise reads its scales packed; no unpacked or skinny kernel
    (void)p;
    (void)l;
    return 1;
  } else if constexpr (KIND == 2) {
    return launch_skinny<OP, OUT, RING>(p, l);
  } else if constexpr (KIND == 3 || KIND == 4) {
    return launch_narrow<OP, OUT, KIND == 3 ? 32 : 64>(p, l);
  } else if constexpr (KIND == 1) {
    // wide waves for int8 / mx / scaled_mm; blockwise and mx32 (per-lane
    // column scales) run the 256 x 256 eight-wave kernel
    if constexpr (OP == BSMM_OP_FP8_BLOCKWISE || OP == BSMM_OP_FP8_MX32_MM ||
                  OP == BSMM_OP_FP8_GROUPWISE)
      return launch_tile<OP, OUT, 4, 2, 5, PKX>(p, l);
    else
      return launch_tile4<OP, OUT, PKX>(p, l);
  } else if constexpr (SK)
    return launch_sk<OP, OUT, WM, WN, RING, PKX>(p, l);
  else
    return launch_tile<OP, OUT, WM, WN, RING, PKX>(p, l);
}

#if defined(BSMM_TU_OP) && defined(BSMM_TU_OUT)
#define BSMM_VARIANT(NAME, TM, TN, WM, WN, RING, SK, PK, WPC, UNPACKED, KIND)               \
  template int launch_kernel<BSMM_TU_OP, BSMM_TU_OUT, WM, WN, RING, SK, PK, KIND>(        \
      const Problem&, const Launch&);
#include "bsmm_variants.inc"
#undef BSMM_VARIANT
#endif

}  // namespace bsmm
