// Internal interface between the host front end (validation, dispatch) and
// the HIP kernels.  Plain C++; no HIP types, so the front end is host code.
#pragma once

#include <cstddef>
#include <cstdint>

#include "bsmm.h"

namespace bsmm {

constexpr int kBlockK = 128;   // K extent of one scale block and one k-step

// One GEMM problem after validation, in a single strided form that covers
// all three entry points.  Element (g, m, k) of A is at
// a + g*a_sg + m*lda + k; element (g, n, k) of B at b + g*b_sg + n*ldb + k.
// Output (g, m, n) at out + (g*o_sg + m*ldo + n) * sizeof(out element).
struct Problem {
  bsmm_op op;
  bsmm_dtype out_dtype;
  int G, M, N, K;
  const uint8_t* a; int64_t a_sg, lda;
  const uint8_t* b; int64_t b_sg, ldb;
  // scales, strides in elements (float for int8 / blockwise, byte for mx)
  //   int8:      sa[m*sa_m], sb[n*sb_n]                       (sb_kb unused)
  //   blockwise: sa[m*sa_m + kb*sa_kb], sb[kb*sb_kb + nb*sb_n]
  //   mx:        sa[g*sa_sg + m*sa_m + kb], sb[g*sb_sg + nb*sb_n + kb]
  //   mx32:      sa[m*sa_m + c], sb[n*sb_n + c] for 32-long K chunk c (bytes)
  //   scaled_mm: sa[m*sa_m], sb[n*sb_n] (fp32; stride 0 for one scalar)
  //   groupwise: sa[m*sa_m + kb*sa_kb], sb[kb*sb_kb + n*sb_n]
  const void* sa; int64_t sa_sg, sa_m, sa_kb;
  const void* sb; int64_t sb_sg, sb_n, sb_kb;
  void* out; int64_t o_sg, ldo;
  // fp8 scaled_mm epilogue: bias [N] (fp32, or bf16 when bias_bf16), result
  // scale (one fp32); null when absent
  const void* bias; int bias_bf16;
  const float* sr;
};

// Operations whose K loop can read its scales from the packed layouts of
// the pre-pass.
inline bool packable_scales(bsmm_op op) {
  return op == BSMM_OP_FP8_BLOCKWISE || op == BSMM_OP_FP8_MX_BMM || op == BSMM_OP_FP8_MX32_MM ||
         op == BSMM_OP_FP8_GROUPWISE;
}

struct Variant;

struct Plan {
  const Variant* v = nullptr;      // main launch
  int split = 1;                   // K slices of the main launch
  const Variant* tail = nullptr;   // second launch for rows [m_split, M)
  int m_split = 0;                 // 0: one launch covers all of M
  int tail_split = 1;              // K slices of the tail launch
  size_t workspace = 0;            // bytes used
  int source = 2;                  // bsmm_plan_info::source
};

// One kernel launch over rows [row_begin, row_end) of a problem.
struct Launch {
  int row_begin, row_end;
  int split;             // K slices (split-K partials in ws)
  void* ws;              // split-K partials / stream-K slots
  size_t ws_bytes;
  const void* psa;       // packed scale_a, already written (packed variants)
  void* stream;
  int sk_grid = 0;       // stream-K grid (0: the device's co-resident capacity)
};

// Kernel variants compiled into the library.
using LaunchFn = int (*)(const Problem& p, const Launch& l);
struct Variant {
  const char* name;
  int tile_m, tile_n;
  unsigned op_mask;     // bit i set: usable for bsmm_op i
  bool masked_tail;     // safe for rows past M (every variant is)
  bool persistent;      // stream-K: one workgroup per slot of the device
  bool packed_scales;   // fp8: repacks scale_a into the workspace first
  int wg_per_cu;        // workgroups one CU holds (LDS / registers)
  const char* unpacked; // the same kernel without packed scales (or null)
  int max_m;            // largest M the kernel takes in one launch (0: any)
  int kind;             // 0 tile, 1 wide-wave tile, 2 skinny, 3 / 4 narrow (32 / 64 columns)
  LaunchFn launch;
};

// Workspace of a narrow-kernel launch split into S K ranges: S partial
// 128 x tile_n tiles (4-byte elements) per output tile, then one 64-bit
// counter per output tile.  It also covers the split-K partials of the tile
// kernel the narrow launch falls back to (at most 128 rows).
inline size_t narrow_workspace(int G, int N, int tile_n, int split) {
  if (split <= 1) return 0;
  const size_t tiles = (size_t)G * (size_t)((N + tile_n - 1) / tile_n);
  return (size_t)split * tiles * 128u * (size_t)tile_n * 4u + tiles * 8u;
}

// Packed scale_a for the fp8 kernels: K block major, rows padded to a
// multiple of 256, and within every 64 rows the element of row
// 64q + 16i + f stored at position 64q + 4f + i, so that one 16-byte
// (fp32) or 4-byte (e8m0) load gives a lane the scales of its four rows
// f, f+16, f+32, f+48.  Layout [G][KB][Mp] (G = 1 for blockwise).
//
// mx32 (32-element K chunks, both operands): a_scale packed as above with
// the chunk c = K/32 index in place of the K block, [KC][Mp] bytes; then
// (at the next 256-byte boundary) b_scale with column 128g + 16j + f at
// position 128g + 8f + j, [KC][Np] bytes (Np = N rounded up to 256), so
// that one 8-byte load gives a lane the scales of its eight columns f,
// f+16, .., f+112 of a 128-column wave tile.
//
// groupwise (1 x 128 groups on both operands): scale_a packed as for
// blockwise, [KB][Mp] fp32; then (at the next 256-byte boundary) scale_b
// in plain column order, [KB][Np] fp32, columns past N repeating column
// N-1.  The K loop stages each K block's slices of both through LDS.
inline int packed_rows(int M) { return (M + 255) / 256 * 256; }
inline size_t packed_gw_a_bytes(int M, int K) {
  return ((size_t)(K / kBlockK) * (size_t)packed_rows(M) * 4u + 255) / 256 * 256;
}
inline size_t packed_mx32_a_bytes(int M, int K) {
  return ((size_t)(K / 32) * (size_t)packed_rows(M) + 255) / 256 * 256;
}
inline size_t packed_scale_bytes(bsmm_op op, int G, int M, int K, int N = 0) {
  if (!packable_scales(op)) return 0;
  if (op == BSMM_OP_FP8_MX32_MM)
    return packed_mx32_a_bytes(M, K) + ((size_t)(K / 32) * (size_t)packed_rows(N) + 255) / 256 * 256;
  if (op == BSMM_OP_FP8_GROUPWISE)
    return packed_gw_a_bytes(M, K) + packed_gw_a_bytes(N, K);
  const size_t elem = op == BSMM_OP_FP8_BLOCKWISE ? 4u : 1u;
  const size_t n = (size_t)(op == BSMM_OP_FP8_MX_BMM ? G : 1) * (size_t)(K / kBlockK) *
                   (size_t)packed_rows(M) * elem;
  return (n + 255) / 256 * 256;
}

// Workspace a persistent (stream-K) variant wants: two partial tiles and
// two 64-bit counters per workgroup, for a device of kPlanCUs compute units.
constexpr int kPlanCUs = 256;
size_t persistent_workspace(const Variant* v, bsmm_op op);

const Variant* variants(int* count);

// One kernel configuration for one (operation, output type); defined in the
// HIP translation units, one per (OP, OUT) pair, for every configuration in
// bsmm_variants.inc.  PK: the fp8 main loop reads packed scale_a, which the
// launch first writes to the start of the workspace.
template <int OP, int OUT, int WM, int WN, int RING, bool SK, bool PK, int KIND>
int launch_kernel(const Problem& p, const Launch& l);

// Write packed scale_a (layout above) for an fp8 problem to dst, which holds
// packed_scale_bytes(...) bytes and is 16-byte aligned.  Returns 0 on success.
int pack_scale_a(const Problem& p, void* dst, void* stream);
const Variant* find_variant(const char* name);

// Bytes of split-K workspace a variant needs for `split` slices.
size_t splitk_workspace(const Problem& p, int rows, int split);

// Benchmark timing of the main launch of each call (bsmm_timing.cpp).
bool timing_on();
void timing_mark(void* stream, const char* name, bool begin);

// Dynamic quantisation of bf16 / fp32 rows (bsmm_quant.hip).  Arguments are
// validated by the entry points before this is called.
//
// kFp8Columns: groups of 128 rows down each column of x [M, K]; codes only
// transposed, qt [K, M] (row stride ldqt); scale (g, c) at scale[g*s_m +
// c*s_kb] for g < M/128.  kFp8Weight: 128 x 128 blocks; codes in q [M, K]
// and / or qt [K, M] (either may be null); scale (g, cb) at scale[g*s_m +
// cb*s_kb].  kFp8RowsColumns: kFp8Columns plus the 1 x 128 row blocks of the
// same input, codes in q [M, K], scale (m, kb) at scale2[m*s2_m + kb*s2_kb].
struct QuantArgs {
  enum Kind { kInt8Rows = 0, kFp8Blocks = 1, kFp8Mx = 2, kFp8Mx32 = 3, kFp8Columns = 4,
              kFp8Weight = 5, kFp8RowsColumns = 6 };
  Kind kind;
  const void* x;        // [M, K] bf16 or fp32, row stride ldx elements
  int64_t ldx;
  bsmm_dtype x_dtype;   // BSMM_BF16 or BSMM_F32
  void* q;              // [M, K] 1-byte codes, row stride ldq
  int64_t ldq;
  void* scale;          // fp32 (kInt8Rows, kFp8Blocks) or e8m0 bytes (kFp8Mx)
  int64_t s_m, s_kb;    // scale strides in elements (s_kb unused for kInt8Rows)
  int64_t M, K;
  void* qt = nullptr;   // transposed codes [K, M] (kFp8Columns, kFp8Weight)
  int64_t ldqt = 0;
  void* scale2 = nullptr;   // row-block scales (kFp8RowsColumns)
  int64_t s2_m = 0, s2_kb = 0;
};
int launch_quant(const QuantArgs& a, void* stream);

// The static device scratch of the allocation-free entry point
// (bsmm_scratch.hip): its size, and the current device's copy's address
// (null, with *err the HIP error, on failure).
constexpr size_t kScratchBytes = (size_t)64 << 20;
void* scratch_device_ptr(int* err);

// Plan selection (host only).
Plan make_plan(bsmm_op op, int G, int M, int N, int K, bsmm_dtype dt,
               size_t workspace_bytes);
Plan make_plan_heuristic(bsmm_op op, int G, int M, int N, int K, bsmm_dtype dt);

}  // namespace bsmm
