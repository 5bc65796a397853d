/*
 * bsmm.h -- block-scaled low-precision matmul for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsmm.so.  Every entry point computes a low-precision GEMM or
 * batched GEMM whose int32 / fp32 accumulator is dequantised by per-row,
 * per-column or per-block scales.  A scale is a dequantisation multiplier:
 * the real value of an operand element is code * scale.
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Pointers: all operand, scale, output and workspace pointers are device
 *   pointers owned by the caller; the library allocates and frees nothing.
 * Operands: A is [M, K] with K contiguous (row-major); B is logically [K, N]
 *   and stored K-contiguous, i.e. column-major, element (k, n) at
 *   b[n * ldb + k].  This is the layout rule of Inductor's
 *   check_supported_striding for _scaled_mm (mat_a row-major, mat_b
 *   column-major) in torch/_inductor/kernel/mm.py.
 * Leading dimensions and batch strides are in elements; operand leading
 *   dimensions (bytes, since operands are 1-byte codes) must be multiples of
 *   16 and operand/output base pointers 16-byte aligned.
 * Supported sizes: K % 128 == 0 (the block-scale shapes imply it); the fp8
 *   entry points also need N % 128 == 0.  Any M >= 0.  M, N, K, G below 2^31;
 *   128 * (operand leading dimension) below 2^31.
 * Degenerate sizes: M == 0, N == 0 or G == 0 returns BSMM_OK and launches
 *   nothing.  K == 0 (which satisfies K % 128 == 0) writes zeros, the value
 *   of an empty sum.
 * Stream: `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *   asynchronous: errors detected from the arguments are returned before
 *   anything is enqueued; a launch failure reported by the HIP runtime is
 *   returned as BSMM_ERR_HIP.  No call synchronises the stream or the host.
 * Workspace: optional device scratch for split-K partial sums.  Pass the size
 *   from bsmm_workspace_bytes for the fastest plan; with less (or NULL) the
 *   call still succeeds with a plan that needs none (except
 *   bsmm_fp8_groupwise, whose kernels read repacked scales from it).  Results do not depend on
 *   the split: int32 accumulators are identical for every split, fp32 sums of
 *   the split partials are added in ascending split order.
 * Threads: the library keeps no mutable state across calls except a
 *   thread-local error message and the optional plan override; calls on
 *   different streams may run concurrently.  Two calls that write the same
 *   output or share a workspace on different streams race.
 */
#ifndef BSMM_H
#define BSMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSMM_VERSION 1

typedef enum {
  BSMM_OK = 0,
  BSMM_ERR_NULL = 1,        /* a required pointer is NULL                      */
  BSMM_ERR_SHAPE = 2,       /* negative size, leading dimension below the row  */
  BSMM_ERR_SCALE_SHAPE = 3, /* scale pointer / strides do not fit the mode     */
  BSMM_ERR_LAYOUT = 4,      /* strides describe an impossible layout           */
  BSMM_ERR_ALIGN = 5,       /* pointer or leading dimension misaligned         */
  BSMM_ERR_DTYPE = 6,       /* output dtype not available for this entry point */
  BSMM_ERR_UNSUPPORTED = 7, /* K % 128, N % 128 (fp8) or size limits           */
  BSMM_ERR_HIP = 8,         /* the HIP runtime reported an error               */
  BSMM_ERR_ARG = 9          /* any other invalid argument                      */
} bsmm_status;

typedef enum {
  BSMM_I32 = 0,  /* raw int32 accumulators (int8 entry point only)  */
  BSMM_F32 = 1,  /* IEEE binary32                                   */
  BSMM_BF16 = 2, /* bfloat16, round-to-nearest-even from binary32   */
  BSMM_E4M3 = 3  /* OCP E4M3FN codes, nearest even from binary32,   */
                 /* saturating at +-448 (bsmm_fp8_scaled_mm only)   */
} bsmm_dtype;

typedef enum {
  BSMM_OP_INT8_ROWWISE = 0,
  BSMM_OP_FP8_BLOCKWISE = 1,
  BSMM_OP_FP8_MX_BMM = 2,
  BSMM_OP_FP8_SCALED_MM = 3,
  BSMM_OP_FP8_MX32_MM = 4,
  BSMM_OP_FP8_GROUPWISE = 5
} bsmm_op;

/*
 * int8 x int8 -> int32 accumulate, rowwise activation scale and per-column
 * weight scale.
 *
 * Defined by torchao's int_scaled_matmul (PR "Remove int_scaled_mm's
 * dependency on triton for cpu": an int32 matmul, a cast to the scale dtype,
 * a multiply) with both scales fused as in the torchao issue "Unify scaled
 * INT8 matmul" (acc_i32.to(f32) * scale.to(f32)), and by the rowwise scale
 * shapes scale_a (M, 1), scale_b (1, N) stated in the PyTorch issue on
 * blockwise _scaled_mm.
 *
 *   acc[m,n] = sum_k a[m*lda + k] * b[n*ldb + k]            (exact int32)
 *   out[m*ldo + n] = (f32(acc) * scale_a[m*sa_m]) * scale_b[n*sb_n]
 * with f32() round-to-nearest-even and each product rounded to binary32 (no
 * fused multiply-add); BSMM_BF16 rounds that binary32 value once more.
 * out_dtype BSMM_I32 stores acc itself; the scales are then ignored and may
 * be NULL.  A scale stride of 0 broadcasts one scalar (tensorwise scaling).
 * a, b: int8.  scale_a, scale_b: fp32.  out: int32 / fp32 / bf16.
 * Any int8 code is accepted (-128 included), so |acc| <= K * 2^14; K above
 * 130944 (the largest multiple of 128 with K * 2^14 < 2^31) is rejected with
 * BSMM_ERR_UNSUPPORTED.
 */
bsmm_status bsmm_int8_rowwise(const int8_t* a, int64_t lda,
                              const int8_t* b, int64_t ldb,
                              const float* scale_a, int64_t sa_m,
                              const float* scale_b, int64_t sb_n,
                              void* out, int64_t ldo, bsmm_dtype out_dtype,
                              int64_t M, int64_t N, int64_t K,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * fp8 E4M3FN x E4M3FN with blockwise fp32 scales: one scale per row per
 * 128-long K block of A, one per 128 x 128 block of B.  Scale shapes
 * scale_a (M, K/128) and scale_b (K/128, N/128) as printed in the PyTorch
 * issue "torch._scaled_mm with blockwise scaling doesn't work with
 * torch.compile" (bug description).
 *
 *   out[m*ldo + n] = sum_kb  scale_a[m*sa_m + kb*sa_kb]
 *                          * scale_b[kb*sb_kb + (n/128)*sb_nb]
 *                          * sum_{k in block kb} A[m,k] * B[k,n]
 * accumulated in fp32 (one fp32 block partial per 128-K block, then one
 * multiply-add by the block's scale product); rounded to bf16 (RNE) or
 * stored as fp32.  a, b: E4M3FN bytes (OCP; NaN codes unsupported).  Scale
 * strides in elements; a stride of 0 broadcasts.
 */
bsmm_status bsmm_fp8_blockwise(const uint8_t* a, int64_t lda,
                               const uint8_t* b, int64_t ldb,
                               const float* scale_a, int64_t sa_m, int64_t sa_kb,
                               const float* scale_b, int64_t sb_kb, int64_t sb_nb,
                               void* out, int64_t ldo, bsmm_dtype out_dtype,
                               int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * bsmm_fp8_blockwise without a workspace argument and without allocating:
 * for callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * caller passes inputs and outputs as for bsmm_fp8_blockwise; the plan's
 * packed scales and split-K partials live in the library's static device
 * scratch, a 64 MiB array that every GPU the library runs on holds until
 * the process ends.  The call runs the plan bsmm_fp8_blockwise runs with a
 * workspace of bsmm_workspace_bytes(BSMM_OP_FP8_BLOCKWISE, 1, M, N, K,
 * out_dtype) bytes, and gives bit-identical results.  A problem whose plan
 * needs more than 64 MiB is rejected with BSMM_ERR_UNSUPPORTED before
 * anything is enqueued (its message gives the size).  All calls on one GPU
 * share that GPU's scratch: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race.  Other errors as for
 * bsmm_fp8_blockwise; BSMM_ERR_HIP if the scratch's device address cannot
 * be obtained.  It needs no clearing: every call writes what it reads.
 */
bsmm_status bsmm_fp8_blockwise_scratch(const uint8_t* a, int64_t lda,
                                       const uint8_t* b, int64_t ldb,
                                       const float* scale_a, int64_t sa_m, int64_t sa_kb,
                                       const float* scale_b, int64_t sb_kb, int64_t sb_nb,
                                       void* out, int64_t ldo, bsmm_dtype out_dtype,
                                       int64_t M, int64_t N, int64_t K, void* stream);

/*
 * fp8 E4M3FN x E4M3FN with fp32 scales per (row of A, 128-long K block) and
 * per (column of B, 128-long K block): 1 x 128 groups on both operands.
 *
 * The backward pass of the blockwise fp8 linear layer whose benchmark the
 * PyTorch issue "torch._scaled_mm with blockwise scaling doesn't work with
 * torch.compile" runs (forward and backward).  Its weight gradient
 * dW = dY^T X contracts over tokens, so both operands are quantised in
 * groups of 128 tokens: A = dY^T with scale_a [N_out, tokens/128], B = X
 * with scale_b [tokens/128, K_in].  (The input gradient dX = dY W is a
 * bsmm_fp8_blockwise call: the weight's 128 x 128 block scales serve the
 * transposed product unchanged.)
 *
 *   a        (m, k)   at a[m*lda + k]           E4M3FN codes, K-contiguous
 *   b        (k, n)   at b[n*ldb + k]           E4M3FN codes, K-contiguous
 *   scale_a  (m, kb)  at scale_a[m*sa_m + kb*sa_kb]    fp32
 *   scale_b  (kb, n)  at scale_b[kb*sb_kb + n*sb_n]    fp32
 *   out      (m, n)   at out[m*ldo + n]                fp32 or bf16
 *
 *   out(m,n) = sum_kb scale_a(m,kb) * scale_b(kb,n)
 *                     * sum_{k in block kb} a(m,k) * b(k,n)
 * accumulated in fp32 (each block's partial by the matrix core, then one
 * multiply by the binary32 scale product and one fused multiply-add per
 * element and block) and stored as bf16 (RNE) or fp32.
 *
 * Requirements: K a multiple of 128; a, b and lda, ldb 16-byte aligned;
 * scale strides >= 0.  N and M need not be multiples of anything.  The
 * kernel reads the scales repacked per K block, which the call writes to
 * the start of the workspace first: the workspace is required and must hold
 * at least bsmm_workspace_bytes(BSMM_OP_FP8_GROUPWISE, 1, M, N, K, out)
 * bytes (BSMM_ERR_ARG otherwise).  Returns the bsmm_status of the first
 * failed check, nothing written.
 */
bsmm_status bsmm_fp8_groupwise(const uint8_t* a, int64_t lda,
                               const uint8_t* b, int64_t ldb,
                               const float* scale_a, int64_t sa_m, int64_t sa_kb,
                               const float* scale_b, int64_t sb_kb, int64_t sb_n,
                               void* out, int64_t ldo, bsmm_dtype out_dtype,
                               int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Batched fp8 E4M3FN GEMM with e8m0 ("mxscale") scales per 128-long K block:
 * per row of x and per 128 x 128 block of w.  Layouts of the ROCm aiter PR
 * "Add opus fp8 mxscale BMM kernels for gfx950" (Motivation): m-major
 * x [M, G, K], w [G, N, K], x_scale [M, G, K/128], w_scale [G, N/128, K/128],
 * out [M, G, N]; and the batch-first layout x [G, M, K], out [G, M, N] named
 * in its test plan.  Both are expressed by strides (elements):
 *
 *   x       (g, m, k)   at x[g*x_sg + m*x_sm + k]
 *           m-major: x_sg = K, x_sm = G*K;  batch-first: x_sg = M*K, x_sm = K
 *   w       (g, n, k)   at w[g*w_sg + n*w_sn + k]
 *   x_scale (g, m, kb)  at x_scale[g*xs_sg + m*xs_sm + kb]
 *   w_scale (g, nb, kb) at w_scale[g*ws_sg + nb*ws_snb + kb]
 *   out     (g, m, n)   at out[g*o_sg + m*o_sm + n]
 *
 *   out(g,m,n) = sum_kb 2^(x_scale(g,m,kb) - 127) * 2^(w_scale(g,n/128,kb) - 127)
 *                       * sum_{k in block kb} x(g,m,k) * w(g,n,k)
 * accumulated in fp32 and stored as bf16 (RNE) or fp32.  Scale byte 255
 * (NaN) is unsupported.
 */
bsmm_status bsmm_fp8_mx_bmm(const uint8_t* x, int64_t x_sg, int64_t x_sm,
                            const uint8_t* w, int64_t w_sg, int64_t w_sn,
                            const uint8_t* x_scale, int64_t xs_sg, int64_t xs_sm,
                            const uint8_t* w_scale, int64_t ws_sg, int64_t ws_snb,
                            void* out, int64_t o_sg, int64_t o_sm,
                            bsmm_dtype out_dtype,
                            int64_t G, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * fp8 E4M3FN x E4M3FN with tensorwise or rowwise fp32 scales, an optional
 * bias and an optional result scale: the fp8 _scaled_mm of Inductor's
 * mm.py (tuned_scaled_mm; the Triton template's load_scales /
 * apply_scaling), with the shape rules the PyTorch blockwise issue prints
 * (tensorwise: both scales scalar; rowwise: scale_a (M, 1), scale_b (1, N)).
 *
 *   acc = sum_k a[m*lda + k] * b[n*ldb + k]        (fp32 accumulation)
 *   y   = acc * (scale_a[m*sa_m] * scale_b[n*sb_n])  (sa_m = sb_n = 0: tensorwise)
 *   y   = y + bias[n]                           (bias != NULL)
 *   y   = y * scale_result[0]                   (scale_result != NULL)
 *   out[m*ldo + n] = y as fp32, bf16 (RNE) or E4M3 (RNE, saturating)
 * Each step is one binary32 operation (no fused multiply-add).  scale_result
 * is named, not defined, by tuned_scaled_mm; here it scales the final value
 * before the conversion to the output type, for every output type.
 * a, b: E4M3FN bytes (NaN codes unsupported).  scale_a, scale_b: fp32 device
 * pointers.  bias: NULL or N values of bias_dtype (BSMM_F32 or BSMM_BF16;
 * ignored without a bias).  scale_result: NULL or a device pointer to one
 * fp32.  out_dtype: BSMM_F32, BSMM_BF16 or BSMM_E4M3.  Any N; K % 128 == 0;
 * otherwise the conventions above.  K == 0 writes (bias) * scale_result, the
 * value of an empty sum.
 */
bsmm_status bsmm_fp8_scaled_mm(const uint8_t* a, int64_t lda,
                               const uint8_t* b, int64_t ldb,
                               const float* scale_a, int64_t sa_m,
                               const float* scale_b, int64_t sb_n,
                               const void* bias, bsmm_dtype bias_dtype,
                               const float* scale_result,
                               void* out, int64_t ldo, bsmm_dtype out_dtype,
                               int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * fp8 E4M3FN x E4M3FN with e8m0 scales on 32-element K blocks of both
 * operands: the MX variants of _scaled_mm that Inductor's tuned_scaled_mm
 * (mm.py) routes away from its Triton templates, with the 32-element block
 * of the OCP microscaling formats (a reading: the pages do not print the
 * block).  One scale byte per row of A and per column of B for each 32-long
 * K chunk c:
 *
 *   out[m*ldo + n] = sum_c 2^(a_scale[m*as_m + c] - 127) * 2^(b_scale[n*bs_n + c] - 127)
 *                          * sum_{k in chunk c} A[m,k] * B[k,n]
 * accumulated in fp32 (the chunk scales are the hardware scale operands of
 * the matrix instruction) and stored as fp32 or bf16 (RNE).  a, b: E4M3FN
 * bytes, A row-major, B K-contiguous (b[n*ldb + k]).  Scale rows are
 * K/32 contiguous bytes.  K % 128 == 0, any N; scale byte 255 (NaN)
 * unsupported; otherwise the conventions above.
 */
bsmm_status bsmm_fp8_mx32_mm(const uint8_t* a, int64_t lda,
                             const uint8_t* b, int64_t ldb,
                             const uint8_t* a_scale, int64_t as_m,
                             const uint8_t* b_scale, int64_t bs_n,
                             void* out, int64_t ldo, bsmm_dtype out_dtype,
                             int64_t M, int64_t N, int64_t K,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Dynamic quantisation: bf16 / fp32 activations -> the 1-byte codes and the
 * scales the three matmuls above consume.  x is [M, K] row-major with row
 * stride ldx elements (x_dtype BSMM_BF16 or BSMM_F32); q is [M, K] with row
 * stride ldq bytes.  A scale is a dequantisation multiplier (x ~ code *
 * scale).  Quotients are correctly rounded binary32, codes are the nearest
 * ones (ties to even); e4m3 saturates at +-448.  A row or block whose fp32
 * scale is 0 -- amax 0, or amax below about 2^-141 so that the division
 * underflows -- stores scale 1 and +0 codes (the e8m0 quantiser: byte 127
 * and +0 codes when amax is 0).  NaN / infinite inputs are unsupported.
 *
 * Pointers are device pointers owned by the caller; x, q and scale must not
 * overlap.  Needs ldx % 8 == 0, ldq % 8 == 0, x 16-byte and q 8-byte
 * aligned, fp32 scales 4-byte aligned; scale strides >= 0 that give every row (block) its
 * own scale (BSMM_ERR_SCALE_SHAPE otherwise).  M == 0 does nothing; K == 0
 * writes only the int8 row scales (1.0).  Asynchronous on `stream`, as the
 * matmuls; errors from the arguments are returned before anything runs.
 *
 * int8, one scale per row (the symmetric per-row activation quantisation of
 * the torchao issue "Unify scaled INT8 matmul"):
 *   scale[m*s_m] = amax_m / 127,  q[m*ldq + k] = clamp(rne(x / scale), -127, 127)
 * K % 8 == 0, M <= 2^26.
 */
bsmm_status bsmm_quant_int8_rowwise(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                    int8_t* q, int64_t ldq,
                                    float* scale, int64_t s_m,
                                    int64_t M, int64_t K, void* stream);

/*
 * fp8 E4M3FN, one fp32 scale per 1 x 128 block of a row (the scale_a
 * (M, K/128) of the PyTorch issue "torch._scaled_mm with blockwise scaling
 * doesn't work with torch.compile"):
 *   scale[m*s_m + kb*s_kb] = amax_{m,kb} / 448,  q = rne_e4m3(x / scale)
 * K % 128 == 0, M * K / 128 < 2^30.  s_m = K/128, s_kb = 1 is the row-major
 * scale tensor; s_m = 1, s_kb = M its column-major transpose.
 */
bsmm_status bsmm_quant_fp8_blockwise(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                     uint8_t* q, int64_t ldq,
                                     float* scale, int64_t s_m, int64_t s_kb,
                                     int64_t M, int64_t K, void* stream);

/*
 * fp8 E4M3FN with an e8m0 scale per 1 x 128 block (the mxscale activations
 * of the ROCm aiter PR "Add opus fp8 mxscale BMM kernels for gfx950",
 * Motivation):  e = ceil(log2(amax / 448)) clamped to >= -127,
 *   scale[m*s_m + kb*s_kb] = e + 127 (byte),  q = rne_e4m3(x * 2^-e)
 * K % 128 == 0, M * K / 128 < 2^30.  The BMM's x [M, G, K] (m-major) or
 * [G, M, K] (batch-first) is M*G rows of K, its x_scale the matching
 * M*G rows of K/128 bytes (s_m = K/128, s_kb = 1).
 */
bsmm_status bsmm_quant_fp8_mx(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                              uint8_t* q, int64_t ldq,
                              uint8_t* scale, int64_t s_m, int64_t s_kb,
                              int64_t M, int64_t K, void* stream);

/*
 * The e8m0 quantiser on 1 x 32 blocks, for bsmm_fp8_mx32_mm's operands (the
 * 32-element block of the OCP microscaling formats; the same definition as
 * bsmm_quant_fp8_mx per 32-element block):  e = ceil(log2(amax / 448))
 * clamped to >= -127,  scale[m*s_m + c*s_kb] = e + 127,  q = rne_e4m3(x * 2^-e).
 * K % 32 == 0, M * K / 32 < 2^30.  s_m = K/32, s_kb = 1 is the a_scale row
 * layout of bsmm_fp8_mx32_mm; for its b_scale, quantise B's rows (N of K).
 */
bsmm_status bsmm_quant_fp8_mx32(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                uint8_t* q, int64_t ldq,
                                uint8_t* scale, int64_t s_m, int64_t s_kb,
                                int64_t M, int64_t K, void* stream);

/*
 * Quantisers for the backward pass of the blockwise fp8 linear layer that
 * the PyTorch issue "torch._scaled_mm with blockwise scaling doesn't work
 * with torch.compile" benchmarks (forward and backward).  Same rounding as
 * bsmm_quant_fp8_blockwise: scale = fl32(amax / 448), code =
 * e4m3_rne(fl32(x / scale)) saturating at +-448; a group whose scale is 0
 * stores scale 1 and +0 codes.
 *
 * bsmm_quant_fp8_columns: x [R, C] (bf16 or fp32, row stride ldx elements)
 * in groups of 128 consecutive rows of one column -- an activation or
 * output gradient with tokens along R, for the weight-gradient GEMM
 * bsmm_fp8_groupwise, which contracts over tokens.  Writes the codes
 * transposed, q_t [C, R] (row stride ldqt bytes), so that each row of q_t
 * is one operand row of that GEMM with its contraction contiguous; scale
 * (g, c) for group g < R/128 of column c at scale[g*s_g + c*s_c] (s_g = C,
 * s_c = 1 is the [R/128, C] array that GEMM takes as scale_b, its
 * transpose as scale_a).
 *   Requirements: R a multiple of 128 (at most 65535 groups), C of 8; x and
 *   ldx 16-byte aligned (ldx a multiple of 8 elements); q_t and ldqt 16-byte
 *   aligned; scale 4-byte aligned with strides that give every (g, c) its
 *   own element.
 *
 * bsmm_quant_fp8_weight: w [R, C] in 128 x 128 blocks (the weight blocks of
 * bsmm_fp8_blockwise's scale_b).  Writes the codes as they are, q [R, C]
 * (row stride ldq), and / or transposed, q_t [C, R] (row stride ldqt);
 * either may be NULL, not both.  scale (rb, cb) at scale[rb*s_r + cb*s_c].
 * The forward GEMM reads W [N, K] as B through q (scale_b = the transpose
 * of the [N/128, K/128] scales); the input gradient dX = dY W reads it as B
 * through q_t with the same scales as [K_contraction/128, N_out/128].
 *   Requirements: R and C multiples of 128; q and ldq 8-byte aligned; q_t
 *   and ldqt 16-byte aligned; as above otherwise.
 */
bsmm_status bsmm_quant_fp8_columns(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                   uint8_t* q_t, int64_t ldqt, float* scale, int64_t s_g,
                                   int64_t s_c, int64_t R, int64_t C, void* stream);
bsmm_status bsmm_quant_fp8_weight(const void* w, int64_t ldw, bsmm_dtype w_dtype, uint8_t* q,
                                  int64_t ldq, uint8_t* q_t, int64_t ldqt, float* scale,
                                  int64_t s_r, int64_t s_c, int64_t R, int64_t C,
                                  void* stream);

/*
 * bsmm_quant_fp8_blockwise_columns: both quantisations of one layer input
 * x [R, C] (tokens along R) from a single read of x -- the 1 x 128 row
 * blocks of bsmm_quant_fp8_blockwise (the forward GEMM's A: codes q [R, C],
 * scale (r, kb) at s_rows[r*sr_m + kb*sr_kb]) and the groups of 128 rows
 * down the columns of bsmm_quant_fp8_columns (the weight gradient's
 * operand: codes q_t [C, R], scale (g, c) at s_cols[g*sc_g + c*sc_c]).
 * Bit-identical to the two separate calls.
 *   Requirements: R and C multiples of 128 (at most 65535 groups of rows);
 *   x as for bsmm_quant_fp8_columns; q and ldq 8-byte aligned; q_t and ldqt
 *   16-byte aligned; both scale arrays 4-byte aligned with strides that give
 *   every block its own element.
 */
bsmm_status bsmm_quant_fp8_blockwise_columns(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                             uint8_t* q, int64_t ldq, float* s_rows,
                                             int64_t sr_m, int64_t sr_kb, uint8_t* q_t,
                                             int64_t ldqt, float* s_cols, int64_t sc_g,
                                             int64_t sc_c, int64_t R, int64_t C,
                                             void* stream);

/* Workspace bytes the fastest plan for this problem wants (0 if none). */
size_t bsmm_workspace_bytes(bsmm_op op, int64_t G, int64_t M, int64_t N,
                            int64_t K, bsmm_dtype out_dtype);

/* The plan the dispatcher picks for a problem (host only, no GPU needed). */
typedef struct {
  char variant[48];   /* kernel variant name                                */
  int32_t tile_m;     /* rows per workgroup tile                            */
  int32_t tile_n;     /* columns per workgroup tile                         */
  int32_t split_k;    /* number of K slices (1 = no split)                  */
  int32_t m_split;    /* rows handled by the bulk launch when M is split,   */
                      /* 0 when the whole M runs in one launch              */
  int64_t workspace;  /* workspace bytes this plan uses                     */
  int32_t source;     /* 0 table hit, 1 padded-M bucket, 2 heuristic,       */
                      /* 3 override                                         */
  char tail_variant[48]; /* variant of the launch for rows [m_split, M),   */
                         /* "" without an M-split                          */
  int32_t tail_split_k;  /* K slices of that launch (0 without M-split)    */
} bsmm_plan_info;

bsmm_status bsmm_query_plan(bsmm_op op, int64_t G, int64_t M, int64_t N,
                            int64_t K, bsmm_dtype out_dtype,
                            size_t workspace_bytes, bsmm_plan_info* info);

/*
 * Force a variant and/or split for subsequent calls in this process (tests
 * and tuning): variant NULL or "" keeps the dispatcher's choice, split_k <= 0
 * keeps its split.  Returns BSMM_ERR_ARG for an unknown variant name.  The
 * environment variables BSMM_FORCE_VARIANT and BSMM_FORCE_SPLITK set the same
 * override at load time; BSMM_LOG=1 prints each dispatch decision to stderr.
 * For plans with a split-K tail launch, BSMM_TAIL_SPLIT caps the tail's K
 * slices and BSMM_TAIL_VARIANT names its kernel (tuning only).
 */
bsmm_status bsmm_set_override(const char* variant, int split_k);

/*
 * Force an M-split for subsequent calls in this process (tests and tuning):
 * rows [0, m_split) run on the main launch (the dispatcher's or the
 * bsmm_set_override kernel), rows [m_split, M) on a second launch of
 * `tail_variant` with `tail_split` K slices.  Applies to calls with
 * m_split < M; m_split 0 removes it.  Returns BSMM_ERR_ARG for an unknown
 * variant or an m_split that is not a non-negative multiple of 64.
 */
bsmm_status bsmm_set_override_tail(int m_split, const char* tail_variant, int tail_split);

/*
 * Grid of the stream-K kernels (variants whose name contains "sk") for
 * subsequent calls in this process (tests and tuning).  0, the default, uses
 * as many workgroups as the device holds at once; any other count is also
 * correct, since no workgroup of that kernel waits for another: a tile split
 * over several workgroups is added up, in K order, by the last of them to
 * finish its part.  The count is further capped by the workspace (two
 * BM x BN partial tiles and 16 bytes per workgroup) and by the work.
 * Returns BSMM_ERR_ARG for a negative count.
 */
bsmm_status bsmm_set_streamk_grid(int workgroups);

/*
 * Matrix-core throughput probe (a measurement aid for the roofline; it
 * computes nothing of use).  Launches `workgroups` workgroups of four waves;
 * every wave issues `iters` x 8 independent matrix instructions on register
 * operands with no memory traffic in between: kind 0 the fp8 E4M3
 * 16 x 16 x 128 instruction with unit e8m0 scales (65536 flops each), kind 1
 * the int8 16 x 16 x 64 one (32768 ops each), kind 2 the int8 32 x 32 x 32
 * one (65536 ops each), kind 3 the fp8 32 x 32 x 64 one with unit e8m0
 * scales (131072 flops each).  Timing the launch gives the
 * rate the matrix cores sustain at the clock the device holds under that
 * load.  out: device buffer of workgroups * 256 floats (one per thread, so
 * the work is not optimised away).  Returns BSMM_ERR_ARG for a kind outside
 * 0..3 or a
 * non-positive count, BSMM_ERR_NULL for a NULL out.
 */
bsmm_status bsmm_mfma_probe(int kind, int workgroups, int iters, float* out, void* stream);

/*
 * Kernel timing for benchmarks.  While enabled (enable != 0), the main launch
 * of every call -- the one launch of a single-launch plan, the bulk launch
 * of an M-split plan; without the split-K reduction -- is bracketed by two
 * HIP events recorded on the call's stream.  Enabling (or disabling) clears
 * the record.  bsmm_timing_read waits for the recorded events and returns
 * the mean duration in milliseconds, the number of timed launches and the
 * variant name of the last one (truncated to name_len, may be NULL).
 * Returns BSMM_ERR_NULL for a NULL mean_ms or count, BSMM_ERR_HIP if an
 * event cannot be created or read.  Not meant for concurrent callers.
 */
bsmm_status bsmm_timing_enable(int enable);
bsmm_status bsmm_timing_read(double* mean_ms, int64_t* count, char* name,
                             size_t name_len);

/* Names of all kernel variants, separated by ','. */
const char* bsmm_variant_names(void);

const char* bsmm_status_string(bsmm_status s);
/* Thread-local detail of the last non-OK status returned on this thread. */
const char* bsmm_last_error(void);
int bsmm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSMM_H */
