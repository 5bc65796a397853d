"""Dynamic quantisation, written from its definition (oracle; test
infrastructure: only tests/, the smoke check and the benchmark's CPU
baseline use it; the library shares no code with it).

This is the step *before* the scaled matmul: it turns fp32 / bf16
activations into the low-precision codes and scales the three entry points
consume.  The recipe is the one the pages state for their workloads:

* int8, per row, symmetric: the torchao issue "Unify scaled INT8 matmul"
  quantises activations per row with ``scale = amax / 127`` and codes in
  [-127, 127];
* fp8 e4m3, 1 x 128 blocks with an fp32 scale ``amax / 448``: the
  blockwise activation scales of the PyTorch issue "torch._scaled_mm with
  blockwise scaling doesn't work with torch.compile" ([M, K/128]);
* fp8 e4m3, 1 x 128 blocks with an e8m0 (power-of-two) scale, the
  mxscale activations of the ROCm aiter PR "Add opus fp8 mxscale BMM
  kernels for gfx950" (Motivation): ``2**ceil(log2(amax / 448))``;
* for the backward pass of the blockwise fp8 linear layer that the PyTorch
  issue benchmarks: the weight's 128 x 128 blocks (the blockwise scale_b
  [K/128, N/128] of that issue, read as a weight's own blocks) with an
  fp32 scale ``amax / 448``, and 1 x 128 groups taken down the columns of
  an activation or gradient (128 consecutive tokens of one feature), the
  operands of the weight-gradient GEMM, whose contraction runs over tokens.

Readings: the quotient ``x / scale`` is the
binary32 quotient (correctly rounded); it is then rounded to the nearest
code, ties to even (to an even integer for int8, to the even mantissa for
e4m3), and e4m3 saturates at +-448.  A row or block whose amax is 0, or
whose fp32 scale underflows to 0 (amax below about 2**-141), gets scale 1
(e8m0 byte 127) and zero codes.  The e8m0 exponent is clamped below at -127
(byte 0): the scale stays the smallest one the format holds, and the codes
are then simply small; the top of the range is out of reach for finite
fp32.  The sign of a value that rounds to zero is kept in the e4m3 code
(0x80).  NaN and infinite inputs are outside the contract.
"""

from __future__ import annotations

import numpy as np

from .formats import e4m3_value, round_f32

BLOCK = 128
E4M3_MAX = 448.0

# the 127 non-negative finite E4M3FN codes (0x00 .. 0x7E) and their values,
# increasing with the code
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = e4m3_value(_POS_CODES)


def e4m3_encode_rne(v) -> np.ndarray:
    """Nearest E4M3FN code of each value (ties to the even code), saturating
    at +-448.  ``v`` is any float array without NaN; the search runs over the
    table of representable magnitudes, so it follows the definition rather
    than a bit-level formula."""
    v = np.asarray(v, dtype=np.float64)
    if np.isnan(v).any() or np.isinf(v).any():
        raise ValueError("e4m3_encode_rne: NaN or infinite input")
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")        # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def _f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def _div_f32(x, s) -> np.ndarray:
    """Correctly rounded binary32 quotient of binary32 operands (the fp64
    quotient of two binary32 values rounds to the same binary32 value)."""
    return round_f32(np.asarray(x, np.float64) / np.asarray(s, np.float64))


def quant_int8_rowwise(x):
    """Per-row int8: ``scale = fl32(amax / 127)`` (1 where amax is 0),
    ``q = clamp(round_half_even(fl32(x / scale)), -127, 127)``.
    ``x`` [M, K] fp32 (bf16 inputs widened exactly).  Returns (q int8
    [M, K], scale fp32 [M])."""
    x = _f32(x)
    amax = np.abs(x).max(axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    scale = _div_f32(amax, np.float32(127.0))
    zero = scale == 0
    scale = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    q = np.rint(_div_f32(x, scale[:, None]).astype(np.float64))
    q = np.where(zero[:, None], 0.0, q)
    return np.clip(q, -127, 127).astype(np.int8), scale


def _blocks(x, block=BLOCK):
    M, K = x.shape
    if K % block:
        raise ValueError(f"K={K} is not a multiple of {block}")
    return x.reshape(M, K // block, block)


def quant_fp8_blockwise(x):
    """1 x 128 blocks, fp32 scale ``fl32(amax / 448)`` (1 where amax is 0),
    codes ``e4m3_rne(fl32(x / scale))``.  Returns (codes uint8 [M, K],
    scale fp32 [M, K/128])."""
    x = _f32(x)
    xb = _blocks(x)
    amax = np.abs(xb).max(axis=2)
    scale = _div_f32(amax, np.float32(E4M3_MAX))
    zero = scale == 0
    scale = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    t = np.where(zero[:, :, None], 0.0, _div_f32(xb, scale[:, :, None]))
    codes = e4m3_encode_rne(t)
    return codes.reshape(x.shape), scale


def e8m0_exponent(amax) -> np.ndarray:
    """``ceil(log2(amax / 448))`` (0 where amax is 0), clamped below at
    -127: the smallest e with ``amax <= 448 * 2**e``.  It is read off the
    binade of the fp64 ratio; 448 = 7 * 2**6, so amax / 448 is a power of two
    only when amax is 7 times one, and then the fp64 quotient is exact; any
    other binary32 amax gives a ratio about 2**-24 (relative) or more away
    from every power of two, far above the fp64 rounding."""
    r = np.asarray(amax, dtype=np.float64) / E4M3_MAX
    f, e = np.frexp(r)                  # r = f * 2**e, f in [0.5, 1)
    ex = np.where(f == 0.5, e - 1, e)   # an exact power of two: its own exponent
    ex = np.where(np.asarray(amax) == 0, 0, ex)
    return np.maximum(ex, -127).astype(np.int64)


def quant_fp8_mx(x, block=BLOCK):
    """1 x ``block`` blocks (128, or 32 for the MX formats' block) with an
    e8m0 scale ``2**e``, ``e = ceil(log2(amax/448))`` (byte e + 127; 127 where
    amax is 0), codes ``e4m3_rne(x * 2**-e)`` (a power-of-two scaling, exact
    in fp64).  Returns (codes uint8 [M, K], scale bytes uint8 [M, K/block])."""
    x = _f32(x)
    xb = _blocks(x, block)
    amax = np.abs(xb).max(axis=2)
    ex = e8m0_exponent(amax)
    codes = e4m3_encode_rne(np.ldexp(xb.astype(np.float64), -ex[:, :, None]))
    codes = np.where((amax == 0)[:, :, None], np.uint8(0), codes).astype(np.uint8)
    return codes.reshape(x.shape), (ex + 127).astype(np.uint8)


def quant_fp8_weight_blocks(w):
    """128 x 128 blocks, fp32 scale ``fl32(amax / 448)`` per block (1 where
    amax is 0), codes ``e4m3_rne(fl32(w / scale))``.  Returns (codes uint8
    [R, C], scale fp32 [R/128, C/128])."""
    w = _f32(w)
    R, C = w.shape
    if R % BLOCK or C % BLOCK:
        raise ValueError(f"shape {w.shape} is not a multiple of {BLOCK} x {BLOCK}")
    wb = w.reshape(R // BLOCK, BLOCK, C // BLOCK, BLOCK)
    amax = np.abs(wb).max(axis=(1, 3))
    scale = _div_f32(amax, np.float32(E4M3_MAX))
    zero = scale == 0
    scale = np.where(zero, np.float32(1.0), scale).astype(np.float32)
    s4 = scale[:, None, :, None]
    t = np.where(zero[:, None, :, None], 0.0, _div_f32(wb, s4))
    codes = e4m3_encode_rne(t)
    return codes.reshape(R, C), scale


def quant_fp8_columns(x):
    """1 x 128 groups down the columns: for each column c and each run of
    128 rows, fp32 scale ``fl32(amax / 448)`` (1 where amax is 0), codes
    ``e4m3_rne(fl32(x / scale))``.  The codes are returned transposed, one
    row per column of x with its rows contiguous (the layout a GEMM whose
    contraction runs over x's rows reads).  Returns (codes uint8 [C, R],
    scale fp32 [R/128, C])."""
    codes_t, scale_t = quant_fp8_blockwise(_f32(x).T)
    return codes_t, np.ascontiguousarray(scale_t.T)
