"""Number formats, written from their definitions (oracle; test infrastructure).

* OCP 8-bit E4M3FN (the "fp8 e4m3" of the pages; the ROCm aiter PR targets
  gfx950, whose fp8 is the OCP format): sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, no infinities, NaN = S.1111.111, largest finite 448,
  smallest subnormal 2**-9.
* OCP E8M0 ("e8m0" block scale in the aiter PR): an unsigned biased exponent,
  value 2**(b - 127); 255 is NaN; there is no zero.
* IEEE-754 binary32 and bfloat16 (8 exponent bits, 8 significant bits) with
  round-to-nearest, ties-to-even.
"""

from __future__ import annotations

import numpy as np


def e4m3_numerator(codes) -> tuple[np.ndarray, np.ndarray]:
    """Integer form of E4M3FN codes.

    For code b with s = b>>7, e = (b>>3)&15, m = b&7 the value is
    (-1)**s * n * 2**-9 with n = m if e == 0 else (8 + m) * 2**(e - 1).
    Returns (n as int64, nan mask).  |n| <= 229376 (= 448 * 2**9).
    """
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = b >> 7
    e = (b >> 3) & 15
    m = b & 7
    n = np.where(e == 0, m, (8 + m) << np.maximum(e - 1, 0))
    n = np.where(s == 1, -n, n)
    nan = (e == 15) & (m == 7)
    return n.astype(np.int64), nan


def e4m3_value(codes) -> np.ndarray:
    """E4M3FN codes -> fp64 values (exact), NaN for the NaN codes."""
    n, nan = e4m3_numerator(codes)
    v = np.ldexp(n.astype(np.float64), -9)
    # keep the sign of negative zero
    b = np.asarray(codes, dtype=np.uint8)
    v = np.where((n == 0) & (b >= 128), -0.0, v)
    return np.where(nan, np.nan, v)


def e8m0_value(codes) -> np.ndarray:
    """E8M0 codes -> fp64 values 2**(b - 127), NaN for 255."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    v = np.ldexp(np.ones(b.shape), b - 127)
    return np.where(b == 255, np.nan, v)


def round_f32(x) -> np.ndarray:
    """Round fp64 (or exact integer) values to binary32, ties to even.

    numpy's float64 -> float32 conversion is the IEEE conversion in the
    default rounding mode (round-to-nearest-even); an int64 below 2**53 is
    first converted to fp64 exactly.
    """
    x = np.asarray(x)
    if x.dtype.kind in "iu":
        if np.any(np.abs(x) >= 2**53):
            raise ValueError("integer too large for an exact fp64 step")
        x = x.astype(np.float64)
    return x.astype(np.float32)


def bf16_bits_from_f32(x) -> np.ndarray:
    """binary32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Keep the upper 16 bits after adding 0x7FFF plus the lowest kept bit
    (the standard integer form of RNE on the dropped 16 bits).  NaN stays a
    quiet NaN.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    return np.where(nan, np.uint16(0x7FC0) | ((u >> 16).astype(np.uint16) & 0x8000), r)


def bf16_bits_from_f64(x) -> np.ndarray:
    """fp64 -> bfloat16 bit patterns with a single round-to-nearest-even.

    Written from the format: a finite nonzero x = f * 2**e with f in
    [0.5, 1); bfloat16 keeps 8 significant bits in binades down to 2**-126,
    below that a fixed quantum of 2**-133 (subnormals); values that round
    past the largest finite (2 - 2**-7) * 2**127 become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    f, e = np.frexp(ax)
    binade = np.maximum(e - 1, -126)
    quantum_e = binade - 7
    mag = np.ldexp(np.rint(np.ldexp(ax, -quantum_e)), quantum_e)
    mag = np.where(mag > (2.0 - 2.0**-7) * 2.0**127, np.inf, mag)
    mag = np.where(ax == 0, 0.0, mag)
    y = np.copysign(mag, x).astype(np.float32)   # exact: 8 significant bits
    bits = (y.view(np.uint32) >> 16).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> fp64 values (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
