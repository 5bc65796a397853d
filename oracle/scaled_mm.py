"""The three scaled matmuls, written out from their definitions (oracle; test
infrastructure only -- see the package docstring).

Notation: A is logically [M, K], B logically [K, N] (any numpy view; storage
order is the GPU side's business).  Scales are *dequantisation multipliers*:
a real operand value is code * scale (Inductor ``mm.py``, ``apply_scaling``
multiplies the accumulator by the row and column scales; torchao's CPU
``int_scaled_matmul`` multiplies the cast accumulator by the scale).

Exactness of the fast routes used below:

* int8: every partial sum of sum_k a*b is an integer below K * 127**2, so an
  fp64 matrix product of the integer-valued matrices is exact whenever
  K * 127**2 < 2**53 (checked).
* fp8: an E4M3 value is n * 2**-9 with |n| <= 229376, so a 128-long block
  partial sum_k nA*nB is an integer below 128 * 229376**2 < 2**43 and its fp64
  matrix product is exact.  Scale products sa*sb of two fp32 numbers are exact
  in fp64.  The only rounding before the final cast is fp64 accumulation of
  the scaled block partials, far below the tolerance.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .formats import (
    e4m3_numerator, e8m0_value, round_f32, bf16_bits_from_f32,
    bf16_bits_from_f64,
)

BLOCK = 128
TWO_M18 = 2.0 ** -18          # 2**-9 from each E4M3 operand


@dataclass
class Result:
    """exact: int64 accumulators (int8 path) or the fp64 value of the scaled
    matmul (fp8 paths).  out: the result in the requested output format
    (int32, float32, or uint16 bfloat16 bit patterns).  bound: the
    elementwise magnitude sum_k |a_deq| * |b_deq| (fp8 paths; None for int8).
    """
    exact: np.ndarray
    out: np.ndarray
    bound: np.ndarray | None = None
    info: dict = field(default_factory=dict)


def _idx(n, sel):
    return np.arange(n) if sel is None else np.asarray(sel, dtype=np.int64)


# ---------------------------------------------------------------------------
# int8 x int8, rowwise activation scale, per-column weight scale.
# torchao PR "Remove int_scaled_mm's dependency on triton for cpu":
#   c = int32 matmul(a, b); return c.to(scale dtype) * scale.
# torchao issue "Unify scaled INT8 matmul": both activation and weight scales
#   are fused; the scale step is acc_i32.to(f32) * scale.to(f32).
# Order of the two multiplies: (f32(acc) * scale_a[m]) * scale_b[n], left to
# right, each rounded to fp32 (the reading stated for this workload).
# ---------------------------------------------------------------------------

def int8_rowwise(a, b_kn, scale_a=None, scale_b=None, out_dtype="f32",
                 rows=None, cols=None) -> Result:
    a = np.asarray(a)
    b_kn = np.asarray(b_kn)
    if a.dtype != np.int8 or b_kn.dtype != np.int8:
        raise TypeError("int8 operands required")
    M, K = a.shape
    K2, N = b_kn.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    if K * 127 * 127 >= 2**53:
        raise ValueError("K too large for the exact fp64 route")
    r = _idx(M, rows)
    c = _idx(N, cols)
    # Exact int64 accumulators via an fp64 product of integer-valued matrices.
    acc = (a[r].astype(np.float64) @ b_kn[:, c].astype(np.float64))
    acc = acc.astype(np.int64)
    info = {"acc_absmax": int(np.abs(acc).max()) if acc.size else 0}
    if out_dtype == "i32":
        if acc.size and np.abs(acc).max() >= 2**31:
            raise OverflowError("int32 accumulator overflow")
        return Result(exact=acc, out=acc.astype(np.int32), info=info)
    sa = np.asarray(scale_a, dtype=np.float32).reshape(-1)[r]
    sb = np.asarray(scale_b, dtype=np.float32).reshape(-1)[c]
    acc32 = round_f32(acc)
    # Each step: exact fp64 product of two binary32 numbers, then one RNE to
    # binary32 -- i.e. an IEEE binary32 multiply with no fused rounding.
    y = round_f32(acc32.astype(np.float64) * sa[:, None].astype(np.float64))
    y = round_f32(y.astype(np.float64) * sb[None, :].astype(np.float64))
    if out_dtype == "f32":
        return Result(exact=acc, out=y, info=info)
    if out_dtype == "bf16":
        return Result(exact=acc, out=bf16_bits_from_f32(y), info=info)
    raise ValueError(out_dtype)


# ---------------------------------------------------------------------------
# fp8 E4M3 blockwise: scale_a [M, K/128] (one scale per row per 128-K block),
# scale_b [K/128, N/128] (one per 128x128 block of B).  Shapes from the
# PyTorch issue on blockwise _scaled_mm: (16640, 64) and (64, 40) for
# M=16640, K=8192, N=5120.  C[m,n] = sum_k (sa[m,k//128] * A[m,k]) *
# (sb[k//128, n//128] * B[k,n]), accumulated per K block.  The last block may
# be partial (ceil-div), which the oracle supports although the library does
# not.
# ---------------------------------------------------------------------------

def _blocks(K, block=BLOCK):
    return [(k0, min(K, k0 + block)) for k0 in range(0, K, block)]


def _finish_fp(C, Bd, out_dtype, info=None):
    if out_dtype == "f32":
        out = round_f32(C)
    elif out_dtype == "bf16":
        out = bf16_bits_from_f64(C)
    else:
        raise ValueError(out_dtype)
    return Result(exact=C, out=out, bound=Bd, info=info or {})


def fp8_blockwise(a, b_kn, scale_a, scale_b, out_dtype="bf16", rows=None,
                  cols=None) -> Result:
    a = np.asarray(a, dtype=np.uint8)
    b_kn = np.asarray(b_kn, dtype=np.uint8)
    M, K = a.shape
    K2, N = b_kn.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    sa = np.asarray(scale_a, dtype=np.float32)
    sb = np.asarray(scale_b, dtype=np.float32)
    KB = -(-K // BLOCK)
    NB = -(-N // BLOCK)
    if sa.shape != (M, KB) or sb.shape != (KB, NB):
        raise ValueError(f"scale shapes {sa.shape}, {sb.shape}; expected "
                         f"({M}, {KB}) and ({KB}, {NB})")
    r = _idx(M, rows)
    c = _idx(N, cols)
    nA, nanA = e4m3_numerator(a[r])
    nB, nanB = e4m3_numerator(b_kn[:, c])
    if nanA.any() or nanB.any():
        raise ValueError("NaN codes in the operands")
    nA = nA.astype(np.float64)
    nB = nB.astype(np.float64)
    C = np.zeros((len(r), len(c)))
    Bd = np.zeros((len(r), len(c)))
    for kb, (k0, k1) in enumerate(_blocks(K)):
        P = nA[:, k0:k1] @ nB[k0:k1, :]                 # exact integers
        Pabs = np.abs(nA[:, k0:k1]) @ np.abs(nB[k0:k1, :])
        s = (sa[r, kb].astype(np.float64)[:, None]
             * sb[kb, c // BLOCK].astype(np.float64)[None, :])   # exact
        C += s * P * TWO_M18
        Bd += np.abs(s) * Pabs * TWO_M18
    return _finish_fp(C, Bd, out_dtype)


# ---------------------------------------------------------------------------
# fp8 E4M3, 1 x 128 groups on both operands (the backward pass's weight
# gradient; PyTorch issue "torch._scaled_mm with blockwise scaling doesn't
# work with torch.compile", whose benchmark is a blockwise fp8 linear layer,
# forward and backward).  The pages give no layout for the backward GEMMs;
# reading: each operand's scale must be constant over each 128-long block of
# the contraction for the per-block dequantisation to factor out of the
# block's partial sum, and the finest such scale is one per (row of A or
# column of B, K block).  scale_a [M, K/128], scale_b [K/128, N]:
#   C[m, n] = sum_kb sa[m, kb] * sb[kb, n] * sum_{k in kb} A[m, k] B[k, n]
# ---------------------------------------------------------------------------

def fp8_groupwise(a, b_kn, scale_a, scale_b, out_dtype="bf16", rows=None,
                  cols=None) -> Result:
    a = np.asarray(a, dtype=np.uint8)
    b_kn = np.asarray(b_kn, dtype=np.uint8)
    M, K = a.shape
    K2, N = b_kn.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    sa = np.asarray(scale_a, dtype=np.float32)
    sb = np.asarray(scale_b, dtype=np.float32)
    KB = -(-K // BLOCK)
    if sa.shape != (M, KB) or sb.shape != (KB, N):
        raise ValueError(f"scale shapes {sa.shape}, {sb.shape}; expected "
                         f"({M}, {KB}) and ({KB}, {N})")
    r = _idx(M, rows)
    c = _idx(N, cols)
    nA, nanA = e4m3_numerator(a[r])
    nB, nanB = e4m3_numerator(b_kn[:, c])
    if nanA.any() or nanB.any():
        raise ValueError("NaN codes in the operands")
    nA = nA.astype(np.float64)
    nB = nB.astype(np.float64)
    C = np.zeros((len(r), len(c)))
    Bd = np.zeros((len(r), len(c)))
    for kb, (k0, k1) in enumerate(_blocks(K)):
        P = nA[:, k0:k1] @ nB[k0:k1, :]                 # exact integers
        Pabs = np.abs(nA[:, k0:k1]) @ np.abs(nB[k0:k1, :])
        s = (sa[r, kb].astype(np.float64)[:, None]
             * sb[kb, c].astype(np.float64)[None, :])   # exact
        C += s * P * TWO_M18
        Bd += np.abs(s) * Pabs * TWO_M18
    return _finish_fp(C, Bd, out_dtype)


# ---------------------------------------------------------------------------
# fp8 E4M3 with e8m0 "mxscale" per-128-K-block scales, batched over G
# (ROCm aiter PR, Motivation): m-major layout x [M, G, K],
# x_scale [M, G, K/128]; batch-first layout x [G, M, K], x_scale [G, M, K/128];
# w [G, N, K] and w_scale [G, N/128, K/128] in both.  For each group g:
#   out[g, m, n] = sum_k 2**(xs[g,m,k//128]-127) x[g,m,k]
#                        * 2**(ws[g,n//128,k//128]-127) w[g,n,k].
# The result is returned in the layout of x: [M, G, N] (m-major) or
# [G, M, N] (batch-first).
# ---------------------------------------------------------------------------

def fp8_mx_bmm(x, w, x_scale, w_scale, layout="m_major", out_dtype="bf16",
               groups=None, rows=None, cols=None) -> Result:
    x = np.asarray(x, dtype=np.uint8)
    w = np.asarray(w, dtype=np.uint8)
    xs = np.asarray(x_scale, dtype=np.uint8)
    ws = np.asarray(w_scale, dtype=np.uint8)
    if layout == "m_major":
        M, G, K = x.shape
    elif layout == "batch_first":
        G, M, K = x.shape
    else:
        raise ValueError(layout)
    G2, N, K2 = w.shape
    if G2 != G or K2 != K:
        raise ValueError("x / w shapes disagree")
    KB = -(-K // BLOCK)
    NB = -(-N // BLOCK)
    want_xs = (M, G, KB) if layout == "m_major" else (G, M, KB)
    if xs.shape != want_xs or ws.shape != (G, NB, KB):
        raise ValueError(f"scale shapes {xs.shape}, {ws.shape}; expected "
                         f"{want_xs} and {(G, NB, KB)}")
    gsel = _idx(G, groups)
    r = _idx(M, rows)
    c = _idx(N, cols)
    C = np.zeros((len(gsel), len(r), len(c)))
    Bd = np.zeros_like(C)
    for gi, g in enumerate(gsel):
        if layout == "m_major":
            xg = x[r, g, :]
            xsg = xs[r, g, :]
        else:
            xg = x[g][r]
            xsg = xs[g][r]
        wg = w[g][c]                # [n, K]
        wsg = ws[g]                 # [NB, KB]
        nX, nanX = e4m3_numerator(xg)
        nW, nanW = e4m3_numerator(wg)
        if nanX.any() or nanW.any():
            raise ValueError("NaN codes in the operands")
        if (xsg == 255).any() or (wsg == 255).any():
            raise ValueError("NaN e8m0 scale")
        nX = nX.astype(np.float64)
        nW = nW.astype(np.float64)
        for kb, (k0, k1) in enumerate(_blocks(K)):
            P = nX[:, k0:k1] @ nW[:, k0:k1].T          # exact integers
            Pabs = np.abs(nX[:, k0:k1]) @ np.abs(nW[:, k0:k1]).T
            s = (e8m0_value(xsg[:, kb])[:, None]
                 * e8m0_value(wsg[c // BLOCK, kb])[None, :])   # exact 2**e
            C[gi] += s * P * TWO_M18
            Bd[gi] += s * Pabs * TWO_M18
    if layout == "m_major":
        C = np.ascontiguousarray(C.transpose(1, 0, 2))
        Bd = np.ascontiguousarray(Bd.transpose(1, 0, 2))
    return _finish_fp(C, Bd, out_dtype)


# ---------------------------------------------------------------------------
# fp8 E4M3 _scaled_mm with tensorwise or rowwise fp32 scales (Inductor
# mm.py: tuned_scaled_mm and the Triton template's load_scales /
# apply_scaling; the PyTorch blockwise issue states the shape rules: both
# scales scalar, or scale_a (M, 1) and scale_b (1, N)).  The fp8 product is
# accumulated over all of K, then multiplied by a_scales[:, None] *
# b_scales[None, :] (or the scalar product); the optional bias [N] is added
# to the result (tuned_scaled_mm's docstring).  scale_result is only named
# there; the reading taken here: it multiplies the final value (after the
# bias) before the conversion to the output type.  Outputs: fp32, bf16, or
# E4M3 codes (nearest, ties to even, saturating at +-448).
#   C[m, n] = (sum_k A[m,k] B[k,n] * (sa[m] * sb[n]) + bias[n]) * sr
# ---------------------------------------------------------------------------

def fp8_scaled_mm(a, b_kn, scale_a, scale_b, bias=None, scale_result=None,
                  out_dtype="bf16", rows=None, cols=None) -> Result:
    a = np.asarray(a, dtype=np.uint8)
    b_kn = np.asarray(b_kn, dtype=np.uint8)
    M, K = a.shape
    K2, N = b_kn.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    sa = np.asarray(scale_a, dtype=np.float32)
    sb = np.asarray(scale_b, dtype=np.float32)
    if sa.size == 1 and sb.size == 1:
        sa_v = np.full(M, sa.reshape(-1)[0], np.float32)        # tensorwise
        sb_v = np.full(N, sb.reshape(-1)[0], np.float32)
    elif sa.shape == (M, 1) and sb.shape == (1, N):
        sa_v, sb_v = sa[:, 0], sb[0, :]                         # rowwise
    else:
        raise ValueError(f"scale shapes {sa.shape}, {sb.shape}: tensorwise needs two "
                         f"scalars, rowwise ({M}, 1) and (1, {N})")
    # every partial sum of the integer numerators is below K * 229376**2
    if K * 229376 ** 2 >= 2 ** 53:
        raise ValueError("K too large for the exact fp64 route")
    r = _idx(M, rows)
    c = _idx(N, cols)
    nA, nanA = e4m3_numerator(a[r])
    nB, nanB = e4m3_numerator(b_kn[:, c])
    if nanA.any() or nanB.any():
        raise ValueError("NaN codes in the operands")
    nA = nA.astype(np.float64)
    nB = nB.astype(np.float64)
    P = nA @ nB                                           # exact integers
    Pabs = np.abs(nA) @ np.abs(nB)
    s = sa_v[r].astype(np.float64)[:, None] * sb_v[c].astype(np.float64)[None, :]   # exact
    C = s * P * TWO_M18
    Bd = np.abs(s) * Pabs * TWO_M18
    if bias is not None:
        bv = np.asarray(bias, dtype=np.float64).reshape(-1)
        if bv.shape != (N,):
            raise ValueError(f"bias must have N = {N} elements")
        C = C + bv[c][None, :]
        Bd = Bd + np.abs(bv[c])[None, :]
    if scale_result is not None:
        sr = float(np.float32(scale_result))
        C = C * sr
        Bd = Bd * abs(sr)
    if out_dtype == "e4m3":
        from .quant import e4m3_encode_rne
        return Result(exact=C, out=e4m3_encode_rne(C), bound=Bd)
    return _finish_fp(C, Bd, out_dtype)


def compare_e4m3(codes, res: Result, gamma: float) -> dict:
    """E4M3 outputs.  If the GPU's binary32 value before the conversion is
    within tol = gamma * Bd of the exact value C, its nearest code q obeys
    |dec(q) - C| <= |dec(RNE(C)) - C| + 2 tol (both are nearest codes to
    points tol apart), and equals RNE(C) wherever C is farther than tol from
    every rounding boundary.  gamma: the fp32 accumulation error bound
    relative to Bd; with gamma = 0 (an exactly representable result) the
    codes must be identical."""
    from .formats import e4m3_value
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape != res.out.shape:
        return {"ok": False, "why": f"shape {codes.shape} vs {res.out.shape}"}
    C = res.exact
    tol = gamma * res.bound
    dq = e4m3_value(codes)
    if np.isnan(dq).any():
        return {"ok": False, "why": "NaN code"}
    dref = e4m3_value(res.out)
    lim = np.abs(dref - np.clip(C, -448.0, 448.0)) + 2 * tol
    bad = np.abs(dq - np.clip(C, -448.0, 448.0)) > lim
    # identical sign bit where the exact value has a sign (zero codes aside)
    bad |= (codes != res.out) & (tol == 0)
    rep = {"ok": not bad.any(), "violations": int(bad.sum()),
           "identical": float((codes == res.out).mean()) if codes.size else 1.0}
    if bad.any():
        rep["first"] = tuple(int(i) for i in np.argwhere(bad)[0])
    return rep


# ---------------------------------------------------------------------------
# fp8 E4M3 with MX block scales of 32 elements along K (the "MX variants" of
# _scaled_mm that Inductor's tuned_scaled_mm routes away from its Triton
# templates; 32 is the block of the OCP microscaling formats -- the reading
# taken for the block size, which the pages do not print): one e8m0 scale per
# row of A per 32-long K chunk, a_scale [M, K/32], and one per column of B
# per chunk, b_scale [N, K/32].
#   C[m, n] = sum_c 2**(a_scale[m,c]-127) * 2**(b_scale[n,c]-127)
#                   * sum_{k in chunk c} A[m,k] B[k,n]
# ---------------------------------------------------------------------------
MX_BLOCK = 32


def fp8_mx32_mm(a, b_kn, a_scale, b_scale, out_dtype="bf16", rows=None, cols=None) -> Result:
    a = np.asarray(a, dtype=np.uint8)
    b_kn = np.asarray(b_kn, dtype=np.uint8)
    M, K = a.shape
    K2, N = b_kn.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    KC = -(-K // MX_BLOCK)
    sa = np.asarray(a_scale, dtype=np.uint8)
    sb = np.asarray(b_scale, dtype=np.uint8)
    if sa.shape != (M, KC) or sb.shape != (N, KC):
        raise ValueError(f"scale shapes {sa.shape}, {sb.shape}; expected ({M}, {KC}) and "
                         f"({N}, {KC})")
    if (sa == 255).any() or (sb == 255).any():
        raise ValueError("NaN e8m0 scale")
    r = _idx(M, rows)
    c = _idx(N, cols)
    nA, nanA = e4m3_numerator(a[r])
    nB, nanB = e4m3_numerator(b_kn[:, c])
    if nanA.any() or nanB.any():
        raise ValueError("NaN codes in the operands")
    nA = nA.astype(np.float64)
    nB = nB.astype(np.float64)
    C = np.zeros((len(r), len(c)))
    Bd = np.zeros((len(r), len(c)))
    for ci, (k0, k1) in enumerate(_blocks(K, MX_BLOCK)):
        P = nA[:, k0:k1] @ nB[k0:k1, :]                 # exact integers
        Pabs = np.abs(nA[:, k0:k1]) @ np.abs(nB[k0:k1, :])
        s = e8m0_value(sa[r, ci])[:, None] * e8m0_value(sb[c, ci])[None, :]   # exact 2**e
        C += s * P * TWO_M18
        Bd += s * Pabs * TWO_M18
    return _finish_fp(C, Bd, out_dtype)


# ---------------------------------------------------------------------------
# Comparison rule.
#   integer accumulators and the int8 path's fp32/bf16 outputs: exact equality
#   (the GPU performs the same binary32 operations in the same order);
#   fp8 paths: relative Frobenius error <= 1e-2 and, elementwise,
#   |Y - C| <= 2**-7 * Bd with Bd = sum_k |a_deq| |b_deq| (Y must be exactly 0
#   where Bd = 0).
# ---------------------------------------------------------------------------

REL_FRO_TOL = 1e-2
ELEM_TOL = 2.0 ** -7


def compare(Y, res: Result, *, exact=False) -> dict:
    """Compare a GPU result Y (numpy; for exact comparisons in the same dtype
    as ``res.out``; otherwise convertible to fp64) with the oracle.
    Returns a report dict with key ``ok``."""
    if exact:
        Y = np.asarray(Y)
        ref = res.out
        if Y.shape != ref.shape:
            return {"ok": False, "why": f"shape {Y.shape} vs {ref.shape}"}
        if ref.dtype.kind == "f":
            a = np.ascontiguousarray(Y.astype(ref.dtype)).view(np.uint32)
            b = np.ascontiguousarray(ref).view(np.uint32)
        else:
            a, b = Y.astype(np.int64), ref.astype(np.int64)
        bad = np.argwhere(a != b)
        rep = {"ok": bad.shape[0] == 0, "mismatches": int(bad.shape[0])}
        if bad.shape[0]:
            rep["first"] = tuple(int(i) for i in bad[0])
        return rep
    Y = np.asarray(Y, dtype=np.float64)
    C = res.exact
    Bd = res.bound
    if Y.shape != C.shape:
        return {"ok": False, "why": f"shape {Y.shape} vs {C.shape}"}
    if not np.isfinite(Y).all():
        return {"ok": False, "why": "non-finite output",
                "nonfinite": int((~np.isfinite(Y)).sum())}
    err = np.abs(Y - C)
    nC = np.linalg.norm(C)
    rel = float(np.linalg.norm(Y - C) / nC) if nC > 0 else float(np.linalg.norm(Y))
    viol = err > ELEM_TOL * Bd
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(Bd > 0, err / Bd, np.where(err > 0, np.inf, 0.0))
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape) if ratio.size else ()
    rep = {
        "ok": bool(rel <= REL_FRO_TOL and not viol.any()),
        "rel_fro": rel,
        "violations": int(viol.sum()),
        "max_err_over_bound": float(ratio.max()) if ratio.size else 0.0,
        "worst": tuple(int(i) for i in worst),
    }
    return rep


def compare_within(Y, res: Result, gamma: float) -> dict:
    """A tighter check than ``compare`` for a result computed in binary32:
    if the GPU's binary32 value Y32 obeys |Y32 - C| <= tol = gamma * Bd (gamma
    the error bound of its fp32 accumulation, relative to Bd), then

    * fp32 output: |Y - C| <= tol;
    * bf16 output: Y is the round-to-nearest-even of a value in
      [C - tol, C + tol], and rounding is monotone, so
      RNE(C - tol) <= Y <= RNE(C + tol).

    Where Bd = 0 the interval is {0}.  ``Y``: float32 values, or uint16
    bfloat16 bit patterns (the oracle's bf16 representation)."""
    from .formats import bf16_bits_to_f64
    Y = np.asarray(Y)
    C = res.exact
    if Y.shape != C.shape:
        return {"ok": False, "why": f"shape {Y.shape} vs {C.shape}"}
    # the endpoints C +- tol are formed in fp64: widen by its rounding
    tol = gamma * res.bound + 2.0 ** -50 * np.abs(C)
    if Y.dtype == np.uint16:
        y = bf16_bits_to_f64(Y)
        lo = bf16_bits_to_f64(bf16_bits_from_f64(C - tol))
        hi = bf16_bits_to_f64(bf16_bits_from_f64(C + tol))
        bad = ~((y >= lo) & (y <= hi))
    else:
        y = Y.astype(np.float64)
        bad = ~(np.abs(y - C) <= tol)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(res.bound > 0, np.abs(y - C) / res.bound,
                         np.where(y != C, np.inf, 0.0))
    rep = {"ok": not bad.any(), "violations": int(bad.sum()),
           "max_err_over_bound": float(ratio.max()) if ratio.size else 0.0}
    if bad.any():
        rep["first"] = tuple(int(i) for i in np.argwhere(bad)[0])
    return rep
