"""Seeded synthetic inputs for the block-scaled matmul.

This module only *produces* operands: low-precision codes (int8 bytes, OCP
fp8 E4M3FN bytes) and their scales (fp32 or e8m0 bytes), shaped like the
workloads the pages describe.  It holds none of the matmul's arithmetic: no
decode, no dot product, no scale application.  Both the CPU oracle and the
GPU path consume the bytes it returns, so parity never depends on how the
operands were quantised.

Recipe (all draws from ``numpy.random.default_rng(seed)``, taken in fp64 and
cast to fp32 before quantisation):

* int8 rowwise / per-column: ``scale = amax / 127`` (fp32),
  ``q = clamp(round_half_even(x / scale), -127, 127)``.  The symmetric
  [-127, 127] range follows the symmetric affine-quantisation primitives
  named in the torchao issue "Unify scaled INT8 matmul".
* fp8 blockwise (1x128 activation blocks, 128x128 weight blocks):
  ``scale = amax / 448`` (fp32), ``q = RNE_e4m3(x / scale)`` saturating at
  +-448.  The block shapes are those of the blockwise ``_scaled_mm`` scale
  tensors printed in the PyTorch issue "torch._scaled_mm with blockwise
  scaling doesn't work with torch.compile".
* fp8 mx (e8m0 per 128-K block): ``scale = 2**ceil(log2(amax / 448))``
  computed exactly, stored as the biased exponent byte, then
  ``q = RNE_e4m3(x / scale)`` (never saturates).  Layouts follow the ROCm
  aiter PR "Add opus fp8 mxscale BMM kernels for gfx950", Motivation.
* A block or row whose amax is 0 gets scale 1.0 (e8m0 byte 127); its codes
  are all zero.

Operand storage: A is ``[M, K]`` row-major; B is logically ``[K, N]`` and is
stored K-contiguous, i.e. as an ``[N, K]`` row-major array, which is the
column-major ``mat_b`` that ``_scaled_mm`` requires (Inductor ``mm.py``,
``check_supported_striding``).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "e4m3_encode",
    "quant_int8_rows",
    "quant_fp8_blocks_fp32",
    "quant_fp8_blocks_e8m0",
    "int8_rowwise_inputs",
    "fp8_blockwise_inputs",
    "fp8_mx_bmm_inputs",
    "fp8_scaled_mm_inputs",
    "fp8_mx32_inputs",
    "fp8_groupwise_inputs",
    "config_inputs",
    "activations",
    "CONFIGS",
]

BLOCK = 128
E4M3_MAX = 448.0
_CHUNK_ELEMS = 1 << 24  # rows are drawn in chunks of about this many values


def _draw(rng, kind, shape, *, loc=0.0, scale=1.0, df=3.0):
    """Draw ``shape`` values of ``kind`` in fp64 row-chunk by row-chunk, cast
    to fp32.  Chunking bounds host memory; the stream is the same as one call.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1) if len(shape) > 1 else out.reshape(-1, 1)
    rows, cols = flat.shape
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        n = (r1 - r0) * cols
        if kind == "normal":
            v = loc + scale * rng.standard_normal(n)
        elif kind == "t":
            v = rng.standard_t(df, n)
        else:
            raise ValueError(kind)
        flat[r0:r1] = v.reshape(r1 - r0, cols).astype(np.float32)
    return out


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round fp32/fp64 values to the nearest OCP E4M3FN code (ties to even),
    saturating to +-448.  Returns uint8 codes.  NaN inputs are not supported.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("e4m3_encode: NaN input")
    neg = np.signbit(x)
    ax = np.abs(x)
    _, e = np.frexp(ax)                 # ax = f * 2**e, f in [0.5, 1)
    expo = np.maximum(e - 1, -6)        # binade, clamped to the subnormal one
    quantum = np.ldexp(1.0, expo - 3)   # 3 mantissa bits
    mag = np.rint(ax / quantum) * quantum   # power-of-two division: exact
    mag = np.minimum(mag, E4M3_MAX)
    n = np.rint(mag * 512.0).astype(np.int64)   # integer numerator of 2**-9
    # n < 8: subnormal, code = n.  Otherwise n = (8 + m) * 2**(E - 1).
    lg = np.frexp(n.astype(np.float64))[1].astype(np.int64) - 1  # floor(log2 n)
    big = n >= 8
    E = np.where(big, lg - 2, 0)
    m = np.where(big, (n >> np.maximum(E - 1, 0)) - 8, n)
    code = (E << 3) | m
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def quant_int8_rows(x: np.ndarray):
    """Per-row symmetric int8 quantisation of a 2-D fp32 array.
    Returns (codes int8 [R, C], scale fp32 [R])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.rint(x / scale[:, None])
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, scale


def _block_view(x2d, br, bc):
    r, c = x2d.shape
    if r % br or c % bc:
        raise ValueError(f"shape {x2d.shape} not divisible by blocks {br}x{bc}")
    return x2d.reshape(r // br, br, c // bc, bc)


def quant_fp8_blocks_fp32(x: np.ndarray, br: int, bc: int):
    """Quantise a 2-D fp32 array in ``br x bc`` blocks to E4M3 with an fp32
    scale ``amax / 448`` per block.  Returns (codes uint8, scale fp32
    [R/br, C/bc])."""
    x = np.asarray(x, dtype=np.float32)
    xb = _block_view(x, br, bc)
    amax = np.abs(xb).max(axis=(1, 3))
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    cb = _block_view(codes, br, bc)
    step = max(1, _CHUNK_ELEMS // (br * x.shape[1]))
    for i0 in range(0, xb.shape[0], step):
        i1 = min(xb.shape[0], i0 + step)
        q = (xb[i0:i1] / scale[i0:i1, None, :, None]).astype(np.float32)
        cb[i0:i1] = e4m3_encode(q)
    return codes, scale


def _e8m0_exponent(amax: np.ndarray) -> np.ndarray:
    """ceil(log2(amax / 448)) computed exactly (amax fp32 -> fp64 division)."""
    r = np.asarray(amax, dtype=np.float64) / E4M3_MAX
    f, e = np.frexp(r)
    ex = np.where(f == 0.5, e - 1, e)
    return np.where(amax == 0, 0, ex).astype(np.int64)


def quant_fp8_blocks_e8m0(x: np.ndarray, br: int, bc: int):
    """Quantise in ``br x bc`` blocks with power-of-two scales
    ``2**ceil(log2(amax/448))``.  Returns (codes uint8, scale bytes uint8
    [R/br, C/bc]) where the byte is the exponent biased by 127."""
    x = np.asarray(x, dtype=np.float32)
    xb = _block_view(x, br, bc)
    amax = np.abs(xb).max(axis=(1, 3))
    ex = _e8m0_exponent(amax)
    if (ex < -127).any() or (ex > 127).any():
        raise ValueError("block scale outside the e8m0 range")
    codes = np.empty(x.shape, dtype=np.uint8)
    cb = _block_view(codes, br, bc)
    step = max(1, _CHUNK_ELEMS // (br * x.shape[1]))
    for i0 in range(0, xb.shape[0], step):
        i1 = min(xb.shape[0], i0 + step)
        q = np.ldexp(xb[i0:i1].astype(np.float64), -ex[i0:i1, None, :, None])
        cb[i0:i1] = e4m3_encode(q)
    return codes, (ex + 127).astype(np.uint8)


def activations(shape, seed, *, dist="normal", row_scale_log2=None):
    """Unquantised fp32 activations for the dynamic quantisers: ``normal(0,1)``
    or ``standard_t(3)`` (``dist="t"``) drawn as above.  ``row_scale_log2``
    (lo, hi) multiplies each row (all but the last axis) by ``2**u``, u
    uniform in [lo, hi), drawn after the values, so rows span many binades.
    """
    rng = np.random.default_rng(seed)
    x = _draw(rng, dist, shape)
    if row_scale_log2 is not None:
        lo, hi = row_scale_log2
        rows = x.reshape(-1, x.shape[-1])
        f = np.exp2(rng.uniform(lo, hi, rows.shape[0])).astype(np.float32)
        rows *= f[:, None]
    return x


# ---------------------------------------------------------------------------
# Whole problems.  Every function returns host numpy arrays in the storage
# layout the C ABI consumes.
# ---------------------------------------------------------------------------

def int8_rowwise_inputs(M, N, K, seed, *, kind="uniform_int", w_std=0.02):
    """int8 rowwise problem.

    kind="uniform_int": codes uniform in [-127, 127], scales uniform in
    [1e-3, 1e-2] (the tiny int8 workload).  kind="dynamic_quant": X ~ N(0,1)
    [M,K] quantised per row, W ~ N(0, w_std) logical [K,N] quantised per
    output column.

    Returns dict(a int8 [M,K], b_nk int8 [N,K], scale_a fp32 [M],
    scale_b fp32 [N]).
    """
    rng = np.random.default_rng(seed)
    if kind == "uniform_int":
        a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
        b_kn = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
        sa = rng.uniform(1e-3, 1e-2, size=M).astype(np.float32)
        sb = rng.uniform(1e-3, 1e-2, size=N).astype(np.float32)
        b_nk = np.ascontiguousarray(b_kn.T)
    elif kind == "dynamic_quant":
        x = _draw(rng, "normal", (M, K))
        w_kn = _draw(rng, "normal", (K, N), scale=w_std)
        a, sa = quant_int8_rows(x)
        del x
        b_nk, sb = quant_int8_rows(np.ascontiguousarray(w_kn.T))
    else:
        raise ValueError(kind)
    return dict(a=a, b_nk=b_nk, scale_a=sa, scale_b=sb)


def fp8_blockwise_inputs(M, N, K, seed, *, dist="normal"):
    """fp8 blockwise problem: A [M,K] with 1x128 scales [M, K/128]; B logical
    [K,N] with 128x128 scales [K/128, N/128]; both ~ N(0,1) (or student-t
    df=3 with dist="t").

    Returns dict(a uint8 [M,K], b_nk uint8 [N,K], scale_a fp32 [M,K/128],
    scale_b fp32 [K/128,N/128])."""
    rng = np.random.default_rng(seed)
    a_f = _draw(rng, dist, (M, K))
    a, sa = quant_fp8_blocks_fp32(a_f, 1, BLOCK)
    del a_f
    b_kn = _draw(rng, dist, (K, N))
    b_q, sb = quant_fp8_blocks_fp32(b_kn, BLOCK, BLOCK)
    del b_kn
    b_nk = np.ascontiguousarray(b_q.T)
    return dict(a=a, b_nk=b_nk, scale_a=sa, scale_b=sb)


def fp8_scaled_mm_inputs(M, N, K, seed, *, scaling="rowwise", bias=None, dist="normal"):
    """fp8 _scaled_mm problem with tensorwise or rowwise fp32 scales: A [M,K]
    quantised per row (rowwise) or as a whole (tensorwise) with scale
    amax/448, B logical [K,N] per output column or as a whole.  ``bias``:
    None, "f32" (N(0,1) values) or "bf16" (the same, cut to bf16-exact
    values).

    Returns dict(a uint8 [M,K], b_nk uint8 [N,K], scale_a fp32 (M,1) or (),
    scale_b fp32 (1,N) or (), bias fp32 [N] or None)."""
    rng = np.random.default_rng(seed)
    a_f = _draw(rng, dist, (M, K))
    b_kn = _draw(rng, dist, (K, N))
    if scaling == "rowwise":
        a, sa = quant_fp8_blocks_fp32(a_f, 1, K)            # sa [M, 1]
        b_q, sb = quant_fp8_blocks_fp32(b_kn, K, 1)         # sb [1, N]
    elif scaling == "tensorwise":
        a, sa = quant_fp8_blocks_fp32(a_f, M, K)
        b_q, sb = quant_fp8_blocks_fp32(b_kn, K, N)
        sa, sb = sa.reshape(()), sb.reshape(())
    else:
        raise ValueError(scaling)
    bv = None
    if bias is not None:
        bv = _draw(rng, "normal", (N,))
        if bias == "bf16":
            bv = (bv.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    return dict(a=a, b_nk=np.ascontiguousarray(b_q.T), scale_a=sa, scale_b=sb, bias=bv)


def fp8_mx32_inputs(M, N, K, seed, *, dist="normal"):
    """fp8 MX problem with 32-element K blocks: A [M,K] quantised per row per
    32-long K chunk, B logical [K,N] per column per chunk, e8m0 scales
    ``2**ceil(log2(amax/448))``.

    Returns dict(a uint8 [M,K], b_nk uint8 [N,K], a_scale uint8 [M,K/32],
    b_scale uint8 [N,K/32])."""
    rng = np.random.default_rng(seed)
    a_f = _draw(rng, dist, (M, K))
    a, sa = quant_fp8_blocks_e8m0(a_f, 1, 32)
    del a_f
    b_kn = _draw(rng, dist, (K, N))
    b_q, sb = quant_fp8_blocks_e8m0(b_kn, 32, 1)          # sb [K/32, N]
    del b_kn
    return dict(a=a, b_nk=np.ascontiguousarray(b_q.T), a_scale=sa,
                b_scale=np.ascontiguousarray(sb.T))


def fp8_groupwise_inputs(M, N, K, seed, *, dist="normal"):
    """fp8 problem with 1x128 fp32 scales on both operands: A [M,K] quantised
    per row per 128-long K block (scale_a [M, K/128]), B logical [K,N] per
    column per 128-long K block (scale_b [K/128, N]).  This is the shape of a
    weight-gradient GEMM, whose contraction runs over tokens.

    Returns dict(a uint8 [M,K], b_nk uint8 [N,K], scale_a fp32 [M,K/128],
    scale_b fp32 [K/128,N])."""
    rng = np.random.default_rng(seed)
    a_f = _draw(rng, dist, (M, K))
    a, sa = quant_fp8_blocks_fp32(a_f, 1, BLOCK)
    del a_f
    b_kn = _draw(rng, dist, (K, N))
    b_q, sb = quant_fp8_blocks_fp32(b_kn, BLOCK, 1)
    del b_kn
    return dict(a=a, b_nk=np.ascontiguousarray(b_q.T), scale_a=sa, scale_b=sb)


def fp8_mx_bmm_inputs(G, M, N, K, seed, *, layout="m_major", dist="normal"):
    """fp8 mx BMM problem with e8m0 per-128-K-block scales.

    layout="m_major": x [M,G,K], x_scale [M,G,K/128].
    layout="batch_first": x [G,M,K], x_scale [G,M,K/128].
    w [G,N,K], w_scale [G,N/128,K/128] in both layouts.
    Values are drawn in the stored layout's order.
    """
    rng = np.random.default_rng(seed)
    kb = K // BLOCK
    xshape = (M, G, K) if layout == "m_major" else (G, M, K)
    x_f = _draw(rng, dist, xshape)
    x_q, xs = quant_fp8_blocks_e8m0(x_f.reshape(-1, K), 1, BLOCK)
    del x_f
    x_q = x_q.reshape(xshape)
    xs = xs.reshape(xshape[0], xshape[1], kb)
    w_f = _draw(rng, dist, (G, N, K))
    w_q, ws = quant_fp8_blocks_e8m0(w_f.reshape(G * N, K), BLOCK, BLOCK)
    del w_f
    w_q = w_q.reshape(G, N, K)
    ws = ws.reshape(G, N // BLOCK, kb)
    if layout not in ("m_major", "batch_first"):
        raise ValueError(layout)
    return dict(x=x_q, w=w_q, x_scale=xs, w_scale=ws, layout=layout)


# The five workloads (shapes, distributions and seeds).  "c4" is run at three
# values of M: single-token decode, a 128-row decode batch and an 8192-row
# prefill, the serving regimes the aiter PR benchmarks.
CONFIGS = {
    "c1": dict(op="int8", M=64, N=128, K=256, seed=1, kind="uniform_int",
               out="f32"),
    "c2": dict(op="int8", M=8192, N=4096, K=4096, seed=2,
               kind="dynamic_quant", out="bf16"),
    "c3": dict(op="fp8_blockwise", M=16640, N=5120, K=8192, seed=3,
               out="bf16"),
    "c4_m1": dict(op="mx", G=8, M=1, N=1024, K=4096, seed=41,
                  layout="m_major", dist="normal", out="bf16"),
    "c4_m128": dict(op="mx", G=8, M=128, N=1024, K=4096, seed=42,
                    layout="m_major", dist="normal", out="bf16"),
    "c4_m8192": dict(op="mx", G=8, M=8192, N=1024, K=4096, seed=43,
                     layout="m_major", dist="normal", out="bf16"),
    "c5": dict(op="mx", G=2, M=9000, N=2048, K=7168, seed=5,
               layout="batch_first", dist="t", out="f32"),
    # the blockwise issue's shape under the rowwise scaling it names, with a
    # bf16 bias (the fp8 scaled_mm epilogue)
    "c3r": dict(op="fp8_scaled_mm", M=16640, N=5120, K=8192, seed=3,
                scaling="rowwise", bias="bf16", out="bf16"),
    # the same shape with 32-element MX (e8m0) block scales
    "c3x": dict(op="fp8_mx32", M=16640, N=5120, K=8192, seed=3, out="bf16"),
    # the backward pass of that layer (y = x w^T with x [16640, 8192] and
    # w [5120, 8192]): the input gradient dx = dy w, a blockwise GEMM over
    # the 5120 output features, and the weight gradient dw = dy^T x, a
    # groupwise GEMM over the 16640 tokens
    "c3d": dict(op="fp8_blockwise", M=16640, N=8192, K=5120, seed=31, out="bf16"),
    "c3w": dict(op="fp8_groupwise", M=5120, N=8192, K=16640, seed=32, out="bf16"),
}


def config_inputs(name: str):
    c = CONFIGS[name]
    if c["op"] == "int8":
        return int8_rowwise_inputs(c["M"], c["N"], c["K"], c["seed"],
                                   kind=c["kind"])
    if c["op"] == "fp8_blockwise":
        return fp8_blockwise_inputs(c["M"], c["N"], c["K"], c["seed"])
    if c["op"] == "fp8_mx32":
        return fp8_mx32_inputs(c["M"], c["N"], c["K"], c["seed"])
    if c["op"] == "fp8_groupwise":
        return fp8_groupwise_inputs(c["M"], c["N"], c["K"], c["seed"])
    if c["op"] == "fp8_scaled_mm":
        return fp8_scaled_mm_inputs(c["M"], c["N"], c["K"], c["seed"],
                                    scaling=c["scaling"], bias=c["bias"])
    return fp8_mx_bmm_inputs(c["G"], c["M"], c["N"], c["K"], c["seed"],
                             layout=c["layout"], dist=c["dist"])
