"""Pins for the dynamic-quantisation oracle (CPU).

The e4m3 encoder is checked against PyTorch's own CPU float8_e4m3fn
conversion (an independent library routine that rounds to nearest, ties to
even) over every midpoint between adjacent codes and across all binades, and
against an exact brute-force search over all finite codes.  The three
quantisers are checked against hand-worked rows, against exact rational
brute force on small inputs (the scale, the binary32 quotient and the
nearest code all found with ``fractions``), and against invariants that any
correct implementation meets: the amax element lands on the top code, the
dequantised value is within half a code step of the input, and the e8m0
exponent is the smallest one that keeps amax within 448.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as Q
from tests.exact import e4m3_exact, rne_f32

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]
EXACT = {c: e4m3_exact(c) for c in FINITE}


def torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def brute_e4m3(t: Fraction, negative: bool) -> int:
    """Nearest finite code to t by exhaustive search, ties to the even code,
    saturating; the sign bit follows ``negative`` for a zero result."""
    best = None
    for c in FINITE:
        d = abs(EXACT[c] - t)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    c = best[1]
    if EXACT[c] == 0:
        c = 0x80 if negative else 0x00
    return c


def brute_int8(t: Fraction) -> int:
    best = None
    for q in range(-127, 128):
        d = abs(q - t)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


# ---------------------------------------------------------------------------
# e4m3 encoder
# ---------------------------------------------------------------------------

def test_e4m3_encode_hand_values():
    v = np.array([0.0, -0.0, 1.0, -1.0, 1.0625, 1.125, 1.1875, 448.0, 449.0, 464.0,
                  480.0, 1e9, -1e9, 2.0**-9, 2.0**-10, 3 * 2.0**-10, 2.0**-11, -(2.0**-11)])
    want = [0x00, 0x80, 0x38, 0xB8, 0x38, 0x39, 0x3A, 0x7E, 0x7E, 0x7E,
            0x7E, 0x7E, 0xFE, 0x01, 0x00, 0x02, 0x00, 0x80]
    # 1.0625 is the midpoint of 1 (mantissa 0, even) and 1.125: goes to 1;
    # 1.1875 is the midpoint of 1.125 (odd) and 1.25: goes to 1.25 = 0x3A;
    # 2**-10 is half the smallest subnormal: ties to 0; 3*2**-10 ties to 2*2**-9
    assert list(Q.e4m3_encode_rne(v)) == want


def test_e4m3_encode_matches_torch_at_every_midpoint_and_code():
    pos = np.array([float(EXACT[c]) for c in range(0x7F)])
    mids = (pos[:-1] + pos[1:]) / 2               # exact in fp32
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    v = np.concatenate([pos, mids, near]).astype(np.float32)
    v = np.concatenate([v, -v])
    assert np.array_equal(Q.e4m3_encode_rne(v), torch_e4m3(v))


def test_e4m3_encode_matches_torch_random_binades():
    rng = np.random.default_rng(3)
    v = (rng.uniform(-1, 1, 50000) * np.exp2(rng.uniform(-14, 8.8, 50000))).astype(np.float32)
    v = v[np.abs(v) <= 448]
    assert np.array_equal(Q.e4m3_encode_rne(v), torch_e4m3(v))


def test_e4m3_encode_brute_force_and_round_trip():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(300) * np.exp2(rng.uniform(-12, 10, 300))).astype(np.float32)
    got = Q.e4m3_encode_rne(v)
    for vi, gi in zip(v, got):
        assert gi == brute_e4m3(Fraction(float(vi)), bool(np.signbit(vi)))
    codes = np.array(FINITE, dtype=np.uint8)
    assert np.array_equal(Q.e4m3_encode_rne(F.e4m3_value(codes)), codes)


def test_e4m3_encode_rejects_nan():
    with pytest.raises(ValueError):
        Q.e4m3_encode_rne(np.array([1.0, np.nan]))


# ---------------------------------------------------------------------------
# int8 per row
# ---------------------------------------------------------------------------

def test_int8_rowwise_hand_row():
    x = np.zeros((3, 8), np.float32)
    x[0, :6] = [127, 63.5, -1, 0.5, 1.5, -2.5]     # scale 1: ties go to even
    x[1, :3] = [-254, 127, 1]                      # scale 2, amax negative
    q, s = Q.quant_int8_rowwise(x)
    assert s.tolist() == [1.0, 2.0, 1.0]           # an all-zero row gets scale 1
    assert q[0, :6].tolist() == [127, 64, -1, 0, 2, -2]
    assert q[1, :3].tolist() == [-127, 64, 0]      # 63.5 -> 64, 0.5 -> 0
    assert not q[2].any()


def test_int8_rowwise_brute_force():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((6, 40)) * np.exp2(rng.uniform(-20, 20, (6, 1)))).astype(np.float32)
    x[2, 7] = 0.0
    q, s = Q.quant_int8_rowwise(x)
    for r in range(x.shape[0]):
        amax = max(abs(Fraction(float(v))) for v in x[r])
        scale = rne_f32(amax / 127)
        assert Fraction(float(s[r])) == scale
        for c in range(x.shape[1]):
            t = rne_f32(Fraction(float(x[r, c])) / scale)
            assert q[r, c] == brute_int8(t)


def test_int8_rowwise_invariants():
    rng = np.random.default_rng(6)
    x = (rng.standard_t(3, (64, 512)) * np.exp2(rng.uniform(-30, 30, (64, 1)))).astype(np.float32)
    q, s = Q.quant_int8_rowwise(x)
    arg = np.abs(x).argmax(axis=1)
    rows = np.arange(x.shape[0])
    assert np.array_equal(np.abs(q[rows, arg]), np.full(x.shape[0], 127))
    assert np.array_equal(np.sign(q[rows, arg]), np.sign(x[rows, arg]))
    err = np.abs(q.astype(np.float64) * s[:, None] - x)
    assert np.all(err <= s[:, None] * (0.5 + 1e-6))
    # the scale is a per-row quantity: permuting rows permutes it
    p = rng.permutation(x.shape[0])
    q2, s2 = Q.quant_int8_rowwise(x[p])
    assert np.array_equal(q2, q[p]) and np.array_equal(s2, s[p])


def test_int8_rowwise_scale_underflow_reads_as_zero_row():
    x = np.zeros((2, 4), np.float32)
    x[0, 1] = np.float32(2.0**-149)                # amax / 127 rounds to 0 in fp32
    x[1, 1] = np.float32(2.0**-120)
    q, s = Q.quant_int8_rowwise(x)
    assert s[0] == 1.0 and not q[0].any()
    assert s[1] == np.float32(np.float64(2.0**-120) / 127) and q[1, 1] == 127


# ---------------------------------------------------------------------------
# fp8, 1 x 128 blocks, fp32 scale
# ---------------------------------------------------------------------------

def test_fp8_blockwise_hand_blocks():
    x = np.zeros((2, 256), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 448.0, -1.0625, 1.1875       # block (0,0): scale 1
    x[0, 128], x[0, 129] = -896.0, 3.0                       # block (0,1): scale 2
    x[1, 5] = 0.5                                            # block (1,0): 0.5/448
    x[1, 130] = -0.0                                         # block (1,1): all zero
    codes, s = Q.quant_fp8_blockwise(x)
    assert s.tolist() == [[1.0, 2.0], [np.float32(0.5 / 448), 1.0]]
    assert codes[0, :3].tolist() == [0x7E, 0xB8, 0x3A]
    assert codes[0, 128:130].tolist() == [0xFE, 0x3C]        # 3/2 = 1.5
    assert codes[1, 5] == 0x7E and not codes[1, 128:].any()
    assert codes[0, 3] == 0x00                               # +0 stays +0


def test_fp8_blockwise_brute_force():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((2, 256)) * np.exp2(rng.uniform(-10, 10, (2, 256)))).astype(np.float32)
    x[1, 200] = -0.0
    codes, s = Q.quant_fp8_blockwise(x)
    for r in range(2):
        for b in range(2):
            blk = x[r, b * 128:(b + 1) * 128]
            amax = max(abs(Fraction(float(v))) for v in blk)
            scale = rne_f32(amax / 448)
            assert Fraction(float(s[r, b])) == scale
            for c in range(0, 128, 3):
                t = rne_f32(Fraction(float(blk[c])) / scale)
                assert codes[r, b * 128 + c] == brute_e4m3(t, bool(np.signbit(blk[c])))
    assert codes[1, 200] == 0x80


def test_fp8_blockwise_invariants():
    rng = np.random.default_rng(8)
    x = (rng.standard_t(3, (32, 1024)) * np.exp2(rng.uniform(-20, 20, (32, 8)).repeat(128, 1))) \
        .astype(np.float32)
    codes, s = Q.quant_fp8_blockwise(x)
    xb = x.reshape(32, 8, 128)
    cb = codes.reshape(32, 8, 128)
    arg = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(cb, arg[:, :, None], 2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    dq = F.e4m3_value(cb) * s[:, :, None]
    # half a code step: 2**-4 relative in the normal range, 2**-10 absolute below it
    bound = np.maximum(np.abs(xb) * 2.0**-4, 2.0**-10 * s[:, :, None]) * (1 + 1e-6)
    assert np.all(np.abs(dq - xb) <= bound)


def test_fp8_blockwise_rejects_ragged_k():
    with pytest.raises(ValueError):
        Q.quant_fp8_blockwise(np.ones((2, 130), np.float32))


# ---------------------------------------------------------------------------
# fp8, 1 x 128 blocks, e8m0 scale
# ---------------------------------------------------------------------------

def test_e8m0_exponent_exact_powers_and_neighbours():
    for k in range(-100, 100, 7):
        a = np.float32(448.0 * 2.0**k)
        up = np.nextafter(a, np.float32(np.inf))
        dn = np.nextafter(a, np.float32(0))
        assert Q.e8m0_exponent(np.array([a, up, dn])).tolist() == [k, k + 1, k]
    assert Q.e8m0_exponent(np.array([0.0, 1.0, 2.0**-149])).tolist() == [0, -8, -127]


def test_e8m0_exponent_brute_force():
    rng = np.random.default_rng(9)
    a = np.abs(rng.standard_normal(2000) * np.exp2(rng.uniform(-100, 100, 2000))).astype(np.float32)
    got = Q.e8m0_exponent(a)
    for ai, gi in zip(a, got):
        fa = Fraction(float(ai))
        assert fa <= 448 * Fraction(2) ** int(gi)
        assert fa > 448 * Fraction(2) ** (int(gi) - 1)


def test_fp8_mx_hand_and_invariants():
    x = np.zeros((1, 256), np.float32)
    x[0, 0], x[0, 1] = 100.0, -0.3                 # amax 100: e = -2 (scale 1/4)
    x[0, 128] = 448.0 * 2.0**5                     # exact power: e = 5
    codes, e = Q.quant_fp8_mx(x)
    assert e.tolist() == [[125, 132]]
    assert codes[0, 0] == Q.e4m3_encode_rne(np.array([400.0]))[0]
    assert codes[0, 1] == Q.e4m3_encode_rne(np.array([-1.2]))[0]
    assert codes[0, 128] == 0x7E

    rng = np.random.default_rng(10)
    x = (rng.standard_normal((16, 512)) * np.exp2(rng.uniform(-60, 60, (16, 4)).repeat(128, 1))) \
        .astype(np.float32)
    codes, e = Q.quant_fp8_mx(x)
    ex = e.astype(np.int64) - 127
    xb = x.reshape(16, 4, 128).astype(np.float64)
    amax = np.abs(xb).max(axis=2)
    r = amax * np.exp2(-ex.astype(np.float64))
    assert np.all((r > 224) & (r <= 448))          # smallest exponent that fits
    # a power-of-two scaling: the codes are the plain e4m3 rounding of the
    # scaled values, which PyTorch's cast computes too (|x 2**-e| <= 448)
    scaled = np.ldexp(xb, -ex[:, :, None]).astype(np.float32)
    assert np.array_equal(codes.reshape(16, 4, 128), torch_e4m3(scaled))


def test_fp8_mx_bottom_clamp_and_zero_block():
    x = np.zeros((1, 256), np.float32)
    x[0, 3] = np.float32(2.0**-140)                # exponent would be -148: clamped
    codes, e = Q.quant_fp8_mx(x)
    assert e.tolist() == [[0, 127]]
    assert codes[0, 3] == Q.e4m3_encode_rne(np.array([2.0**-13]))[0] == 0x00
    x[0, 3] = np.float32(2.0**-130)                # 2**-130 * 2**127 = 2**-3
    codes, e = Q.quant_fp8_mx(x)
    assert e[0, 0] == 0 and codes[0, 3] == 0x20      # exponent field 4
    assert not codes[0, 128:].any()
    x[0, 130] = -0.0                               # an all-zero block: +0 codes
    assert not Q.quant_fp8_mx(x)[0][0, 128:].any()
    x[0, 5] = -0.0                                 # in a live block -0 keeps its sign
    assert Q.quant_fp8_mx(x)[0][0, 5] == 0x80


def test_fp8_mx_32_element_blocks():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 256)) * np.exp2(rng.uniform(-30, 30, (6, 8)).repeat(32, 1))) \
        .astype(np.float32)
    codes, e = Q.quant_fp8_mx(x, block=32)
    assert e.shape == (6, 8)
    ex = e.astype(np.int64) - 127
    xb = x.reshape(6, 8, 32).astype(np.float64)
    r = np.abs(xb).max(axis=2) * np.exp2(-ex.astype(np.float64))
    assert np.all((r > 224) & (r <= 448))          # the smallest fitting exponent, per 32
    scaled = np.ldexp(xb, -ex[:, :, None]).astype(np.float32)
    assert np.array_equal(codes.reshape(6, 8, 32), torch_e4m3(scaled))
    # four 32-blocks of equal exponent give the 128-block result
    y = np.tile(np.linspace(-300, 400, 32, dtype=np.float32), (2, 4))
    c32, e32 = Q.quant_fp8_mx(y, block=32)
    c128, e128 = Q.quant_fp8_mx(y)
    assert np.array_equal(c32, c128) and (e32 == e128[:, :1]).all()
    with pytest.raises(ValueError):
        Q.quant_fp8_mx(np.ones((2, 48), np.float32), block=32)


# ---------------------------------------------------------------------------
# fp8, 128 x 128 weight blocks, fp32 scale
# ---------------------------------------------------------------------------

def test_weight_blocks_hand_values():
    w = np.zeros((256, 256), np.float32)
    w[3, 100], w[77, 5] = -896.0, 3.0          # block (0,0): scale 2
    w[200, 10] = 0.5                           # block (1,0): 0.5 / 448
    w[130, 250] = 448.0                        # block (1,1): scale 1
    codes, s = Q.quant_fp8_weight_blocks(w)
    assert s.tolist() == [[2.0, 1.0], [np.float32(0.5 / 448), 1.0]]
    assert codes[3, 100] == 0xFE and codes[77, 5] == 0x3C     # 3/2 = 1.5
    assert codes[200, 10] == 0x7E and codes[130, 250] == 0x7E
    assert not codes[:128, 128:].any()                       # block (0,1) all zero


def test_weight_blocks_brute_force():
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((256, 384)) * np.exp2(rng.uniform(-8, 8, (256, 384)))) \
        .astype(np.float32)
    w[5, 300] = -0.0
    codes, s = Q.quant_fp8_weight_blocks(w)
    for bi in range(2):
        for bj in range(3):
            blk = w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            amax = max(abs(Fraction(float(v))) for v in blk.ravel())
            scale = rne_f32(amax / 448)
            assert Fraction(float(s[bi, bj])) == scale
            for r in range(0, 128, 29):
                for c in range(0, 128, 31):
                    t = rne_f32(Fraction(float(blk[r, c])) / scale)
                    assert codes[bi * 128 + r, bj * 128 + c] == \
                        brute_e4m3(t, bool(np.signbit(blk[r, c])))
    assert codes[5, 300] == 0x80


def test_weight_blocks_invariants():
    rng = np.random.default_rng(22)
    w = (rng.standard_t(3, (384, 512)) * np.exp2(rng.uniform(-20, 20, (3, 1, 4, 1)))
         .repeat(128, 1).repeat(128, 3).reshape(384, 512)).astype(np.float32)
    codes, s = Q.quant_fp8_weight_blocks(w)
    wb = w.reshape(3, 128, 4, 128).transpose(0, 2, 1, 3).reshape(3, 4, -1)
    cb = codes.reshape(3, 128, 4, 128).transpose(0, 2, 1, 3).reshape(3, 4, -1)
    arg = np.abs(wb).argmax(axis=2)
    top = np.take_along_axis(cb, arg[:, :, None], 2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    dq = F.e4m3_value(cb) * s[:, :, None]
    bound = np.maximum(np.abs(wb) * 2.0**-4, 2.0**-10 * s[:, :, None]) * (1 + 1e-6)
    assert np.all(np.abs(dq - wb) <= bound)


def test_weight_blocks_reject_ragged_shapes():
    with pytest.raises(ValueError):
        Q.quant_fp8_weight_blocks(np.ones((128, 200), np.float32))


# ---------------------------------------------------------------------------
# fp8, 1 x 128 groups down the columns, transposed codes
# ---------------------------------------------------------------------------

def test_columns_hand_values():
    x = np.zeros((256, 3), np.float32)
    x[0, 0], x[127, 0], x[128, 0] = 448.0, -1.0625, 0.25      # column 0, groups 0 and 1
    x[40, 2] = -896.0                                        # column 2, group 0: scale 2
    codes_t, s = Q.quant_fp8_columns(x)
    assert codes_t.shape == (3, 256) and s.shape == (2, 3)
    assert s.tolist() == [[1.0, 1.0, 2.0], [np.float32(0.25 / 448), 1.0, 1.0]]
    assert codes_t[0, 0] == 0x7E and codes_t[0, 127] == 0xB8 and codes_t[0, 128] == 0x7E
    assert codes_t[2, 40] == 0xFE and not codes_t[1].any()


def test_columns_brute_force():
    rng = np.random.default_rng(23)
    x = (rng.standard_normal((384, 40)) * np.exp2(rng.uniform(-10, 10, (384, 40)))) \
        .astype(np.float32)
    codes_t, s = Q.quant_fp8_columns(x)
    for c in (0, 13, 39):
        for g in range(3):
            col = x[g * 128:(g + 1) * 128, c]
            amax = max(abs(Fraction(float(v))) for v in col)
            scale = rne_f32(amax / 448)
            assert Fraction(float(s[g, c])) == scale
            for r in range(0, 128, 7):
                t = rne_f32(Fraction(float(col[r])) / scale)
                assert codes_t[c, g * 128 + r] == brute_e4m3(t, bool(np.signbit(col[r])))


def test_columns_invariants():
    rng = np.random.default_rng(24)
    x = (rng.standard_t(3, (512, 96)) * np.exp2(rng.uniform(-20, 20, (4, 1, 96)))
         .repeat(128, 1).reshape(512, 96)).astype(np.float32)
    codes_t, s = Q.quant_fp8_columns(x)
    xg = x.T.reshape(96, 4, 128)
    cg = codes_t.reshape(96, 4, 128)
    arg = np.abs(xg).argmax(axis=2)
    top = np.take_along_axis(cg, arg[:, :, None], 2)[:, :, 0]
    assert np.all((top & 0x7F) == 0x7E)
    dq = F.e4m3_value(cg) * s.T[:, :, None]
    bound = np.maximum(np.abs(xg) * 2.0**-4, 2.0**-10 * s.T[:, :, None]) * (1 + 1e-6)
    assert np.all(np.abs(dq - xg) <= bound)
