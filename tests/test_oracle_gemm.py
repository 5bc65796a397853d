"""Pins for the oracle's scaled matmuls (CPU).

Each pin is independent of the oracle's own code path:

* brute force: pure-Python loops in exact rational arithmetic on tiny shapes;
* library routines: numpy int64 matmul, PyTorch fp64 dequantise-then-matmul;
* special cases: unit scales give a plain integer GEMM exactly;
* invariants: block-scale homogeneity, rowwise/blockwise and blockwise/mx
  cross-consistency, m-major vs batch-first layout invariance;
* the scale-shape rules printed in the PyTorch blockwise ``_scaled_mm`` issue
  (``tests/golden/blockwise_scale_shapes.txt``).

``test_pins_catch_planted_mistakes`` plants plausible mistakes in copies of the
oracle (on the CPU) and checks that the brute-force pin rejects each one.
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import scaled_mm as S
from oracle.formats import e4m3_value, e8m0_value, bf16_bits_to_f64
from synth import (e4m3_encode, fp8_blockwise_inputs, fp8_mx_bmm_inputs,
                   int8_rowwise_inputs)
from tests.exact import e4m3_exact, rne_bf16, rne_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- int8 ----

def _brute_int8(a, b_kn):
    M, K = a.shape
    N = b_kn.shape[1]
    return [[sum(int(a[m, k]) * int(b_kn[k, n]) for k in range(K))
             for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 0), (3, 5, 7, 1),
                                        (4, 3, 130, 2), (2, 9, 256, 3)])
def test_int8_acc_brute_force(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = rng.integers(-127, 128, (K, N)).astype(np.int8)
    res = S.int8_rowwise(a, b, out_dtype="i32")
    assert res.out.dtype == np.int32
    assert res.exact.tolist() == _brute_int8(a, b)


def test_int8_acc_vs_numpy_int64_and_extremes():
    p = int8_rowwise_inputs(64, 128, 256, 1)
    b_kn = p["b_nk"].T
    res = S.int8_rowwise(p["a"], b_kn, out_dtype="i32")
    ref = p["a"].astype(np.int64) @ b_kn.astype(np.int64)
    assert np.array_equal(res.exact, ref)
    assert np.abs(ref).max() <= 256 * 127 * 127
    # the extreme magnitude K * 127**2 is reached exactly
    a = np.full((2, 4096), -127, np.int8)
    b = np.full((4096, 3), 127, np.int8)
    assert (S.int8_rowwise(a, b, out_dtype="i32").exact == -4096 * 127 * 127).all()
    with pytest.raises(OverflowError):
        S.int8_rowwise(np.full((1, 140000), 127, np.int8),
                       np.full((140000, 1), 127, np.int8), out_dtype="i32")


def test_int8_epilogue_exact_rounding():
    """y = f32(f32(f32(acc) * sa) * sb), every step one IEEE RNE; bf16 of y."""
    p = int8_rowwise_inputs(6, 7, 256, 11)
    a, b_kn, sa, sb = p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"]
    r32 = S.int8_rowwise(a, b_kn, sa, sb, "f32")
    r16 = S.int8_rowwise(a, b_kn, sa, sb, "bf16")
    acc = _brute_int8(a, b_kn)
    for m in range(6):
        for n in range(7):
            y = rne_f32(rne_f32(rne_f32(acc[m][n]) * Fraction(float(sa[m])))
                        * Fraction(float(sb[n])))
            assert Fraction(float(r32.out[m, n])) == y
            assert Fraction(float(bf16_bits_to_f64(r16.out[m, n]))) == rne_bf16(y)


def test_int8_large_acc_rounds_to_nearest_even():
    # acc beyond 2**24 must be rounded (RNE) before scaling
    a = np.zeros((1, 2048), np.int8)
    b = np.zeros((2048, 1), np.int8)
    a[0, :1041] = 127
    b[:1041, 0] = 127
    a[0, 1041], b[1041, 0] = 1, 2      # acc = 1041*16129 + 2 = 16790291
    res = S.int8_rowwise(a, b, np.ones(1, np.float32), np.ones(1, np.float32), "f32")
    acc = 1041 * 16129 + 2
    assert res.exact[0, 0] == acc
    assert Fraction(float(res.out[0, 0])) == rne_f32(acc)


def test_int8_single_scale_form():
    """scale_b == 1 reduces to torchao's single-scale int_scaled_matmul:
    int32 matmul, cast to fp32, times the activation scale."""
    p = int8_rowwise_inputs(16, 32, 384, 5)
    ones = np.ones(32, np.float32)
    res = S.int8_rowwise(p["a"], p["b_nk"].T, p["scale_a"], ones, "f32")
    ref = (torch.from_numpy(p["a"].astype(np.int64)) @ torch.from_numpy(
        p["b_nk"].T.astype(np.int64))).to(torch.float32) * torch.from_numpy(p["scale_a"])[:, None]
    assert np.array_equal(res.out, ref.numpy())


# ------------------------------------------------------------ fp8 blockwise ----

def _brute_blockwise(a, b_kn, sa, sb, cols):
    """Exact C and bound as Fractions for columns ``cols``, straight from the
    definition C[m,n] = sum_k (sa[m,k//128] A[m,k]) (sb[k//128,n//128] B[k,n])."""
    M, K = a.shape
    C, B = [], []
    for m in range(M):
        rowc, rowb = [], []
        for n in cols:
            c = bsum = Fraction(0)
            for k in range(K):
                av = Fraction(float(sa[m, k // 128])) * e4m3_exact(int(a[m, k]))
                bv = Fraction(float(sb[k // 128, n // 128])) * e4m3_exact(int(b_kn[k, n]))
                c += av * bv
                bsum += abs(av) * abs(bv)
            rowc.append(c)
            rowb.append(bsum)
        C.append(rowc)
        B.append(rowb)
    return C, B


def _close(x, frac, scale):
    return abs(Fraction(float(x)) - frac) <= Fraction(1, 2**45) * scale


def _tiny_blockwise(seed, M=3, N=256, K=256):
    p = fp8_blockwise_inputs(M, N, K, seed)
    return p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"]


def test_blockwise_brute_force():
    a, b_kn, sa, sb = _tiny_blockwise(7, M=2, N=256, K=256)
    cols = np.array([0, 5, 127, 128, 200, 255])
    res = S.fp8_blockwise(a, b_kn, sa, sb, "f32", cols=cols)
    C, B = _brute_blockwise(a, b_kn, sa, sb, cols)
    for m in range(2):
        for j in range(len(cols)):
            assert _close(res.exact[m, j], C[m][j], B[m][j])
            assert _close(res.bound[m, j], B[m][j], B[m][j])
            assert Fraction(float(res.out[m, j])) == rne_f32(Fraction(float(res.exact[m, j])))


def test_blockwise_vs_torch_dequant_matmul():
    p = fp8_blockwise_inputs(64, 384, 512, 8)
    a, b_kn, sa, sb = p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"]
    res = S.fp8_blockwise(a, b_kn, sa, sb, "bf16")
    A = torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64)
    Bm = torch.from_numpy(np.ascontiguousarray(b_kn)).view(torch.float8_e4m3fn).to(torch.float64)
    A = A * torch.from_numpy(sa).double().repeat_interleave(128, dim=1)
    Bm = Bm * torch.from_numpy(sb).double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    ref = (A @ Bm).numpy()
    refb = (A.abs() @ Bm.abs()).numpy()
    assert np.allclose(res.exact, ref, rtol=0, atol=1e-13 * refb.max())
    assert np.allclose(res.bound, refb, rtol=1e-13)
    assert (res.bound >= np.abs(res.exact)).all()
    # bf16 output is one rounding of the fp64 value
    tb = torch.from_numpy(res.exact).to(torch.float32).to(torch.bfloat16)
    diff = np.abs(bf16_bits_to_f64(res.out) - tb.double().numpy())
    assert (diff <= np.abs(res.exact) * 2.0**-8).all()


def test_blockwise_unit_scales_give_integer_gemm():
    rng = np.random.default_rng(9)
    M, N, K = 8, 256, 384
    a = rng.integers(0, 256, (M, K)).astype(np.uint8)
    b = rng.integers(0, 256, (K, N)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0
    b[(b & 0x7F) == 0x7F] = 0
    res = S.fp8_blockwise(a, b, np.ones((M, 3), np.float32),
                          np.ones((3, 2), np.float32), "f32")
    nA = (e4m3_value(a) * 512).astype(np.int64)
    nB = (e4m3_value(b) * 512).astype(np.int64)
    assert np.array_equal(res.exact * 2.0**18, (nA @ nB).astype(np.float64))


def test_blockwise_homogeneity():
    """Scaling one block's scale by 2**k changes only that block's
    contribution, by exactly (2**k - 1) times it."""
    a, b_kn, sa, sb = _tiny_blockwise(10, M=4, N=256, K=384)
    base = S.fp8_blockwise(a, b_kn, sa, sb, "f32")
    # row block (m0, kb0)
    m0, kb0 = 2, 1
    sa2 = sa.copy()
    sa2[m0, kb0] *= 8
    r2 = S.fp8_blockwise(a, b_kn, sa2, sb, "f32")
    only = a.copy()
    only[:, :kb0 * 128] = 0
    only[:, (kb0 + 1) * 128:] = 0
    contrib = S.fp8_blockwise(only, b_kn, sa, sb, "f32").exact
    d = r2.exact - base.exact
    tol = 1e-13 * base.bound.max()
    assert np.abs(np.delete(d, m0, axis=0)).max() == 0.0
    assert np.allclose(d[m0], 7 * contrib[m0], rtol=0, atol=tol)
    # weight block (kb0, nb0)
    nb0 = 1
    sb2 = sb.copy()
    sb2[kb0, nb0] *= 0.25
    r3 = S.fp8_blockwise(a, b_kn, sa, sb2, "f32")
    d = r3.exact - base.exact
    assert np.abs(d[:, :128]).max() == 0.0
    onlyb = b_kn.copy()
    onlyb[:kb0 * 128] = 0
    onlyb[(kb0 + 1) * 128:] = 0
    cb = S.fp8_blockwise(a, onlyb, sa, sb, "f32").exact
    assert np.allclose(d[:, 128:], -0.75 * cb[:, 128:], rtol=0, atol=tol)


def test_rowwise_is_blockwise_with_constant_scales():
    """Operands that are small integers are exact in both int8 and E4M3; with
    per-row / per-column-block scales constant along K, the blockwise result
    equals the integer accumulator times the two scales."""
    rng = np.random.default_rng(12)
    M, N, K = 5, 256, 512
    ai = rng.integers(-16, 17, (M, K)).astype(np.int8)
    bi = rng.integers(-16, 17, (K, N)).astype(np.int8)
    a8 = e4m3_encode(ai.astype(np.float64))
    b8 = e4m3_encode(bi.astype(np.float64))
    ra = rng.uniform(0.5, 2, M).astype(np.float32)
    rb = rng.uniform(0.5, 2, 2).astype(np.float32)
    sa = np.repeat(ra[:, None], 4, 1)
    sb = np.repeat(rb[None, :], 4, 0)
    res = S.fp8_blockwise(a8, b8, sa, sb, "f32")
    acc = S.int8_rowwise(ai, bi, out_dtype="i32").exact
    ref = acc * ra[:, None].astype(np.float64) * np.repeat(rb, 128)[None, :].astype(np.float64)
    assert (np.abs(res.exact - ref) <= 1e-14 * res.bound).all()


def test_scale_shape_rules_from_golden():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "blockwise_scale_shapes.txt"))
             if l.strip() and not l.startswith("#")]
    dims = {l[0]: int(l[1]) for l in lines if len(l) == 2}
    M, N, K = dims["M"], dims["N"], dims["K"]
    rules = {l[0]: (eval(l[1]), eval(l[2])) for l in lines if len(l) == 4}
    assert rules["blockwise"] == ((M, K // 128), (K // 128, N // 128))
    assert rules["rowwise"] == ((M, 1), (1, N))
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((K, N), np.uint8)
    sa = np.ones(rules["blockwise"][0], np.float32)
    sb = np.ones(rules["blockwise"][1], np.float32)
    res = S.fp8_blockwise(a, b, sa, sb, "bf16", rows=[0, M - 1], cols=[0, N - 1])
    assert res.exact.shape == (2, 2) and (res.exact == 0).all()
    with pytest.raises(ValueError):
        S.fp8_blockwise(a, b, np.ones(rules["rowwise"][0], np.float32),
                        np.ones(rules["rowwise"][1], np.float32), rows=[0], cols=[0])


# ------------------------------------------------------------------ mx BMM ----

def test_mx_equals_blockwise_with_decoded_scales():
    p = fp8_mx_bmm_inputs(2, 37, 256, 384, 13, layout="batch_first")
    res = S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], "batch_first", "f32")
    for g in range(2):
        sa = e8m0_value(p["x_scale"][g]).astype(np.float32)
        sb = e8m0_value(p["w_scale"][g]).T.astype(np.float32)
        bw = S.fp8_blockwise(p["x"][g], p["w"][g].T, sa, sb, "f32")
        assert np.array_equal(bw.exact, res.exact[g])
        assert np.array_equal(bw.bound, res.bound[g])


def test_mx_brute_force_tiny():
    p = fp8_mx_bmm_inputs(2, 2, 128, 256, 14, layout="m_major")
    cols = [0, 77, 127]
    res = S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], "m_major", "bf16",
                       cols=cols)
    x, w, xs, ws = p["x"], p["w"], p["x_scale"], p["w_scale"]
    for m in range(2):
        for g in range(2):
            for j, n in enumerate(cols):
                c = bsum = Fraction(0)
                for k in range(256):
                    av = Fraction(2) ** (int(xs[m, g, k // 128]) - 127) * e4m3_exact(int(x[m, g, k]))
                    bv = Fraction(2) ** (int(ws[g, n // 128, k // 128]) - 127) * e4m3_exact(int(w[g, n, k]))
                    c += av * bv
                    bsum += abs(av) * abs(bv)
                assert _close(res.exact[m, g, j], c, bsum)
                assert Fraction(float(bf16_bits_to_f64(res.out[m, g, j]))) == rne_bf16(
                    Fraction(float(res.exact[m, g, j])))


def test_mx_layout_invariance():
    p = fp8_mx_bmm_inputs(3, 20, 256, 256, 15, layout="m_major")
    mm = S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], "m_major", "f32")
    xb = np.ascontiguousarray(p["x"].transpose(1, 0, 2))
    xsb = np.ascontiguousarray(p["x_scale"].transpose(1, 0, 2))
    bf = S.fp8_mx_bmm(xb, p["w"], xsb, p["w_scale"], "batch_first", "f32")
    assert np.array_equal(mm.exact.transpose(1, 0, 2), bf.exact)
    assert np.array_equal(mm.out.transpose(1, 0, 2), bf.out)


def test_mx_unit_scales_integer_gemm():
    rng = np.random.default_rng(16)
    G, M, N, K = 2, 4, 128, 256
    x = rng.integers(0, 127, (G, M, K)).astype(np.uint8)
    w = rng.integers(0, 127, (G, N, K)).astype(np.uint8)
    res = S.fp8_mx_bmm(x, w, np.full((G, M, 2), 127, np.uint8),
                       np.full((G, 1, 2), 127, np.uint8), "batch_first", "f32")
    nx = (e4m3_value(x) * 512).astype(np.int64)
    nw = (e4m3_value(w) * 512).astype(np.int64)
    ref = np.einsum("gmk,gnk->gmn", nx, nw)
    assert np.array_equal(res.exact * 2.0**18, ref.astype(np.float64))


# ----------------------------------------------------------- comparison ----

def test_compare_accepts_oracle_and_rejects_planted_error():
    p = fp8_blockwise_inputs(32, 256, 512, 17)
    res = S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], "bf16")
    Y = bf16_bits_to_f64(res.out)
    assert S.compare(Y, res)["ok"]
    bad = Y.copy()
    bad[3, 7] += 2.0**-6 * res.bound[3, 7]
    rep = S.compare(bad, res)
    assert not rep["ok"] and rep["violations"] == 1 and rep["worst"] == (3, 7)
    # exact mode for the int8 path
    q = int8_rowwise_inputs(8, 16, 128, 3)
    r = S.int8_rowwise(q["a"], q["b_nk"].T, q["scale_a"], q["scale_b"], "f32")
    assert S.compare(r.out.copy(), r, exact=True)["ok"]
    off = r.out.copy()
    off[1, 1] = np.nextafter(off[1, 1], np.float32(np.inf))
    assert not S.compare(off, r, exact=True)["ok"]


def test_compare_within_fp32_and_bf16_intervals():
    """The tight rule: a binary32 rounding of the exact value passes with
    gamma = 2**-24 (its error is at most 2**-24 |C| <= 2**-24 Bd); one ulp
    further fails once gamma is below that ulp; the bf16 result must lie in
    [RNE(C - tol), RNE(C + tol)] -- with gamma = 0 exactly RNE(C)."""
    p = fp8_blockwise_inputs(32, 256, 1024, 18)
    r32 = S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], "f32")
    assert S.compare_within(r32.out, r32, 2.0**-24)["ok"]
    # an error of 4 * 2**-24 Bd (after rounding, at least 3 * 2**-24 Bd) fails
    off = r32.out.copy()
    off[5, 9] = np.float32(r32.exact[5, 9] + 4 * 2.0**-24 * r32.bound[5, 9])
    rep = S.compare_within(off, r32, 2.0**-24)
    assert not rep["ok"] and rep["first"] == (5, 9) and rep["violations"] == 1
    rb = S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], "bf16")
    assert S.compare_within(rb.out, rb, 0.0)["ok"]
    # one bf16 ulp away from RNE(C), where C is not within tol of a rounding
    # boundary, is rejected
    bits = rb.out.copy()
    C = rb.exact[2, 3]
    ulp = 2.0 ** (np.floor(np.log2(abs(C))) - 7)
    bits[2, 3] = bits[2, 3] + 1 if (C > 0) == (bf16_bits_to_f64(bits[2, 3]) >= C) else bits[2, 3] - 1
    assert abs(bf16_bits_to_f64(bits[2, 3]) - C) > 0.5 * ulp
    assert not S.compare_within(bits, rb, 2.0**-24)["ok"]
    # the interval rule agrees with exact rounding at its ends: C - tol and
    # C + tol rounded by the exact-rational RNE bracket the accepted values
    tol = 2.0**-12 * rb.bound[2, 3]
    lo, hi = rne_bf16(Fraction(C) - Fraction(tol)), rne_bf16(Fraction(C) + Fraction(tol))
    for v in (lo, hi):
        q = rb.out.copy()
        q[2, 3] = np.float32(float(v)).view(np.uint32) >> 16
        assert S.compare_within(q, rb, 2.0**-12)["ok"]


def test_compare_within_zero_bound_needs_zero_and_catches_one_misscaled_block():
    """Where Bd = 0 only 0 passes.  A K block whose scale is off by a factor
    of two in one row fails the tight rule at the fp32 accumulation bound of
    the kernels in that row and nowhere else."""
    p = fp8_blockwise_inputs(16, 256, 8192, 19)
    a = p["a"].copy()
    a[4, :] = 0                                      # a zero row: Bd = 0 there
    res = S.fp8_blockwise(a, p["b_nk"].T, p["scale_a"], p["scale_b"], "f32")
    assert (res.bound[4] == 0).all()
    y = res.out.copy()
    assert S.compare_within(y, res, 2.0**-20)["ok"]
    y[4, 0] = np.float32(2.0**-140)
    assert not S.compare_within(y, res, 2.0**-20)["ok"]
    sa = p["scale_a"].copy()
    sa[7, 40] *= 2
    wrong = S.fp8_blockwise(a, p["b_nk"].T, sa, p["scale_b"], "f32")
    gamma = 2.0**-17 + 72 * 2.0**-24
    rep = S.compare_within(wrong.out, res, gamma)
    assert not rep["ok"] and {f[0] for f in np.argwhere(wrong.out != res.out)} == {7}


def _brute_check(fn):
    """Run the brute-force blockwise pin against oracle function ``fn``."""
    a, b_kn, sa, sb = _tiny_blockwise(21, M=2, N=256, K=256)
    cols = np.array([1, 130, 250])
    res = fn(a, b_kn, sa, sb, "f32", cols=cols)
    C, B = _brute_blockwise(a, b_kn, sa, sb, cols)
    return all(_close(res.exact[m, j], C[m][j], B[m][j])
               for m in range(2) for j in range(len(cols)))


def test_pins_catch_planted_mistakes(monkeypatch):
    assert _brute_check(S.fp8_blockwise)
    # 1. dropped last K block
    monkeypatch.setattr(S, "_blocks", lambda K, block=128: [(k0, min(K, k0 + block))
                                                             for k0 in range(0, K - block, block)])
    assert not _brute_check(S.fp8_blockwise)
    monkeypatch.undo()
    # 2. sign of the decoded code dropped
    from oracle import formats as F
    real = F.e4m3_numerator
    monkeypatch.setattr(S, "e4m3_numerator", lambda c: (np.abs(real(c)[0]), real(c)[1]))
    assert not _brute_check(S.fp8_blockwise)
    monkeypatch.undo()
    # 3. weight scale indexed transposed (sb[n//128, kb] instead of sb[kb, n//128])
    def transposed(a, b_kn, sa, sb, out, cols=None):
        return S.fp8_blockwise(a, b_kn, sa, np.ascontiguousarray(sb.T), out, cols=cols)
    assert not _brute_check(transposed)
    # 4. wrong exponent bias in the decode (2**-8 instead of 2**-9 per operand)
    monkeypatch.setattr(S, "TWO_M18", 2.0**-16)
    assert not _brute_check(S.fp8_blockwise)
