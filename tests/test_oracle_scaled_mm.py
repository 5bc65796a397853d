"""Pins for the oracle's fp8 ``_scaled_mm`` with tensorwise / rowwise scales,
bias and scale_result (CPU).

* brute force in exact rationals on tiny shapes (every term of the
  definition: products, both scales, bias, scale_result);
* PyTorch's fp64 dequantise-then-matmul (its own float8 decode and BLAS);
* special cases: unit scales give the integer GEMM of the E4M3 numerators;
  tensorwise equals rowwise with constant scales;
* invariants: a power-of-two row or column scale scales exactly that row or
  column; a bias shifts each column exactly;
* output formats: hand-worked E4M3 results (round to nearest even, ties,
  saturation) and the comparison rule for E4M3 outputs;
* the tensorwise and rowwise shape rules of the PyTorch blockwise issue
  (``tests/golden/blockwise_scale_shapes.txt``).
"""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import scaled_mm as S
from oracle.formats import bf16_bits_to_f64, e4m3_numerator, e4m3_value, round_f32
from synth import fp8_scaled_mm_inputs
from tests.exact import e4m3_exact, rne_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute(a, b_kn, sa, sb, bias, sr, rows, cols):
    """Exact values, and the magnitude (|acc s| + |bias|) |sr| that bounds the
    oracle's fp64 rounding (one product, one sum)."""
    K = a.shape[1]
    out, mag = [], []
    for m in rows:
        row, mrow = [], []
        for n in cols:
            acc = sum(e4m3_exact(int(a[m, k])) * e4m3_exact(int(b_kn[k, n])) for k in range(K))
            v = acc * (Fraction(float(sa[m])) * Fraction(float(sb[n])))
            g = abs(v)
            if bias is not None:
                v += Fraction(float(bias[n]))
                g += abs(Fraction(float(bias[n])))
            if sr is not None:
                v *= Fraction(float(np.float32(sr)))
                g *= abs(Fraction(float(np.float32(sr))))
            row.append(v)
            mrow.append(g)
        out.append(row)
        mag.append(mrow)
    return out, mag


def _close(x, w, g):
    return abs(Fraction(float(x)) - w) <= g * Fraction(1, 2**50) + Fraction(1, 2**80)


def _vectors(p, M, N):
    sa = np.broadcast_to(np.asarray(p["scale_a"], np.float32).reshape(-1), (M,)) \
        if np.asarray(p["scale_a"]).size == 1 else p["scale_a"][:, 0]
    sb = np.broadcast_to(np.asarray(p["scale_b"], np.float32).reshape(-1), (N,)) \
        if np.asarray(p["scale_b"]).size == 1 else p["scale_b"][0, :]
    return sa, sb


@pytest.mark.parametrize("scaling,bias,sr", [("rowwise", None, None), ("rowwise", "f32", 0.375),
                                             ("tensorwise", "bf16", None),
                                             ("tensorwise", None, 3.0)])
def test_brute_force_exact_rationals(scaling, bias, sr):
    M, N, K = 3, 5, 40
    p = fp8_scaled_mm_inputs(M, N, K, 7, scaling=scaling, bias=bias)
    b_kn = p["b_nk"].T
    res = S.fp8_scaled_mm(p["a"], b_kn, p["scale_a"], p["scale_b"], bias=p["bias"],
                          scale_result=sr, out_dtype="f32")
    sa, sb = _vectors(p, M, N)
    want, mag = _brute(p["a"], b_kn, sa, sb, p["bias"], sr, range(M), range(N))
    for m in range(M):
        for n in range(N):
            w = want[m][n]
            assert _close(res.exact[m, n], w, mag[m][n])
            # the fp32 output is the exact value rounded once (the fp64 error
            # is far below half an fp32 ulp of these values)
            assert Fraction(float(res.out[m, n])) == rne_f32(w)


def test_vs_torch_dequant_matmul():
    M, N, K = 40, 256, 384
    p = fp8_scaled_mm_inputs(M, N, K, 3, bias="f32")
    b_kn = p["b_nk"].T
    res = S.fp8_scaled_mm(p["a"], b_kn, p["scale_a"], p["scale_b"], bias=p["bias"],
                          scale_result=0.5, out_dtype="bf16")
    A = torch.from_numpy(p["a"].copy()).view(torch.float8_e4m3fn).to(torch.float64)
    B = torch.from_numpy(np.ascontiguousarray(b_kn)).view(torch.float8_e4m3fn).to(torch.float64)
    sa = torch.from_numpy(p["scale_a"]).to(torch.float64)
    sb = torch.from_numpy(p["scale_b"]).to(torch.float64)
    ref = ((A @ B) * (sa * sb) + torch.from_numpy(p["bias"]).to(torch.float64)) * 0.5
    assert np.allclose(res.exact, ref.numpy(), rtol=1e-12, atol=1e-12)
    # the bf16 output is the exact value rounded once
    got = bf16_bits_to_f64(res.out)
    assert np.allclose(got, ref.numpy(), rtol=2.0**-8, atol=0)


def test_unit_scales_give_integer_gemm_and_tensorwise_is_constant_rowwise():
    M, N, K = 6, 128, 256
    rng = np.random.default_rng(2)
    a = rng.integers(0, 0x7F, (M, K), dtype=np.uint8)
    b = rng.integers(0, 0x7F, (K, N), dtype=np.uint8)
    one = np.float32(1.0)
    res = S.fp8_scaled_mm(a, b, one, one, out_dtype="f32")
    nA, _ = e4m3_numerator(a)
    nB, _ = e4m3_numerator(b)
    P = nA.astype(object) @ nB.astype(object)
    assert all(Fraction(float(res.exact[m, n])) == Fraction(int(P[m, n]), 2**18)
               for m in range(M) for n in range(N))
    c_a, c_b = np.float32(0.3), np.float32(-1.7)
    t = S.fp8_scaled_mm(a, b, c_a, c_b, out_dtype="f32")
    r = S.fp8_scaled_mm(a, b, np.full((M, 1), c_a), np.full((1, N), c_b), out_dtype="f32")
    assert np.array_equal(t.exact, r.exact) and np.array_equal(t.out, r.out)


def test_row_and_column_homogeneity_and_bias_shift():
    M, N, K = 9, 256, 256
    p = fp8_scaled_mm_inputs(M, N, K, 5)
    b_kn = p["b_nk"].T
    base = S.fp8_scaled_mm(p["a"], b_kn, p["scale_a"], p["scale_b"], out_dtype="f32").exact
    sa = p["scale_a"].copy()
    sa[4, 0] *= 8
    sb = p["scale_b"].copy()
    sb[0, 100] *= 0.25
    got = S.fp8_scaled_mm(p["a"], b_kn, sa, sb, out_dtype="f32").exact
    want = base.copy()
    want[4, :] *= 8
    want[:, 100] *= 0.25
    assert np.array_equal(got, want)
    bias = np.linspace(-3, 3, N).astype(np.float32)
    shifted = S.fp8_scaled_mm(p["a"], b_kn, p["scale_a"], p["scale_b"], bias=bias,
                              out_dtype="f32").exact
    # shifted by the bias, up to the one fp64 rounding of the sum
    diff = shifted - base - bias.astype(np.float64)[None, :]
    assert np.all(np.abs(diff) <= 2.0**-50 * (np.abs(base) + np.abs(bias)[None, :]))


def test_e4m3_output_hand_values():
    a = np.full((1, 128), 0x38, np.uint8)             # 1.0
    b = np.full((128, 1), 0x38, np.uint8)
    one = np.float32(1)
    cases = [(2.0, None, 0x70),     # 130 -> 128 (nearest)
             (8.0, None, 0x70),     # 136: halfway 128 / 144, the even mantissa (128)
             (9.0, None, 0x71),     # 137 -> 144
             (2.0, 2.0, 0x78),      # 260 -> 256
             (2.0, 1e4, 0x7E),      # saturates at 448
             (2.0, -1e4, 0xFE)]
    for bias, sr, code in cases:
        r = S.fp8_scaled_mm(a, b, one, one, bias=np.array([bias], np.float32),
                            scale_result=sr, out_dtype="e4m3")
        assert r.out[0, 0] == code, (bias, sr, hex(r.out[0, 0]))


def test_compare_e4m3_rule():
    p = fp8_scaled_mm_inputs(16, 128, 256, 9, bias="f32")
    res = S.fp8_scaled_mm(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], bias=p["bias"],
                          out_dtype="e4m3")
    assert S.compare_e4m3(res.out, res, 2.0**-20)["ok"]
    bad = res.out.copy()
    # two code steps away (same sign, away from zero) is never within the rule
    i = np.argwhere((bad & 0x7F) < 0x70)[0]
    bad[tuple(i)] += 2
    rep = S.compare_e4m3(bad, res, 2.0**-20)
    assert not rep["ok"] and rep["violations"] == 1
    # an exactly representable result: any other code is rejected, even an
    # equally near neighbour of a tie
    a = np.full((1, 128), 0x38, np.uint8)
    b = np.full((128, 1), 0x38, np.uint8)
    r = S.fp8_scaled_mm(a, b, np.float32(1), np.float32(1), bias=np.array([8.0], np.float32),
                        out_dtype="e4m3")
    assert S.compare_e4m3(np.array([[0x70]], np.uint8), r, 0.0)["ok"]
    assert not S.compare_e4m3(np.array([[0x71]], np.uint8), r, 0.0)["ok"]


def test_scale_shape_rules_from_golden():
    lines = [l.split() for l in open(os.path.join(GOLDEN, "blockwise_scale_shapes.txt"))
             if l.strip() and not l.startswith("#")]
    dims = {l[0]: int(l[1]) for l in lines if len(l) == 2}
    M, N, K = dims["M"], dims["N"], dims["K"]
    rules = {l[0]: (eval(l[1]), eval(l[2])) for l in lines if len(l) == 4}
    a = np.zeros((M, K), np.uint8)
    b = np.zeros((K, N), np.uint8)
    for kind in ("rowwise", "tensorwise"):
        sa = np.ones(rules[kind][0], np.float32)
        sb = np.ones(rules[kind][1], np.float32)
        r = S.fp8_scaled_mm(a, b, sa, sb, rows=[0, M - 1], cols=[0, N - 1], out_dtype="f32")
        assert (r.exact == 0).all()
    with pytest.raises(ValueError):
        S.fp8_scaled_mm(a, b, np.ones(rules["blockwise"][0], np.float32),
                        np.ones(rules["blockwise"][1], np.float32), rows=[0], cols=[0])


def test_planted_mistakes_are_caught(monkeypatch):
    M, N, K = 2, 3, 24
    p = fp8_scaled_mm_inputs(M, N, K, 11, bias="f32")
    b_kn = p["b_nk"].T
    sa, sb = _vectors(p, M, N)
    want, mag = _brute(p["a"], b_kn, sa, sb, p["bias"], 0.75, range(M), range(N))

    def ok(res):
        return all(_close(res.exact[m, n], want[m][n], mag[m][n])
                   for m in range(M) for n in range(N))

    call = lambda: S.fp8_scaled_mm(p["a"], b_kn, p["scale_a"], p["scale_b"], bias=p["bias"],
                                   scale_result=0.75, out_dtype="f32")
    assert ok(call())
    plain = S.fp8_scaled_mm(p["a"], b_kn, p["scale_a"], p["scale_b"], out_dtype="f32").exact
    s = sa[:, None].astype(np.float64) * sb[None, :]
    # the bias scaled by the operand scales (added before the scaling)
    assert not ok(S.Result(exact=(plain + p["bias"][None, :] * s) * 0.75, out=None))
    # scale_result ignored
    assert not ok(S.fp8_scaled_mm(p["a"], b_kn, p["scale_a"], p["scale_b"], bias=p["bias"],
                                  out_dtype="f32"))
    # column scale indexed by row
    assert not ok(S.Result(exact=(plain / sb[None, :] * sb[:M, None] + p["bias"][None, :])
                           * 0.75, out=None))
    # wrong exponent bias in the decode
    monkeypatch.setattr(S, "TWO_M18", 2.0**-16)
    assert not ok(call())


# ------------------------------------------------------------- MX, 32 blocks --

def _mx32_random(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K)).astype(np.uint8) & 0xF7          # no NaN codes
    b = rng.integers(0, 256, (K, N)).astype(np.uint8) & 0xF7
    sa = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    return a, b, sa, sb


def test_mx32_brute_force_exact_rationals():
    M, N, K = 3, 4, 96
    a, b, sa, sb = _mx32_random(M, N, K, 1)
    res = S.fp8_mx32_mm(a, b, sa, sb, "f32")
    for m in range(M):
        for n in range(N):
            w = sum(e4m3_exact(int(a[m, k])) * e4m3_exact(int(b[k, n]))
                    * Fraction(2) ** (int(sa[m, k // 32]) - 127)
                    * Fraction(2) ** (int(sb[n, k // 32]) - 127) for k in range(K))
            g = sum(abs(e4m3_exact(int(a[m, k])) * e4m3_exact(int(b[k, n])))
                    * Fraction(2) ** (int(sa[m, k // 32]) + int(sb[n, k // 32]) - 254)
                    for k in range(K))
            assert _close(res.exact[m, n], w, g)
            assert Fraction(float(res.out[m, n])) == rne_f32(w)


def test_mx32_vs_torch_dequant_matmul():
    M, N, K = 24, 64, 256
    a, b, sa, sb = _mx32_random(M, N, K, 2)
    res = S.fp8_mx32_mm(a, b, sa, sb, "f32")
    A = torch.from_numpy(a.copy()).view(torch.float8_e4m3fn).to(torch.float64)
    B = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64)
    A = A * torch.from_numpy(np.exp2(sa.astype(np.float64) - 127)).repeat_interleave(32, 1)
    B = B * torch.from_numpy(np.exp2(sb.astype(np.float64) - 127)).T.repeat_interleave(32, 0)
    ref = (A @ B).numpy()
    assert np.allclose(res.exact, ref, rtol=1e-12, atol=1e-300)


def test_mx32_equals_mx128_when_scales_are_constant_per_128_block():
    G, M, N, K = 1, 7, 256, 384
    rng = np.random.default_rng(3)
    a, b, _, _ = _mx32_random(M, N, K, 3)
    xs = rng.integers(115, 135, (M, K // 128)).astype(np.uint8)
    ws = rng.integers(115, 135, (N // 128, K // 128)).astype(np.uint8)
    sa = np.repeat(xs, 4, axis=1)                       # each 128-block's 4 chunks alike
    sb = np.repeat(np.repeat(ws, 128, axis=0), 4, axis=1)
    r32 = S.fp8_mx32_mm(a, b, sa, sb, "f32")
    r128 = S.fp8_mx_bmm(a[None], np.ascontiguousarray(b.T)[None], xs[None], ws[None],
                        layout="batch_first", out_dtype="f32")
    assert np.allclose(r32.exact, r128.exact[0], rtol=1e-13, atol=0)


def test_mx32_unit_scales_and_chunk_homogeneity():
    M, N, K = 4, 32, 128
    a, b, _, _ = _mx32_random(M, N, K, 4)
    one_a = np.full((M, K // 32), 127, np.uint8)
    one_b = np.full((N, K // 32), 127, np.uint8)
    res = S.fp8_mx32_mm(a, b, one_a, one_b, "f32")
    nA, _ = e4m3_numerator(a)
    nB, _ = e4m3_numerator(b)
    P = nA.astype(object) @ nB.astype(object)
    assert all(Fraction(float(res.exact[m, n])) == Fraction(int(P[m, n]), 2**18)
               for m in range(M) for n in range(N))
    # raising one chunk's scale by one doubles that chunk's share of its row only
    sa = one_a.copy()
    sa[2, 1] += 1
    got = S.fp8_mx32_mm(a, b, sa, one_b, "f32").exact
    part = nA[2, 32:64].astype(np.float64) @ nB[32:64, :].astype(np.float64) * 2.0**-18
    want = res.exact.copy()
    want[2] += part
    assert np.allclose(got, want, rtol=1e-14, atol=0)
    with pytest.raises(ValueError):
        S.fp8_mx32_mm(a, b, one_a[:, :2], one_b, "f32")


# ------------------------------------------- groupwise (1 x 128 on both sides) --

def _gw_random(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K)).astype(np.uint8) & 0xF7          # no NaN codes
    b = rng.integers(0, 256, (K, N)).astype(np.uint8) & 0xF7
    sa = (rng.uniform(0.5, 2, (M, K // 128)) * np.exp2(rng.integers(-12, 12, (M, K // 128)))) \
        .astype(np.float32)
    sb = (rng.uniform(0.5, 2, (K // 128, N)) * np.exp2(rng.integers(-12, 12, (K // 128, N)))) \
        .astype(np.float32)
    sb[0, 1] *= -1
    return a, b, sa, sb


def test_groupwise_brute_force_exact_rationals():
    M, N, K = 3, 5, 384
    a, b, sa, sb = _gw_random(M, N, K, 11)
    res = S.fp8_groupwise(a, b, sa, sb, "f32")
    for m in range(M):
        for n in range(N):
            w = g = Fraction(0)
            for k in range(K):
                t = (e4m3_exact(int(a[m, k])) * e4m3_exact(int(b[k, n]))
                     * Fraction(float(sa[m, k // 128])) * Fraction(float(sb[k // 128, n])))
                w += t
                g += abs(t)
            assert _close(res.exact[m, n], w, g)
            assert Fraction(float(res.out[m, n])) == rne_f32(w)


def test_groupwise_vs_torch_dequant_matmul():
    M, N, K = 20, 72, 512
    a, b, sa, sb = _gw_random(M, N, K, 12)
    res = S.fp8_groupwise(a, b, sa, sb, "f32")
    A = torch.from_numpy(a.copy()).view(torch.float8_e4m3fn).to(torch.float64)
    B = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64)
    A = A * torch.from_numpy(sa.astype(np.float64)).repeat_interleave(128, 1)
    B = B * torch.from_numpy(sb.astype(np.float64)).repeat_interleave(128, 0)
    assert np.allclose(res.exact, (A @ B).numpy(), rtol=1e-12, atol=1e-300)


def test_groupwise_equals_blockwise_when_column_scales_are_constant_per_128_columns():
    M, N, K = 9, 256, 384
    a, b, sa, _ = _gw_random(M, N, K, 13)
    rng = np.random.default_rng(14)
    sbb = rng.uniform(0.25, 4, (K // 128, N // 128)).astype(np.float32)
    gw = S.fp8_groupwise(a, b, sa, np.repeat(sbb, 128, axis=1), "f32")
    bw = S.fp8_blockwise(a, b, sa, sbb, "f32")
    assert np.array_equal(gw.exact, bw.exact)


def test_groupwise_column_scale_multiplies_its_own_column_and_block():
    M, N, K = 4, 32, 384
    a, b, _, _ = _gw_random(M, N, K, 15)
    one_a = np.ones((M, K // 128), np.float32)
    one_b = np.ones((K // 128, N), np.float32)
    base = S.fp8_groupwise(a, b, one_a, one_b, "f32").exact
    sb = one_b.copy()
    sb[2, 7] = 3.0                              # K block 2 of column 7 only
    got = S.fp8_groupwise(a, b, one_a, sb, "f32").exact
    nA, _ = e4m3_numerator(a)
    nB, _ = e4m3_numerator(b)
    part = nA[:, 256:384].astype(np.float64) @ nB[256:384, 7].astype(np.float64) * 2.0**-18
    want = base.copy()
    want[:, 7] += 2 * part
    assert np.allclose(got, want, rtol=1e-14, atol=0)
    sa = one_a.copy()
    sa[1, 0] = 0.5                              # K block 0 of row 1 only
    got = S.fp8_groupwise(a, b, sa, one_b, "f32").exact
    part = nA[1, :128].astype(np.float64) @ nB[:128].astype(np.float64) * 2.0**-18
    want = base.copy()
    want[1] -= 0.5 * part
    assert np.allclose(got, want, rtol=1e-14, atol=0)


def test_groupwise_rejects_blockwise_scale_shapes():
    a, b, sa, _ = _gw_random(4, 256, 256, 16)
    with pytest.raises(ValueError):
        S.fp8_groupwise(a, b, sa, np.ones((2, 2), np.float32))
