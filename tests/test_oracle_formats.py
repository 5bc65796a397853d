"""Pins for the oracle's number formats (CPU).

E4M3FN and E8M0 decode are checked against hand-derived values of the OCP
format definitions, against PyTorch's own CPU float8 conversions (a library
routine written independently of the oracle), and for monotonicity.  Rounding
to binary32 and bfloat16 is checked against exact rational rounding and
against PyTorch's conversion.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from tests.exact import e4m3_exact, rne_bf16, rne_f32

ALL = np.arange(256, dtype=np.uint8)


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0**-9), (0x07, 7 * 2.0**-9), (0x08, 2.0**-6),
    (0x09, 9 * 2.0**-9), (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0),
    (0x77, 240.0), (0x7E, 448.0), (0x81, -(2.0**-9)), (0xB8, -1.0),
    (0xFE, -448.0),
])
def test_e4m3_hand_values(code, value):
    assert F.e4m3_value(np.uint8(code)) == value


def test_e4m3_nan_codes_and_signed_zero():
    v = F.e4m3_value(ALL)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isnan(v).sum() == 2
    assert v[0x80] == 0.0 and np.signbit(v[0x80])


def test_e4m3_matches_torch_all_codes():
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_value(ALL)
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    assert np.array_equal(ref[~both_nan], ours[~both_nan])


def test_e4m3_matches_exact_definition_and_numerator():
    n, nan = F.e4m3_numerator(ALL)
    for c in range(256):
        if nan[c]:
            continue
        assert Fraction(int(n[c]), 512) == e4m3_exact(c)
    assert np.abs(n[~nan]).max() == 229376


def test_e4m3_monotone_positive_codes():
    v = F.e4m3_value(ALL[:127])
    assert np.all(np.diff(v) > 0)


def test_e8m0_values_and_torch():
    v = F.e8m0_value(ALL)
    assert v[0] == 2.0**-127 and v[127] == 1.0 and v[128] == 2.0
    assert v[254] == 2.0**127 and np.isnan(v[255])
    ref = torch.from_numpy(ALL.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(ref[:255], v[:255]) and np.isnan(ref[255])


def test_round_f32_ties_to_even():
    cases = {2**24 + 1: 2**24, 2**24 + 3: 2**24 + 4, 2**25 + 2: 2**25,
             2**25 + 6: 2**25 + 8, 2**25 + 5: 2**25 + 4, -(2**24 + 1): -(2**24)}
    got = F.round_f32(np.array(list(cases), dtype=np.int64))
    assert [int(g) for g in got] == list(cases.values())


def test_round_f32_vs_exact_random_ints():
    rng = np.random.default_rng(0)
    x = rng.integers(-(2**31), 2**31, size=2000)
    got = F.round_f32(x)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == rne_f32(int(xi))


def test_bf16_from_f32_vs_torch_and_exact():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ties = np.array([1 + 2.0**-8, 1 + 3 * 2.0**-8, -(1 + 2.0**-8), 3.3895314e38,
                     0.0, -0.0, 1e-40, np.inf, -np.inf], dtype=np.float32)
    x = np.concatenate([x, ties])
    ours = F.bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert F.bf16_bits_to_f64(F.bf16_bits_from_f32(np.float32(1 + 2.0**-8))) == 1.0
    assert F.bf16_bits_to_f64(F.bf16_bits_from_f32(np.float32(1 + 3 * 2.0**-8))) == 1 + 2.0**-6
    for xi in x[:500]:
        got = F.bf16_bits_to_f64(F.bf16_bits_from_f32(np.array([xi])))[0]
        assert Fraction(float(got)) == rne_bf16(float(xi))


def test_bf16_from_f64_single_rounding():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    # a value just above a bf16 tie: one rounding goes up, rounding via fp32
    # first lands on the tie and goes to even (down)
    x = np.concatenate([x, [1 + 2.0**-8 + 2.0**-40, 1 + 2.0**-8]])
    got = F.bf16_bits_to_f64(F.bf16_bits_from_f64(x))
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == rne_bf16(float(xi))
    assert got[-2] == 1 + 2.0**-7 and got[-1] == 1.0
    # on values exactly representable in binary32 it equals the fp32 route
    x32 = x[:-2].astype(np.float32)
    assert np.array_equal(F.bf16_bits_from_f64(x32.astype(np.float64)),
                          F.bf16_bits_from_f32(x32))
    assert F.bf16_bits_to_f64(F.bf16_bits_from_f64(np.array([3.5e38])))[0] == np.inf
