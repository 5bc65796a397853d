"""How the gfx950 fp8 matrix instruction sums a 128-long block, measured
through the library's own entry points (GPU).  These tests pin the error
model behind the fp32 accumulation bound of the fp8 parity tests
(``gpu_util.gamma_fp32``):

* a block's 128 products are added in groups of 16 (in the instruction's K
  order; the blockwise kernels hand it 16 consecutive K values per group);
* within a group, an addition drops the bits of the smaller operand below
  2**-13 of the larger operand's binade, toward zero: a term beside 448
  (binade 2**8) keeps only whole multiples of 2**-5.  A group's 15
  additions lose less than 15 * 2**-13 of its magnitude sum, so a block
  errs by less than 2**-9 of its magnitude sum;
* group sums are combined, and blocks accumulated (mx, in place), without
  that loss: products in different groups add exactly where binary32 can
  hold the sum.

With K = 128 and unit scales the blockwise output is the instruction's block
partial itself (the fold multiplies it by 1 and adds it to 0, both exact).
"""

import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsmm
from oracle.formats import e4m3_value
from tests.gpu_util import DEV, dev, host_out, say

pytestmark = pytest.mark.gpu

ONE, BIG = 0x38, 0x7E            # E4M3 codes of 1.0 and 448
SMALL = np.arange(1, 0x7F, dtype=np.uint8)


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def block_partials(a, b_nk):
    """The instruction's fp32 partial of every (row of a, row of b_nk) pair
    of one 128-long block, through bsmm_fp8_blockwise with unit scales."""
    M, N = a.shape[0], b_nk.shape[0]
    y = bsmm.bsmm_fp8_blockwise(dev(a), dev(b_nk).t(), torch.ones((M, 1), device=DEV),
                                torch.ones((1, N // 128), device=DEV), out_dtype="f32")
    return host_out(y).astype(np.float64)


def exact(a, b_nk):
    va, vb = e4m3_value(a), e4m3_value(b_nk)
    return va @ vb.T, np.abs(va) @ np.abs(vb).T


def test_random_full_range_blocks_within_the_model():
    """One million random blocks over the whole E4M3 range: every partial
    within 2**-9 of its magnitude sum (measured about 2**-12)."""
    rng = np.random.default_rng(61)
    a = rng.integers(0, 256, (1024, 128)).astype(np.uint8)
    b = rng.integers(0, 256, (1024, 128)).astype(np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x7E
    b[(b & 0x7F) == 0x7F] = 0x7E
    say("fp8 block partials: 1M random full-range blocks")
    y = block_partials(a, b)
    C, Bd = exact(a, b)
    r = np.abs(y - C) / Bd
    say(f"max |error| / sum|p| = {r.max():.3g} (2^{np.log2(r.max()):.2f}), "
        f"inexact fraction {(r > 0).mean():.3f}")
    assert r.max() < 2.0**-9
    assert (r > 0).any()             # not the correctly rounded fp32 sum


def test_group_of_16_truncates_below_the_largest_product():
    """448 at K 0 and one small x at K 1 keeps only the whole multiples of
    2**-5 of x (13 bits below 448's binade 2**8); fifteen copies of x at
    K 1..15 (the same group) lose less than 2**-5 each and stay within
    2**-9 of the magnitude sum; the same x at K 16..31 or K 32..63 (other
    groups) adds exactly."""
    rows = []
    for lo, hi in ((1, 2), (1, 16), (16, 32), (32, 64)):
        a = np.zeros((len(SMALL), 128), np.uint8)
        a[:, lo:hi] = SMALL[:, None]
        a[:, 0] = BIG
        rows.append(a)
    a = np.concatenate(rows)
    b = np.full((128, 128), ONE, np.uint8)
    say("fp8 block partials: one large and several small products")
    y = block_partials(a, b)[:, 0]
    C, Bd = exact(a, b)
    C, Bd = C[:, 0], Bd[:, 0]
    n = len(SMALL)
    single, same_group, next_group, far_group = (slice(i * n, (i + 1) * n) for i in range(4))
    err = y - C
    x = e4m3_value(SMALL)
    assert np.array_equal(-err[single], np.mod(x, 2.0**-5))
    assert (err[same_group] <= 0).all() and (err[same_group] > -15 * 2.0**-5).all()
    assert (np.abs(err[same_group]) / Bd[same_group] < 2.0**-9).all()
    assert (err[same_group] < 0).any()
    assert (err[next_group] == 0).all() and (err[far_group] == 0).all()


def test_mx_accumulates_blocks_in_place_without_that_loss():
    """448 in block 0 and 128 copies of a small x in block 1: the mx kernel
    accumulates the second block's partial into the first in place, and the
    sum is exact (448 + 128 x fits binary32)."""
    x = np.zeros((1, len(SMALL), 256), np.uint8)
    x[0, :, 0] = BIG
    x[0, :, 128:] = SMALL[:, None]
    w = np.full((1, 128, 256), ONE, np.uint8)
    say("mx in-place accumulation across blocks")
    y = bsmm.bsmm_fp8_mx_bmm(dev(x), dev(w), dev(np.full((1, len(SMALL), 2), 127, np.uint8)),
                             dev(np.full((1, 1, 2), 127, np.uint8)), layout="batch_first",
                             out_dtype="f32")
    got = host_out(y)[0, :, 0].astype(np.float64)
    assert np.array_equal(got, 448.0 + 128.0 * e4m3_value(SMALL))
