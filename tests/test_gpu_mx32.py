"""Parity of the fp8 MX matmul with 32-element e8m0 block scales (GPU).

The scale bytes vary independently per (row, 32-long K chunk) and per
(column, chunk) over a range of 2**30, so a scale applied to the wrong K
values, row or column gives errors far outside the floating-point bar.
Inputs whose sums are exact in fp32 (small integer codes, scales within a
few binades) must match bit for bit.  Every kernel path runs: the tile
kernel with packed and unpacked scales, split-K, stream-K, the eight-wave
fallback of the wide variant, and the skinny kernel.
"""

import numpy as np
import pytest
import torch

from oracle import scaled_mm as S
from oracle.formats import bf16_bits_to_f64
from synth import fp8_mx32_inputs

pytestmark = pytest.mark.gpu


def random_problem(M, N, K, seed, lo=112, hi=142):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K)).astype(np.uint8) & 0xF7          # no NaN codes
    b = rng.integers(0, 256, (N, K)).astype(np.uint8) & 0xF7
    sa = rng.integers(lo, hi, (M, K // 32)).astype(np.uint8)
    sb = rng.integers(lo, hi, (N, K // 32)).astype(np.uint8)
    return dict(a=a, b_nk=b, a_scale=sa, b_scale=sb)


def run(bsmm, p, out, variant=None, split=0):
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    if variant or split:
        bsmm.bsmm_set_override(variant, split)
    try:
        y = bsmm.bsmm_fp8_mx32_mm(d(p["a"]), d(p["b_nk"]).t(), d(p["a_scale"]), d(p["b_scale"]),
                                  out_dtype=out)
        torch.cuda.synchronize()
    finally:
        if variant or split:
            bsmm.bsmm_set_override(None, 0)
    if out == "f32":
        return y.cpu().numpy().astype(np.float64)
    return bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))


def oracle(p, out, rows=None):
    return S.fp8_mx32_mm(p["a"], p["b_nk"].T, p["a_scale"], p["b_scale"], out, rows=rows)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(200, 384, 512), (8, 300, 256), (300, 130, 1024),
                                   (1, 128, 128), (64, 64, 384)])
def test_mx32_parity(gpu_lib, out, M, N, K):
    p = random_problem(M, N, K, M + 7 * N + K)
    rep = S.compare(run(gpu_lib, p, out), oracle(p, out))
    assert rep["ok"], f"{M}x{N}x{K} {out}: {rep}"


@pytest.mark.parametrize("variant,split", [("t128x128", 4), ("t256x256sk", 0), ("w256x256", 0),
                                           ("t64x256", 3), ("t256x128", 0), ("t128x256p", 2),
                                           ("t256x256p", 0), ("t256x256skp", 0)])
def test_mx32_every_kernel_path(gpu_lib, variant, split):
    M, N, K = 600, 640, 1024
    p = random_problem(M, N, K, 77)
    rep = S.compare(run(gpu_lib, p, "bf16", variant, split), oracle(p, "bf16"))
    assert rep["ok"], f"{variant} split {split}: {rep}"


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K,variant", [(64, 256, 1024, None), (5, 96, 512, None),
                                           (300, 384, 768, "t128x128")])
def test_mx32_bit_exact_when_exactly_representable(gpu_lib, out, M, N, K, variant):
    """Codes of the integers 1..8 with random signs and chunk scales 2**-1 ..
    2**1 on each side: every partial sum is a multiple of 2**-2 below 2**18
    (20 significant bits), exact in fp32 in any order."""
    rng = np.random.default_rng(M + K)
    ints = np.array([0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)
    sign = lambda s: (rng.integers(0, 2, s) << 7).astype(np.uint8)
    p = dict(a=ints[rng.integers(0, 8, (M, K))] | sign((M, K)),
             b_nk=ints[rng.integers(0, 8, (N, K))] | sign((N, K)),
             a_scale=rng.integers(126, 129, (M, K // 32)).astype(np.uint8),
             b_scale=rng.integers(126, 129, (N, K // 32)).astype(np.uint8))
    got = run(gpu_lib, p, out, variant, 2 if variant else 0)
    res = oracle(p, out)
    if out == "f32":
        assert np.array_equal(got.astype(np.float32).view(np.uint32), res.out.view(np.uint32))
    else:
        assert np.array_equal(got, bf16_bits_to_f64(res.out))


def test_mx32_scale_lands_on_its_own_chunk(gpu_lib):
    """One chunk of one row carries a huge scale: only that (row, chunk)
    product may grow, so the result shows which K values each scale byte
    multiplies."""
    M, N, K = 32, 128, 256
    p = random_problem(M, N, K, 5, lo=127, hi=128)
    for m, c in ((0, 0), (5, 3), (17, 7), (31, 4)):
        q = dict(p, a_scale=p["a_scale"].copy(), b_scale=p["b_scale"].copy())
        q["a_scale"][m, c] = 127 + 20
        q["b_scale"][(m * 7) % N, (c + 1) % (K // 32)] = 127 - 20
        rep = S.compare(run(gpu_lib, q, "f32"), oracle(q, "f32"))
        assert rep["ok"], f"row {m} chunk {c}: {rep}"


def test_mx32_rejects_shapes(gpu_lib):
    a = torch.zeros((16, 256), dtype=torch.uint8, device="cuda")
    b = torch.zeros((32, 256), dtype=torch.uint8, device="cuda").t()
    with pytest.raises(ValueError):
        gpu_lib.bsmm_fp8_mx32_mm(a, b, torch.zeros((16, 2), dtype=torch.uint8, device="cuda"),
                                 torch.zeros((32, 8), dtype=torch.uint8, device="cuda"))


def test_mx32_full_size_sampled_rows(gpu_lib):
    """The blockwise issue's shape with 32-element MX scales (the measured
    workload), output rows sampled for the oracle."""
    M, N, K = 16640, 5120, 8192
    p = fp8_mx32_inputs(M, N, K, 3)
    got = run(gpu_lib, p, "bf16")
    rows = np.unique(np.concatenate([[0, 16383, 16384, M - 1],
                                     np.random.default_rng(1).choice(M, 24)]))
    rep = S.compare(got[rows], oracle(p, "bf16", rows=rows))
    assert rep["ok"], rep
