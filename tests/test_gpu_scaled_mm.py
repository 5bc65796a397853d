"""Parity of the fp8 scaled_mm (tensorwise / rowwise scales, bias,
scale_result; fp32, bf16 and E4M3 outputs) with the oracle (GPU).

fp32 / bf16 outputs are held to the oracle's floating-point bar (relative
Frobenius error and the elementwise bound); E4M3 outputs to the rule of
``compare_e4m3``, with the fp32 error bound gamma of the accumulation and
the epilogue (products exact, each 128-long MFMA partial summed with at
most 128 roundings, K/128 accumulator additions, four epilogue roundings).
Inputs whose every partial sum is exact in fp32 (small integer codes,
power-of-two scales, quarter-integer bias) must match bit for bit,
ties of the E4M3 rounding included.  Every kernel path runs: the tile
kernel, split-K, the wide-wave kernel, stream-K, and the skinny kernel.
"""

import numpy as np
import pytest
import torch

from oracle import scaled_mm as S
from oracle.formats import bf16_bits_to_f64
from synth import fp8_scaled_mm_inputs

pytestmark = pytest.mark.gpu


def gamma(K):
    return (K / 128) * 2.0**-17 + 8 * 2.0**-24


def dev(x):
    x = np.asarray(x)
    return torch.from_numpy(x if x.ndim == 0 else np.ascontiguousarray(x)).cuda()


def run(bsmm, p, out, sr=None, bias_dtype=torch.float32, variant=None, split=0):
    a = dev(p["a"])
    b = dev(p["b_nk"]).t()
    sa = dev(np.asarray(p["scale_a"], np.float32))
    sb = dev(np.asarray(p["scale_b"], np.float32))
    bias = None if p["bias"] is None else dev(p["bias"]).to(bias_dtype)
    if variant or split:
        bsmm.bsmm_set_override(variant, split)
    try:
        y = bsmm.bsmm_fp8_scaled_mm(a, b, sa, sb, bias=bias, scale_result=sr, out_dtype=out)
        torch.cuda.synchronize()
    finally:
        if variant or split:
            bsmm.bsmm_set_override(None, 0)
    if out == "f32":
        return y.cpu().numpy().astype(np.float64)
    if out == "bf16":
        return bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))
    return y.view(torch.uint8).cpu().numpy()


def check(p, got, out, sr, K, where):
    res = S.fp8_scaled_mm(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], bias=p["bias"],
                          scale_result=sr, out_dtype=out)
    if out == "e4m3":
        rep = S.compare_e4m3(got, res, gamma(K))
    else:
        rep = S.compare(got, res)
    assert rep["ok"], f"{where}: {rep}"
    return rep


@pytest.mark.parametrize("out", ["f32", "bf16", "e4m3"])
@pytest.mark.parametrize("scaling,bias,sr", [("rowwise", None, None), ("rowwise", "f32", 0.5),
                                             ("tensorwise", "bf16", None),
                                             ("tensorwise", None, 4.0)])
@pytest.mark.parametrize("M,N,K", [(200, 384, 512), (8, 300, 256), (300, 130, 1024)])
def test_scaled_mm_parity(gpu_lib, out, scaling, bias, sr, M, N, K):
    p = fp8_scaled_mm_inputs(M, N, K, M + N + K, scaling=scaling, bias=bias)
    bdt = torch.bfloat16 if bias == "bf16" else torch.float32
    got = run(gpu_lib, p, out, sr=sr, bias_dtype=bdt)
    check(p, got, out, sr, K, f"{scaling} bias={bias} sr={sr} {M}x{N}x{K} {out}")


@pytest.mark.parametrize("variant,split", [("t128x128", 4), ("w256x256", 0), ("t256x256sk", 0),
                                           ("t256x128sk", 0), ("t256x256p", 0), ("t64x128", 3)])
@pytest.mark.parametrize("out", ["bf16", "e4m3"])
def test_scaled_mm_every_kernel_path(gpu_lib, variant, split, out):
    M, N, K = 600, 640, 1024
    p = fp8_scaled_mm_inputs(M, N, K, 31, bias="f32")
    got = run(gpu_lib, p, out, sr=0.75, variant=variant, split=split)
    check(p, got, out, 0.75, K, f"{variant} split {split} {out}")


def exact_inputs(M, N, K, seed):
    """Codes of the integers 1..8 with random signs, power-of-two scales,
    quarter-integer bias: every partial sum and epilogue step is exact in
    fp32 (|acc| <= 64 K < 2**24)."""
    rng = np.random.default_rng(seed)
    ints = np.array([0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)   # 1..8
    a = ints[rng.integers(0, 8, (M, K))] | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    b = ints[rng.integers(0, 8, (N, K))] | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    sa = np.exp2(rng.integers(-6, -2, (M, 1))).astype(np.float32)
    sb = np.exp2(rng.integers(-6, -2, (1, N))).astype(np.float32)
    sb[0, ::7] *= -1
    bias = (rng.integers(-400, 400, N) / 4).astype(np.float32)
    return dict(a=a, b_nk=b, scale_a=sa, scale_b=sb, bias=bias)


@pytest.mark.parametrize("out", ["f32", "bf16", "e4m3"])
@pytest.mark.parametrize("M,N,K,variant", [(64, 256, 1024, None), (7, 96, 512, None),
                                           (300, 384, 768, "t128x128")])
def test_scaled_mm_bit_exact_when_exactly_representable(gpu_lib, out, M, N, K, variant):
    p = exact_inputs(M, N, K, M * 3 + K)
    got = run(gpu_lib, p, out, sr=0.5, variant=variant, split=2 if variant else 0)
    res = S.fp8_scaled_mm(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], bias=p["bias"],
                          scale_result=0.5, out_dtype=out)
    if out == "e4m3":
        rep = S.compare_e4m3(got, res, 0.0)
        assert rep["ok"], rep
        # the values are large enough that many land on E4M3 rounding ties
        assert (got & 0x7F).max() == 0x7E or np.abs(res.exact).max() < 448
    elif out == "f32":
        assert np.array_equal(got.astype(np.float32).view(np.uint32),
                              res.out.view(np.uint32))
    else:
        assert np.array_equal(got, bf16_bits_to_f64(res.out))


def test_scaled_mm_empty_k_and_sign_of_zero(gpu_lib):
    M, N = 5, 40
    p = dict(a=np.zeros((M, 0), np.uint8), b_nk=np.zeros((N, 0), np.uint8),
             scale_a=np.linspace(-1, 1, M).astype(np.float32).reshape(M, 1),
             scale_b=np.linspace(1, 2, N).astype(np.float32).reshape(1, N),
             bias=np.linspace(-3, 3, N).astype(np.float32))
    a = torch.zeros((M, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((N, 0), dtype=torch.uint8, device="cuda").t()
    sa, sb = dev(p["scale_a"]), dev(p["scale_b"])
    for bias in (None, dev(p["bias"])):
        y = gpu_lib.bsmm_fp8_scaled_mm(a, b, sa, sb, bias=bias, scale_result=2.0, out_dtype="f32")
        q = dict(p, bias=None if bias is None else p["bias"])
        res = S.fp8_scaled_mm(q["a"], q["b_nk"].T, q["scale_a"], q["scale_b"], bias=q["bias"],
                              scale_result=2.0, out_dtype="f32")
        assert np.array_equal(y.cpu().numpy().view(np.uint32), res.out.view(np.uint32))


def test_scaled_mm_rejects_shapes(gpu_lib):
    a = torch.zeros((16, 256), dtype=torch.uint8, device="cuda")
    b = torch.zeros((32, 256), dtype=torch.uint8, device="cuda").t()
    with pytest.raises(ValueError):
        gpu_lib.bsmm_fp8_scaled_mm(a, b, torch.ones(16, 2, device="cuda"),
                                   torch.ones(2, 1, device="cuda"))
    with pytest.raises(ValueError):
        gpu_lib.bsmm_fp8_scaled_mm(a, b, torch.ones(16, 1, device="cuda"),
                                   torch.ones(1, 32, device="cuda"),
                                   bias=torch.ones(31, device="cuda"))


def test_scaled_mm_full_size_sampled_rows(gpu_lib):
    """The blockwise-issue shape with rowwise scales and a bias (the
    measured workload), output rows sampled for the oracle."""
    M, N, K = 16640, 5120, 8192
    p = fp8_scaled_mm_inputs(M, N, K, 3, bias="bf16")
    got = run(gpu_lib, p, "bf16", bias_dtype=torch.bfloat16)
    rows = np.unique(np.concatenate([[0, 16383, 16384, M - 1],
                                     np.random.default_rng(0).choice(M, 28)]))
    res = S.fp8_scaled_mm(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], bias=p["bias"],
                          out_dtype="bf16", rows=rows)
    rep = S.compare(got[rows], res)
    assert rep["ok"], rep
