"""Parity of the fp8 matmuls of a blockwise fp8 linear layer's backward pass
with the oracle (GPU): the groupwise GEMM (1 x 128 groups on both operands,
the weight gradient) and the blockwise GEMM at the input-gradient shape.

The scales vary independently per (row, K block) and per (K block, column)
over a range of 2**24, so a scale applied to the wrong row, column or K
block gives errors far outside the floating-point bar.  Inputs whose sums
are exact in fp32 (small integer codes, power-of-two scales) must match bit
for bit.  Every packed-scale kernel path runs: the tile kernel at three tile
shapes, split-K, stream-K and the eight-wave variant of the wide kernel.
"""

import numpy as np
import pytest
import torch

from oracle import scaled_mm as S
from oracle.formats import bf16_bits_to_f64
from synth import config_inputs, CONFIGS

pytestmark = pytest.mark.gpu


def random_problem(M, N, K, seed, span=12):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 256, (M, K)).astype(np.uint8) & 0xF7          # no NaN codes
    b = rng.integers(0, 256, (N, K)).astype(np.uint8) & 0xF7
    KB = K // 128
    sa = (rng.uniform(0.5, 1, (M, KB)) * np.exp2(rng.integers(-span, span, (M, KB)))) \
        .astype(np.float32)
    sb = (rng.uniform(0.5, 1, (KB, N)) * np.exp2(rng.integers(-span, span, (KB, N)))) \
        .astype(np.float32)
    return dict(a=a, b_nk=b, scale_a=sa, scale_b=sb)


def run(bsmm, p, out, variant=None, split=0, sb_col_major=False):
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    sb = d(p["scale_b"].T).t() if sb_col_major else d(p["scale_b"])
    if variant or split:
        bsmm.bsmm_set_override(variant, split)
    try:
        y = bsmm.bsmm_fp8_groupwise(d(p["a"]), d(p["b_nk"]).t(), d(p["scale_a"]), sb,
                                    out_dtype=out)
        torch.cuda.synchronize()
    finally:
        if variant or split:
            bsmm.bsmm_set_override(None, 0)
    if out == "f32":
        return y.cpu().numpy().astype(np.float64)
    return bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))


def oracle(p, out, rows=None):
    return S.fp8_groupwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], out, rows=rows)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(200, 384, 512), (8, 300, 256), (300, 130, 1024),
                                   (1, 128, 128), (64, 64, 384), (520, 777, 640)])
def test_groupwise_parity(gpu_lib, out, M, N, K):
    print(f"groupwise {M}x{N}x{K} {out}", flush=True)
    p = random_problem(M, N, K, M + 7 * N + K)
    rep = S.compare(run(gpu_lib, p, out), oracle(p, out))
    assert rep["ok"], f"{M}x{N}x{K} {out}: {rep}"


@pytest.mark.parametrize("variant,split", [("t256x256p", 0), ("t256x256p", 3), ("t256x128p", 0),
                                           ("t128x256p", 2), ("t256x256skp", 0),
                                           ("w256x256p", 0)])
def test_groupwise_every_kernel_path(gpu_lib, variant, split):
    print(f"groupwise {variant} split {split}", flush=True)
    M, N, K = 600, 640, 1024
    p = random_problem(M, N, K, 77)
    rep = S.compare(run(gpu_lib, p, "bf16", variant, split), oracle(p, "bf16"))
    assert rep["ok"], f"{variant} split {split}: {rep}"


def test_groupwise_column_major_scale_b(gpu_lib):
    """scale_b given as the transpose of an [N, K/128] array (the layout of
    per-column quantisation) goes through the same packing."""
    p = random_problem(256, 384, 768, 5)
    rep = S.compare(run(gpu_lib, p, "f32", sb_col_major=True), oracle(p, "f32"))
    assert rep["ok"], rep


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K,variant", [(64, 256, 1024, None), (5, 96, 512, None),
                                           (300, 384, 768, "t256x128p")])
def test_groupwise_bit_exact_when_exactly_representable(gpu_lib, out, M, N, K, variant):
    """Codes of the integers 1..8 with random signs and scales 2**-1 .. 2**1
    on each side: every partial sum is a multiple of 2**-2 below 2**18, exact
    in fp32 in any order."""
    print(f"groupwise exact {M}x{N}x{K} {out} {variant}", flush=True)
    rng = np.random.default_rng(M + K)
    ints = np.array([0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)
    sign = lambda s: (rng.integers(0, 2, s) << 7).astype(np.uint8)
    p = dict(a=ints[rng.integers(0, 8, (M, K))] | sign((M, K)),
             b_nk=ints[rng.integers(0, 8, (N, K))] | sign((N, K)),
             scale_a=np.exp2(rng.integers(-1, 2, (M, K // 128))).astype(np.float32),
             scale_b=np.exp2(rng.integers(-1, 2, (K // 128, N))).astype(np.float32))
    got = run(gpu_lib, p, out, variant, 2 if variant else 0)
    res = oracle(p, out)
    if out == "f32":
        assert np.array_equal(got.astype(np.float32).view(np.uint32), res.out.view(np.uint32))
    else:
        assert np.array_equal(got, bf16_bits_to_f64(res.out))


def test_groupwise_scales_land_on_their_own_row_column_and_block(gpu_lib):
    """One (row, K block) and one (K block, column) carry huge scales: only
    those products may grow, so the result shows which K values, rows and
    columns each staged scale multiplies."""
    M, N, K = 256, 256, 512
    p = random_problem(M, N, K, 9, span=1)
    for m, n, kb in ((0, 0, 0), (77, 130, 3), (255, 255, 2), (130, 3, 1)):
        q = dict(p, scale_a=p["scale_a"].copy(), scale_b=p["scale_b"].copy())
        q["scale_a"][m, kb] = 2.0**20
        q["scale_b"][kb, n] = 2.0**-20
        rep = S.compare(run(gpu_lib, q, "f32"), oracle(q, "f32"))
        assert rep["ok"], f"row {m} column {n} block {kb}: {rep}"


def test_groupwise_empty_k(gpu_lib):
    a = torch.zeros((40, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((72, 0), dtype=torch.uint8, device="cuda").t()
    y = gpu_lib.bsmm_fp8_groupwise(a, b, torch.zeros((40, 0), device="cuda"),
                                   torch.zeros((0, 72), device="cuda"), out_dtype="f32",
                                   out=torch.full((40, 72), 7.0, device="cuda"))
    assert not y.cpu().numpy().any()


def test_groupwise_rejects_blockwise_scale_shapes(gpu_lib):
    a = torch.zeros((16, 256), dtype=torch.uint8, device="cuda")
    b = torch.zeros((256, 256), dtype=torch.uint8, device="cuda").t()
    with pytest.raises(ValueError):
        gpu_lib.bsmm_fp8_groupwise(a, b, torch.ones(16, 2, device="cuda"),
                                   torch.ones(2, 2, device="cuda"))


def _sampled(got, res_fn, M, seed, edges):
    """Compare sampled output rows: the first and last, the rows on both
    sides of each launch boundary in ``edges``, and random ones."""
    rows = np.unique(np.concatenate([[0, M - 1], edges,
                                     np.random.default_rng(seed).choice(M, 22)]))
    rep = S.compare(got[rows], res_fn(rows))
    assert rep["ok"], rep


def test_weight_gradient_full_size_sampled_rows(gpu_lib):
    """dW = dY^T X of the 16640-token layer (5120 x 8192 over 16640 tokens),
    the measured workload, output rows sampled for the oracle (rows 4095 and
    4096 sit on either side of the bulk launch's end and the split-K tail's
    start)."""
    c = CONFIGS["c3w"]
    print("groupwise c3w", flush=True)
    p = config_inputs("c3w")
    got = run(gpu_lib, p, "bf16")
    _sampled(got, lambda r: oracle(p, "bf16", rows=r), c["M"], 4, [4095, 4096])


def test_input_gradient_full_size_sampled_rows(gpu_lib):
    """dX = dY W of the same layer: a blockwise GEMM over the 5120 output
    features (16640 x 8192 x 5120), output rows sampled."""
    c = CONFIGS["c3d"]
    print("blockwise c3d", flush=True)
    p = config_inputs("c3d")
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = gpu_lib.bsmm_fp8_blockwise(d(p["a"]), d(p["b_nk"]).t(), d(p["scale_a"]),
                                   d(p["scale_b"]), out_dtype="bf16")
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))
    _sampled(got, lambda r: S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"],
                                            "bf16", rows=r), c["M"], 5, [8191, 8192, 16383, 16384])
