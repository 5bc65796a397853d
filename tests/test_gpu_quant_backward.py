"""Parity of the backward pass's quantisers, and of the backward GEMMs fed
by them, with the oracle (GPU).

Codes and scales must be bit-identical to oracle/quant.py
(``quant_fp8_columns``, ``quant_fp8_weight_blocks``) on the same inputs:
seeded columns across many binades, zero and underflowing groups, -0, ragged
column counts, both input dtypes, each output layout of the weight
quantiser.  Then the two backward GEMMs run end to end from bf16 tensors
(quantise on the GPU, multiply on the GPU) against the oracle's quantisers
and matmuls: the weight gradient dW = dY^T X (groupwise) and the input
gradient dX = dY W (blockwise, the weight read through its transposed
codes), plus the forward product through the untransposed codes.  The
layer's full-size activations run with sampled columns compared one by one.
"""

import numpy as np
import pytest
import torch

from oracle import quant as Q
from oracle import scaled_mm as S
from oracle.formats import bf16_bits_to_f64
from synth import activations

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def device_input(x32, dt):
    """(device tensor of dtype dt, the fp32 values it holds)."""
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(DTYPES[dt])
    return t.cuda(), t.float().numpy()


def u8(t):
    return t.view(torch.uint8).cpu().numpy()


def assert_same(got, want, where):
    (qg, sg), (qw, sw) = got, want
    bad = np.argwhere(sg.view(np.uint32) != sw.view(np.uint32))
    assert bad.size == 0, f"{where}: {len(bad)} scales differ, first {bad[:4].tolist()}"
    bad = np.argwhere(qg != qw)
    assert bad.size == 0, (f"{where}: {len(bad)} codes differ, first {bad[:4].tolist()} got "
                           f"{qg[tuple(bad[0])]} want {qw[tuple(bad[0])]}")


def spread(R, C, seed, *, zero_cols=(), tiny_cols=(), neg_zero=True):
    """Columns at random binades (2**-30 .. 2**30), some all-zero, some so
    small that amax / 448 underflows, -0 entries."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((R, C)) * np.exp2(rng.integers(-30, 30, (1, C)))).astype(np.float32)
    for c in zero_cols:
        x[:, c] = 0.0
    for c in tiny_cols:
        x[:, c] = rng.standard_normal(R).astype(np.float32) * np.float32(2.0**-140)
    if neg_zero:
        x[3, :] = -0.0
    return x


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("R,C", [(128, 64), (256, 200), (384, 8), (1280, 520)])
def test_columns_parity(gpu_lib, dt, R, C):
    print(f"quant columns {R}x{C} {dt}", flush=True)
    x = spread(R, C, R + C, zero_cols=(0, C - 1), tiny_cols=(min(5, C - 1),))
    xd, xv = device_input(x, dt)
    q_t, s = gpu_lib.bsmm_quant_fp8_columns(xd)
    torch.cuda.synchronize()
    assert tuple(q_t.shape) == (C, R) and tuple(s.shape) == (R // 128, C)
    assert_same((u8(q_t), s.cpu().numpy()), Q.quant_fp8_columns(xv), f"columns {R}x{C} {dt}")


def test_columns_strided_input_and_scale(gpu_lib):
    """x as a column slice of a wider row-major array; scale written through a
    transposed [C, R/128] view."""
    R, C = 256, 96
    base = spread(R, 160, 7)
    xd_full, xv_full = device_input(base, "bf16")
    xd, xv = xd_full[:, 32:32 + C], xv_full[:, 32:32 + C]
    sc = torch.empty((C, R // 128), dtype=torch.float32, device="cuda").t()
    q_t, s = gpu_lib.bsmm_quant_fp8_columns(xd, scale=sc)
    torch.cuda.synchronize()
    assert_same((u8(q_t), s.cpu().numpy()), Q.quant_fp8_columns(xv), "strided columns")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("R,C", [(128, 128), (256, 384), (512, 256)])
def test_weight_parity(gpu_lib, dt, R, C):
    print(f"quant weight {R}x{C} {dt}", flush=True)
    rng = np.random.default_rng(R * C)
    w = (rng.standard_t(3, (R, C)) * np.exp2(rng.integers(-25, 25, (R // 128, 1, C // 128, 1)))
         .repeat(128, 1).repeat(128, 3).reshape(R, C)).astype(np.float32)
    w[:128, :128] = 0.0                                    # a zero block
    if C > 128:
        w[:128, 128:256] *= np.float32(2.0**-150)          # an underflowing block
    w[5, :] = -0.0
    wd, wv = device_input(w, dt)
    q, q_t, s = gpu_lib.bsmm_quant_fp8_weight(wd)
    torch.cuda.synchronize()
    qw, sw = Q.quant_fp8_weight_blocks(wv)
    assert_same((u8(q), s.cpu().numpy()), (qw, sw), f"weight {R}x{C} {dt} plain")
    assert np.array_equal(u8(q_t), qw.T), f"weight {R}x{C} {dt}: transposed codes differ"
    # each layout alone
    q1, none1, s1 = gpu_lib.bsmm_quant_fp8_weight(wd, transposed=False)
    none2, q2, s2 = gpu_lib.bsmm_quant_fp8_weight(wd, plain=False)
    torch.cuda.synchronize()
    assert none1 is None and none2 is None
    assert np.array_equal(u8(q1), qw) and np.array_equal(u8(q2), qw.T)
    assert np.array_equal(s1.cpu().numpy(), sw) and np.array_equal(s2.cpu().numpy(), sw)


def bf16_out(y):
    return bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))


def test_weight_gradient_end_to_end(gpu_lib):
    """dW = dY^T X: both operands quantised in groups of 128 tokens down
    their columns, then the groupwise GEMM."""
    T, N, K = 640, 256, 384
    dy_d, dy = device_input(activations((T, N), 11, row_scale_log2=(-4, 4)), "bf16")
    x_d, xv = device_input(activations((T, K), 12, dist="t"), "bf16")
    dyq_t, s_dy = gpu_lib.bsmm_quant_fp8_columns(dy_d)
    xq_t, s_x = gpu_lib.bsmm_quant_fp8_columns(x_d)
    dw = gpu_lib.bsmm_fp8_groupwise(dyq_t, xq_t.t(), s_dy.t(), s_x, out_dtype="bf16")
    torch.cuda.synchronize()
    oq_dy, os_dy = Q.quant_fp8_columns(dy)
    oq_x, os_x = Q.quant_fp8_columns(xv)
    assert_same((u8(dyq_t), s_dy.cpu().numpy()), (oq_dy, os_dy), "dY columns")
    assert_same((u8(xq_t), s_x.cpu().numpy()), (oq_x, os_x), "X columns")
    res = S.fp8_groupwise(oq_dy, oq_x.T, os_dy.T, os_x, "bf16")
    rep = S.compare(bf16_out(dw), res)
    assert rep["ok"], rep


def test_input_gradient_and_forward_end_to_end(gpu_lib):
    """dX = dY W with W's transposed codes and its block scales as stored;
    Y = X W^T with its plain codes and the transposed scales."""
    M, N, K = 300, 256, 384
    dy_d, dy = device_input(activations((M, N), 21), "bf16")
    x_d, xv = device_input(activations((M, K), 22), "bf16")
    w_d, wv = device_input(activations((N, K), 23) * np.float32(0.02), "bf16")
    wq, wq_t, s_w = gpu_lib.bsmm_quant_fp8_weight(w_d)
    dyq, s_dy = gpu_lib.bsmm_quant_fp8_blockwise(dy_d)
    xq, s_x = gpu_lib.bsmm_quant_fp8_blockwise(x_d)
    dx = gpu_lib.bsmm_fp8_blockwise(dyq, wq_t.t(), s_dy, s_w, out_dtype="bf16")
    y = gpu_lib.bsmm_fp8_blockwise(xq, wq.t(), s_x, s_w.t(), out_dtype="bf16")
    torch.cuda.synchronize()
    oq_w, os_w = Q.quant_fp8_weight_blocks(wv)
    oq_dy, os_dy = Q.quant_fp8_blockwise(dy)
    oq_x, os_x = Q.quant_fp8_blockwise(xv)
    assert np.array_equal(u8(wq_t), oq_w.T) and np.array_equal(u8(dyq), oq_dy)
    rep = S.compare(bf16_out(dx), S.fp8_blockwise(oq_dy, oq_w, os_dy, os_w, "bf16"))
    assert rep["ok"], f"dX: {rep}"
    rep = S.compare(bf16_out(y), S.fp8_blockwise(oq_x, oq_w.T, os_x, os_w.T, "bf16"))
    assert rep["ok"], f"Y: {rep}"


def test_layer_activations_full_size_sampled_columns(gpu_lib):
    """X [16640, 8192] and dY [16640, 5120] of the 16640-token layer and its
    weight W [5120, 8192]: codes and scales of sampled columns (and, for the
    weight, sampled 128-column block stripes) against the oracle."""
    print("quant backward full size", flush=True)
    rng = np.random.default_rng(5)
    for shape, seed in (((16640, 8192), 31), ((16640, 5120), 32)):
        xd, xv = device_input(activations(shape, seed, row_scale_log2=(-3, 3)), "bf16")
        q_t, s = gpu_lib.bsmm_quant_fp8_columns(xd)
        torch.cuda.synchronize()
        cols = np.unique(np.concatenate([[0, shape[1] - 1], rng.choice(shape[1], 14)]))
        qo, so = Q.quant_fp8_columns(xv[:, cols])
        assert_same((q_t[cols].view(torch.uint8).cpu().numpy(), s[:, cols].cpu().numpy()),
                    (qo, so), f"columns {shape}")
        del xd, q_t, s
    wd, wv = device_input(activations((5120, 8192), 33) * np.float32(0.02), "bf16")
    q, q_t, s = gpu_lib.bsmm_quant_fp8_weight(wd)
    torch.cuda.synchronize()
    for cb in (0, 29, 63):
        stripe = wv[:, 128 * cb:128 * (cb + 1)]
        qo, so = Q.quant_fp8_weight_blocks(stripe)
        assert np.array_equal(q[:, 128 * cb:128 * (cb + 1)].view(torch.uint8).cpu().numpy(), qo)
        assert np.array_equal(q_t[128 * cb:128 * (cb + 1)].view(torch.uint8).cpu().numpy(), qo.T)
        assert np.array_equal(s[:, cb].cpu().numpy(), so[:, 0])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("R,C", [(128, 128), (256, 384), (384, 256), (1280, 640)])
def test_blockwise_and_columns_from_one_read(gpu_lib, dt, R, C):
    """The fused quantiser equals the two separate quantisations bit for bit:
    the row blocks of quant_fp8_blockwise and the column groups of
    quant_fp8_columns, zero and underflowing rows and columns included."""
    print(f"quant rows+columns {R}x{C} {dt}", flush=True)
    x = spread(R, C, 3 * R + C, zero_cols=(0,), tiny_cols=(C - 1,))
    x[7, :] = 0.0                                       # a zero row (all its blocks)
    x[9, 128:] *= np.float32(2.0**-150)                 # underflowing row blocks
    xd, xv = device_input(x, dt)
    q, s, q_t, s_t = gpu_lib.bsmm_quant_fp8_blockwise_columns(xd)
    torch.cuda.synchronize()
    assert_same((u8(q), s.cpu().numpy()), Q.quant_fp8_blockwise(xv), f"rows {R}x{C} {dt}")
    assert_same((u8(q_t), s_t.cpu().numpy()), Q.quant_fp8_columns(xv), f"columns {R}x{C} {dt}")


def test_blockwise_and_columns_full_size_sampled(gpu_lib):
    """X [16640, 8192] of the 16640-token layer: sampled rows and columns."""
    print("quant rows+columns full size", flush=True)
    xd, xv = device_input(activations((16640, 8192), 34, row_scale_log2=(-3, 3)), "bf16")
    q, s, q_t, s_t = gpu_lib.bsmm_quant_fp8_blockwise_columns(xd)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 16639], rng.choice(16640, 14)]))
    qo, so = Q.quant_fp8_blockwise(xv[rows])
    assert_same((q[rows].view(torch.uint8).cpu().numpy(), s[rows].cpu().numpy()), (qo, so),
                "rows")
    cols = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 14)]))
    qo, so = Q.quant_fp8_columns(xv[:, cols])
    assert_same((q_t[cols].view(torch.uint8).cpu().numpy(), s_t[:, cols].cpu().numpy()),
                (qo, so), "columns")
