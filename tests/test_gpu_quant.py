"""Parity of the HIP dynamic quantisers with the oracle (GPU).

Codes and scales must be bit-identical to oracle/quant.py on the same
inputs: seeded random rows across many binades, every e4m3 rounding tie
(and the values one ulp either side), int8 half-integer ties, zero, -0,
underflowing and subnormal scales, the slow-division range, and the e8m0
exponent boundaries amax = 448 * 2**k.  The activation shapes of the
matmul workloads run at full size with sampled rows compared one by one.
"""

import numpy as np
import pytest
import torch

from oracle import quant as Q
from synth import activations
from tests.exact import e4m3_exact

pytestmark = pytest.mark.gpu

DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def device_input(x32, dt):
    """(device tensor of dtype dt, the fp32 values it holds) -- bf16 inputs
    reach the oracle exactly as the kernel sees them."""
    t = torch.from_numpy(np.ascontiguousarray(x32)).to(DTYPES[dt])
    return t.cuda(), t.float().numpy()


def run(bsmm, kind, xd):
    fn = {"int8": bsmm.bsmm_quant_int8_rowwise, "fp8": bsmm.bsmm_quant_fp8_blockwise,
          "mx": bsmm.bsmm_quant_fp8_mx,
          "mx32": lambda x: bsmm.bsmm_quant_fp8_mx(x, block=32)}[kind]
    q, s = fn(xd)
    torch.cuda.synchronize()
    q = q.view(torch.uint8).cpu().numpy() if kind != "int8" else q.cpu().numpy()
    return q, s.cpu().numpy()


def oracle(kind, xv):
    rows = xv.reshape(-1, xv.shape[-1])
    if kind == "int8":
        q, s = Q.quant_int8_rowwise(rows)
        return q, s.reshape(-1, 1)
    if kind == "fp8":
        return Q.quant_fp8_blockwise(rows)
    if kind == "mx32":
        return Q.quant_fp8_mx(rows, block=32)
    return Q.quant_fp8_mx(rows)


def assert_same(kind, got, want, where=""):
    (qg, sg), (qw, sw) = got, want
    qg = qg.reshape(qw.shape)
    sg = sg.reshape(sw.shape)
    if sw.dtype == np.float32:
        bad = np.argwhere(sg.view(np.uint32) != sw.view(np.uint32))
        assert bad.size == 0, f"{kind}{where}: {len(bad)} scales differ, first {bad[:4].tolist()}"
    else:
        assert np.array_equal(sg, sw), f"{kind}{where}: e8m0 scales differ"
    bad = np.argwhere(qg.view(np.uint8) != qw.view(np.uint8))
    assert bad.size == 0, (f"{kind}{where}: {len(bad)} codes differ, first {bad[:4].tolist()} "
                           f"got {qg.view(np.uint8)[tuple(bad[0])]} want "
                           f"{qw.view(np.uint8)[tuple(bad[0])]}")


# ---------------------------------------------------------------- random rows --

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,K", [(37, 8), (37, 520), (5, 4096), (6, 4104), (3, 12288),
                                 (129, 1024), (7, 1536), (9, 2048), (4, 8200)])
def test_int8_rows_parity(gpu_lib, dt, M, K):
    x = activations((M, K), seed=M * 7 + K, dist="t", row_scale_log2=(-40, 40))
    xd, xv = device_input(x, dt)
    assert_same("int8", run(gpu_lib, "int8", xd), oracle("int8", xv), f" {dt} {M}x{K}")


@pytest.mark.parametrize("kind", ["fp8", "mx", "mx32"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("M,K", [(37, 128), (37, 384), (21, 7168), (1, 128), (64, 1024)])
def test_fp8_blocks_parity(gpu_lib, kind, dt, M, K):
    x = activations((M, K), seed=M * 11 + K, dist="normal", row_scale_log2=(-60, 60))
    # vary the magnitude per block as well, so neighbouring blocks differ
    rng = np.random.default_rng(M + K)
    bl = 32 if kind == "mx32" else 128
    x = (x.reshape(M, K // bl, bl) *
         np.exp2(rng.integers(-20, 20, (M, K // bl, 1))).astype(np.float32)).reshape(M, K)
    xd, xv = device_input(x, dt)
    assert_same(kind, run(gpu_lib, kind, xd), oracle(kind, xv), f" {dt} {M}x{K}")


# ----------------------------------------------------------- ties and edges --

def e4m3_tie_blocks():
    """Blocks whose amax is exactly 448 (scale 1, e8m0 exponent 0) holding every
    midpoint between adjacent e4m3 values and the fp32 values one ulp either
    side, both signs; all are exact in bf16 as well except the neighbours."""
    pos = np.array([float(e4m3_exact(c)) for c in range(0x7F)], dtype=np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9)), pos.astype(np.float32)])
    vals = np.concatenate([vals, -vals])
    per = 127
    nb = -(-len(vals) // per)
    out = np.zeros((nb, 128), np.float32)
    out[:, 0] = 448.0
    flat = np.zeros(nb * per, np.float32)
    flat[:len(vals)] = vals
    out[:, 1:] = flat.reshape(nb, per)
    return out


def edge_blocks():
    """Rows of 128 that exercise the special cases of the definition."""
    b = []
    z = np.zeros(128, np.float32)
    b.append(z.copy())                                   # all zero
    r = z.copy(); r[5] = -0.0; r[9] = -0.0; b.append(r)  # all zero with -0
    r = z.copy(); r[3] = np.float32(2.0**-149); r[4] = -np.float32(2.0**-149); b.append(r)
    r = z.copy(); r[0] = np.float32(2.0**-120); r[1] = -np.float32(2.0**-125); r[2] = -0.0
    b.append(r)                                          # subnormal fp32 scale, slow division
    r = np.linspace(-1, 1, 128).astype(np.float32) * np.float32(2.0**-75); b.append(r)
    r = np.linspace(-1, 1, 128).astype(np.float32) * np.float32(3e38); b.append(r)
    for k in (-100, -8, 0, 5, 100):                      # e8m0 exponent boundaries
        for a in (np.float32(448.0 * 2.0**k),
                  np.nextafter(np.float32(448.0 * 2.0**k), np.float32(np.inf)),
                  np.nextafter(np.float32(448.0 * 2.0**k), np.float32(0))):
            r = np.linspace(-0.9, 0.9, 128).astype(np.float32) * a
            r[17] = -a
            b.append(r.astype(np.float32))
    r = z.copy(); r[1] = np.float32(2.0**-130); r[2] = -np.float32(2.0**-139); b.append(r)
    return np.stack(b)


@pytest.mark.parametrize("kind", ["fp8", "mx", "mx32"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fp8_ties_and_edges(gpu_lib, kind, dt):
    x = np.concatenate([e4m3_tie_blocks(), edge_blocks()])
    # two blocks per row so both columns of blocks are exercised
    if len(x) % 2:
        x = np.concatenate([x, np.zeros((1, 128), np.float32)])
    x = x.reshape(-1, 256)
    xd, xv = device_input(x, dt)
    assert_same(kind, run(gpu_lib, kind, xd), oracle(kind, xv), f" {dt} edges")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_int8_ties_and_edges(gpu_lib, dt):
    rows = []
    r = np.zeros(256, np.float32)
    r[0] = 127.0
    r[1:255] = np.arange(-127, 127) + 0.5             # every half-integer tie
    rows.append(r)
    rows.append(-r)
    e = edge_blocks()
    rows += [np.concatenate([v, v[::-1]]) for v in e]
    x = np.stack(rows).astype(np.float32)
    xd, xv = device_input(x, dt)
    assert_same("int8", run(gpu_lib, "int8", xd), oracle("int8", xv), f" {dt} edges")


# ------------------------------------------------------ layouts and strides --

def test_strided_input_output_and_column_major_scales(gpu_lib):
    M, K = 45, 1024
    x = activations((M, K + 256), seed=5, row_scale_log2=(-8, 8))
    xd, xv = device_input(x, "bf16")
    xs, xvs = xd[:, 128:128 + K], xv[:, 128:128 + K]           # ldx = K + 256
    qbig = torch.full((M, K + 64), 0x55, dtype=torch.uint8, device="cuda")
    q = qbig[:, :K].view(torch.float8_e4m3fn)
    sc = torch.full((K // 128, M), -1.0, device="cuda").t()     # s_m = 1, s_kb = M
    gpu_lib.bsmm_quant_fp8_blockwise(xs, q=q, scale=sc)
    torch.cuda.synchronize()
    qw, sw = Q.quant_fp8_blockwise(xvs)
    assert np.array_equal(qbig[:, :K].cpu().numpy(), qw)
    assert np.all(qbig[:, K:].cpu().numpy() == 0x55)           # padding untouched
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), sw.view(np.uint32))

    qi = torch.full((M, K + 16), 7, dtype=torch.int8, device="cuda")
    si = torch.full((M, 1), -1.0, device="cuda")
    gpu_lib.bsmm_quant_int8_rowwise(xs, q=qi[:, :K], scale=si)
    torch.cuda.synchronize()
    qw, sw = Q.quant_int8_rowwise(xvs)
    assert np.array_equal(qi[:, :K].cpu().numpy(), qw)
    assert np.all(qi[:, K:].cpu().numpy() == 7)
    assert np.array_equal(si.cpu().numpy()[:, 0].view(np.uint32), sw.view(np.uint32))


@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
def test_mx_3d_activation_layouts(gpu_lib, layout):
    G, M, K = 3, 19, 512
    shape = (M, G, K) if layout == "m_major" else (G, M, K)
    x = activations(shape, seed=9, dist="t", row_scale_log2=(-30, 30))
    xd, xv = device_input(x, "bf16")
    q, s = gpu_lib.bsmm_quant_fp8_mx(xd)
    torch.cuda.synchronize()
    assert tuple(q.shape) == shape and tuple(s.shape) == shape[:2] + (K // 128,)
    qw, sw = Q.quant_fp8_mx(xv.reshape(-1, K))
    assert np.array_equal(q.view(torch.uint8).cpu().numpy().reshape(-1, K), qw)
    assert np.array_equal(s.cpu().numpy().reshape(-1, K // 128), sw)


@pytest.mark.parametrize("M,K", [(37, 96), (5, 224), (130, 32)])
def test_mx32_quant_short_rows(gpu_lib, M, K):
    """K a multiple of 32 but not of 128; ragged block counts per workgroup."""
    x = activations((M, K), seed=K, dist="t", row_scale_log2=(-20, 20))
    xd, xv = device_input(x, "bf16")
    assert_same("mx32", run(gpu_lib, "mx32", xd), oracle("mx32", xv), f" {M}x{K}")


def test_mx32_quantise_then_matmul(gpu_lib):
    """bf16 activations and weights quantised on the GPU feed the MX matmul;
    the oracle quantises the same bf16 values itself and multiplies."""
    from oracle import scaled_mm as S
    from oracle.formats import bf16_bits_to_f64
    M, N, K = 200, 384, 1024
    xd, xv = device_input(activations((M, K), seed=1), "bf16")
    wd, wv = device_input(activations((N, K), seed=2, dist="t"), "bf16")
    qx, sx = gpu_lib.bsmm_quant_fp8_mx(xd, block=32)
    qw, sw = gpu_lib.bsmm_quant_fp8_mx(wd, block=32)
    y = gpu_lib.bsmm_fp8_mx32_mm(qx, qw.t(), sx, sw, out_dtype="bf16")
    torch.cuda.synchronize()
    got = bf16_bits_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16))
    ax, ex = Q.quant_fp8_mx(xv, block=32)
    aw, ew = Q.quant_fp8_mx(wv, block=32)
    rep = S.compare(got, S.fp8_mx32_mm(ax, aw.T, ex, ew, "bf16"))
    assert rep["ok"], rep


def test_degenerate_sizes(gpu_lib):
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = gpu_lib.bsmm_quant_fp8_blockwise(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)
    x = torch.zeros((5, 0), dtype=torch.float32, device="cuda")
    q, s = gpu_lib.bsmm_quant_int8_rowwise(x)
    torch.cuda.synchronize()
    assert q.shape == (5, 0) and np.all(s.cpu().numpy() == 1.0)   # an empty row: scale 1
    q, s = gpu_lib.bsmm_quant_fp8_mx(torch.zeros((4, 2, 0), device="cuda"))
    assert q.shape == (4, 2, 0) and s.shape == (4, 2, 0)
    with pytest.raises(gpu_lib.BsmmError):
        gpu_lib.bsmm_quant_fp8_mx(torch.zeros((4, 200), device="cuda"))


# ------------------------------------------------ workload sizes, sampled rows --

WORKLOADS = {
    "mx32_a_16640x8192": ("mx32", (16640, 8192), "normal", 3),
    # the activations of the matmul workloads, bf16 as a model holds them
    "int8_x_8192x4096": ("int8", (8192, 4096), "normal", 2),
    "fp8_a_16640x8192": ("fp8", (16640, 8192), "normal", 3),
    "mx_x_8192x8x4096": ("mx", (8192, 8, 4096), "normal", 43),
    "mx_x_2x9000x7168": ("mx", (2, 9000, 7168), "t", 5),
}


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_size_sampled_rows(gpu_lib, name):
    kind, shape, dist, seed = WORKLOADS[name]
    x = activations(shape, seed=seed, dist=dist)
    xd, xv = device_input(x, "bf16")
    del x
    q, s = run(gpu_lib, kind, xd)
    K = shape[-1]
    rows_x = xv.reshape(-1, K)
    q = q.reshape(-1, K)
    s = s.reshape(rows_x.shape[0], -1)
    R = rows_x.shape[0]
    pick = np.unique(np.concatenate([[0, R - 1], np.random.default_rng(seed).choice(R, 96)]))
    want = oracle(kind, rows_x[pick])
    assert_same(kind, (q[pick], s[pick]), want, f" {name} sampled rows")
    # every row / block: a positive scale, and its amax lands on the top code
    if kind == "int8":
        assert np.all(s > 0) and np.all(np.abs(q.astype(np.int16)).max(axis=1) == 127)
    else:
        bl = 32 if kind == "mx32" else 128
        top = (q.reshape(R, K // bl, bl) & 0x7F).max(axis=2)
        if kind == "fp8":
            assert np.all(top == 0x7E)
        else:   # amax * 2**-e lies in (224, 448]: codes 0x76 (224) to 0x7E (448)
            assert np.all((top >= 0x76) & (top <= 0x7E))
