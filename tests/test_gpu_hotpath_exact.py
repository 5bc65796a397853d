"""Exactness, scale-placement, range and guard-band parity of the two fp8
hot-path entry points, bsmm_fp8_blockwise and bsmm_fp8_mx_bmm (both
layouts), through every kernel path: each tile variant, packed scales, the
wide-wave kernel, forced split-K, stream-K at several grid sizes (more
workgroups than the device holds at once included) and the skinny kernel.

* Inputs whose sums are exact in binary32 (codes of the integers 1..8 with
  random signs, power-of-two scales) must match the oracle bit for bit.
* One (row, K block) of scale_a / x_scale and one (K block, column block) of
  scale_b / w_scale carry 2**20 and 2**-20: only the products of that block
  may grow, so a scale applied to a wrong row, column block or K block shows
  far outside the bound.
* Codes over the whole E4M3 range (+-448 and the subnormals), fp32 scales
  spanning 2**+-12 per block, scales near the ends of the binary32 range
  whose products stay normal, and e8m0 bytes from 0 to 254 (paired so that
  the scaled values stay inside the binary32 range).
* All-zero blocks, rows and columns: the result must be exactly 0 there.
* Outputs written through strided views inside sentinel buffers, ragged M.

Every fp8 result is held to the spec bar (relative Frobenius error
<= 1e-2 and |Y - C| <= 2**-7 Bd) and to the tighter bound of the kernels'
binary32 accumulation (``gamma_fp32``): |Y32 - C| <= gamma Bd, the bf16
output the rounding of such a value.
"""

import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsmm
from oracle import scaled_mm as S
from tests.gpu_util import DEV, Forced, as_f64, check_within, dev, host_out, say

pytestmark = pytest.mark.gpu

TILE_VARIANTS = ["t256x256", "t256x128", "t128x256", "t128x128", "t64x256", "t64x128",
                 "t256x256p", "t256x128p", "t128x256p", "w256x256", "w256x256p",
                 "t256x256sk", "t256x128sk", "t128x128sk", "t256x256skp"]
INTS = np.array([0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)   # 1..8


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield
    bsmm.bsmm_set_override(None, 0)
    bsmm.bsmm_set_streamk_grid(0)


def _int_codes(rng, shape):
    return INTS[rng.integers(0, 8, shape)] | (rng.integers(0, 2, shape) << 7).astype(np.uint8)


def _any_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E          # no NaN codes; +-448 twice as likely
    return c


def _pow2_scales(rng, shape, lo, hi):
    return np.exp2(rng.integers(lo, hi + 1, shape)).astype(np.float32)


def _wide_scales(rng, shape, lo, hi):
    return (rng.uniform(0.5, 1.0, shape) * np.exp2(rng.integers(lo, hi + 1, shape))) \
        .astype(np.float32)


# ------------------------------------------------------------- blockwise --

def bw_problem(M, N, K, seed, codes="int", scales=(-1, 1), sb_scales=None):
    rng = np.random.default_rng(seed)
    KB, NB = K // 128, N // 128
    mk = _int_codes if codes == "int" else _any_codes
    p = dict(a=mk(rng, (M, K)), b_nk=mk(rng, (N, K)))
    lo, hi = scales
    slo, shi = sb_scales or scales
    if codes == "int":
        p["scale_a"] = _pow2_scales(rng, (M, KB), lo, hi)
        p["scale_b"] = _pow2_scales(rng, (KB, NB), slo, shi)
    else:
        p["scale_a"] = _wide_scales(rng, (M, KB), lo, hi)
        p["scale_b"] = _wide_scales(rng, (KB, NB), slo, shi)
    return p


def bw_run(p, out_dtype, out=None, workspace=None):
    return bsmm.bsmm_fp8_blockwise(dev(p["a"]), dev(p["b_nk"]).t(), dev(p["scale_a"]),
                                   dev(p["scale_b"]), out_dtype=out_dtype, out=out,
                                   workspace=workspace)


def bw_oracle(p, out_dtype, rows=None):
    return S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], out_dtype,
                           rows=rows)


def bw_check(p, out_dtype, y, exact=False, rows=None):
    got = host_out(y)
    if rows is not None:
        got = got[rows]
    res = bw_oracle(p, out_dtype, rows)
    if exact:
        rep = S.compare(got, res, exact=True)
        assert rep["ok"], rep
        return rep
    rep = S.compare(as_f64(got), res)
    assert rep["ok"], rep
    return check_within(got, res, p["a"].shape[1] // 128)


@pytest.mark.parametrize("variant", TILE_VARIANTS)
def test_blockwise_bit_exact_every_variant(variant):
    p = bw_problem(300, 384, 1024, 11)
    for dt in ("f32", "bf16"):
        say(f"blockwise exact {variant} {dt} 300x384x1024")
        with Forced(variant, 1):
            y = bw_run(p, dt)
        bw_check(p, dt, y, exact=True)


@pytest.mark.parametrize("variant,split", [("t128x256", 2), ("t128x128", 3), ("t64x128", 8),
                                           ("t256x256p", 5), ("t256x128p", 4)])
def test_blockwise_bit_exact_split_k(variant, split):
    p = bw_problem(300, 384, 1024, 12)
    say(f"blockwise exact {variant} split {split}")
    with Forced(variant, split):
        y = bw_run(p, "bf16")
    bw_check(p, "bf16", y, exact=True)


@pytest.mark.parametrize("M", [1, 7, 16])
def test_blockwise_bit_exact_skinny(M):
    p = bw_problem(M, 384, 1408, 13 + M)
    say(f"blockwise exact skinny M={M}")
    assert bsmm.bsmm_query_plan(bsmm.OP_FP8_BLOCKWISE, 1, M, 384, 1408, "f32")["variant"] \
        == "s16x16"
    bw_check(p, "f32", bw_run(p, "f32"), exact=True)


@pytest.mark.parametrize("grid", [0, 3, 7, 40, 2048])
def test_blockwise_streamk_grids(grid):
    """The stream-K kernel at grids of 3, 7 and 40 workgroups (tiles cut at
    different K offsets) and 2048, more than the device holds at once: the
    fix-up of a split tile is done by whichever segment finishes last, so
    no workgroup waits for one that has not started."""
    M, N, K = 1024, 1024, 4096
    p = bw_problem(M, N, K, 14)
    ws = torch.empty(2048 * 2 * (256 * 256 * 4 + 8), dtype=torch.uint8, device=DEV)
    say(f"blockwise exact stream-K grid {grid} {M}x{N}x{K}")
    bsmm.bsmm_set_streamk_grid(grid)
    with Forced("t256x256sk", 0):
        y = bw_run(p, "f32", workspace=ws)
        y2 = bw_run(p, "f32", workspace=ws)
    rows = np.r_[0:40, 500:540, 980:1024]
    bw_check(p, "f32", y, exact=True, rows=rows)
    assert np.array_equal(host_out(y).view(np.uint32), host_out(y2).view(np.uint32))


@pytest.mark.parametrize("variant,split", [(None, 0), ("t256x256p", 1), ("t128x128", 3),
                                           ("t256x256skp", 0), ("w256x256p", 1),
                                           ("t64x256", 2)])
def test_blockwise_scales_land_on_their_own_blocks(variant, split):
    """One (row, K block) of scale_a times 2**20 and one (K block, column
    block) of scale_b times 2**-20, at corners and in the middle."""
    M, N, K = 520, 640, 1280
    base = bw_problem(M, N, K, 15, codes="any", scales=(-1, 1))
    for m, kb, nb, kb2 in ((0, 0, 0, 0), (519, 9, 4, 9), (263, 4, 2, 7), (64, 1, 3, 5)):
        p = dict(base, scale_a=base["scale_a"].copy(), scale_b=base["scale_b"].copy())
        p["scale_a"][m, kb] *= np.float32(2.0**20)
        p["scale_b"][kb2, nb] *= np.float32(2.0**-20)
        say(f"blockwise own block {variant} split {split} row {m} kb {kb} / kb {kb2} nb {nb}")
        with Forced(variant, split):
            y = bw_run(p, "f32")
        bw_check(p, "f32", y)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant", [None, "t256x256", "t128x128", "t256x256skp", "w256x256p"])
def test_blockwise_full_code_range_wide_scales(variant, out_dtype):
    p = bw_problem(300, 512, 1536, 16, codes="any", scales=(-12, 12))
    say(f"blockwise full range {variant} {out_dtype}")
    with Forced(variant, 0):
        y = bw_run(p, out_dtype)
    bw_check(p, out_dtype, y)


def test_blockwise_scales_near_the_ends_of_binary32():
    """scale_a near 2**-125 .. 2**-100 with scale_b near 2**100 .. 2**120 (and
    the reverse): every scale product is normal, so the kernels' binary32
    product sa * sb is exact to 2**-24 and the bound holds."""
    for lo, hi, slo, shi in ((-125, -100, 100, 120), (100, 120, -125, -100)):
        p = bw_problem(130, 256, 1024, 17, codes="any", scales=(lo, hi), sb_scales=(slo, shi))
        for variant in (None, "t128x128", "t256x256p"):
            say(f"blockwise extreme scales {lo}..{hi} x {slo}..{shi} {variant}")
            with Forced(variant, 0):
                y = bw_run(p, "f32")
            bw_check(p, "f32", y)


@pytest.mark.parametrize("variant,split", [(None, 0), ("t256x256p", 1), ("t128x256", 3),
                                           ("t256x256sk", 0), ("s16x16", 0)])
def test_blockwise_zero_blocks_give_exact_zeros(variant, split):
    M = 16 if variant == "s16x16" else 300
    rng = np.random.default_rng(18)
    p = bw_problem(M, 384, 1024, 18, codes="any", scales=(-4, 4))
    a, b = p["a"], p["b_nk"]
    a[3, :] = 0                                   # a zero row
    b[130, :] = 0                                 # a zero column
    for _ in range(20):                           # zero (row, K block) blocks
        a[rng.integers(0, M), 128 * rng.integers(0, 8) + np.arange(128)] = 0
    b[0:128, 256:384] = 0                         # a zero 128 x 128 block of B
    a[M - 1, 0:128] = 0x80                        # negative zeros
    a[M - 1, 128:] = 0
    say(f"blockwise zero blocks {variant} split {split}")
    with Forced(variant, split):
        y = bw_run(p, "f32")
    res = bw_oracle(p, "f32")
    got = host_out(y)
    assert (got[3] == 0).all() and (got[:, 130] == 0).all() and (got[M - 1] == 0).all()
    assert (got[res.bound == 0] == 0).all()
    bw_check(p, "f32", y)


@pytest.mark.parametrize("variant,split", [(None, 0), ("t256x256p", 2), ("t256x256sk", 0),
                                           ("t64x128", 1)])
def test_blockwise_guard_bands_ragged(variant, split):
    """Outputs written through strided views of a sentinel-filled buffer, at a
    16-byte-aligned column offset (vector stores) and a 4-byte one (scalar
    stores); nothing outside the view changes."""
    M, N, K = 300, 384, 768
    p = bw_problem(M, N, K, 19, codes="any", scales=(-3, 3))
    for dt, c0 in (("f32", 4), ("bf16", 8), ("f32", 1), ("bf16", 2)):
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        big = torch.full((M + 7, N + 20), -3.25, dtype=tdt, device=DEV)
        view = big[5:5 + M, c0:c0 + N]
        say(f"blockwise guard band {variant} split {split} {dt} column offset {c0}")
        with Forced(variant, split):
            bw_run(p, dt, out=view)
        h = host_out(big)
        mask = np.ones(h.shape, bool)
        mask[5:5 + M, c0:c0 + N] = False
        sentinel = host_out(torch.full((1,), -3.25, dtype=tdt, device=DEV))[0]
        assert (h[mask] == sentinel).all()
        bw_check(p, dt, view)


def test_blockwise_guard_bands_bulk_and_split_tail():
    """A call whose plan is a packed bulk launch over whole rounds plus a
    ragged split-K tail launch, written into a strided view."""
    M, N, K = 16534, 1024, 2048
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_BLOCKWISE, 1, M, N, K, "bf16")
    assert plan["m_split"] and plan["tail_split_k"] > 1, plan
    p = bw_problem(M, N, K, 20, codes="any", scales=(-6, 6))
    big = torch.full((M + 3, N + 64), 5.5, dtype=torch.bfloat16, device=DEV)
    view = big[1:1 + M, 32:32 + N]
    say("blockwise guard band bulk + split tail")
    bw_run(p, "bf16", out=view)
    h = host_out(big)
    mask = np.ones(h.shape, bool)
    mask[1:1 + M, 32:32 + N] = False
    sentinel = host_out(torch.full((1,), 5.5, dtype=torch.bfloat16, device=DEV))[0]
    assert (h[mask] == sentinel).all()
    rows = np.r_[0:8, 16376:16392, M - 150:M]
    bw_check(p, "bf16", view, rows=rows)


# -------------------------------------------------------------------- mx --

def mx_problem(G, M, N, K, seed, layout, codes="int", xs=(126, 128), ws=(126, 128)):
    rng = np.random.default_rng(seed)
    KB, NB = K // 128, N // 128
    mk = _int_codes if codes == "int" else _any_codes
    xshape = (M, G, K) if layout == "m_major" else (G, M, K)
    sshape = (M, G, KB) if layout == "m_major" else (G, M, KB)
    return dict(x=mk(rng, xshape), w=mk(rng, (G, N, K)),
                x_scale=rng.integers(xs[0], xs[1] + 1, sshape).astype(np.uint8),
                w_scale=rng.integers(ws[0], ws[1] + 1, (G, NB, KB)).astype(np.uint8),
                layout=layout)


def mx_run(p, out_dtype, out=None, workspace=None):
    return bsmm.bsmm_fp8_mx_bmm(dev(p["x"]), dev(p["w"]), dev(p["x_scale"]), dev(p["w_scale"]),
                                layout=p["layout"], out_dtype=out_dtype, out=out,
                                workspace=workspace)


def mx_check(p, out_dtype, y, exact=False, rows=None):
    res = S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], p["layout"], out_dtype,
                       rows=rows)
    got = host_out(y)
    if rows is not None:
        got = got[rows] if p["layout"] == "m_major" else got[:, rows]
    if exact:
        rep = S.compare(got, res, exact=True)
        assert rep["ok"], rep
        return rep
    rep = S.compare(as_f64(got), res)
    assert rep["ok"], rep
    return check_within(got, res, p["x"].shape[2] // 128)


@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
@pytest.mark.parametrize("variant", TILE_VARIANTS)
def test_mx_bit_exact_every_variant(variant, layout):
    p = mx_problem(3, 300, 384, 1024, 31, layout)
    for dt in ("f32", "bf16"):
        say(f"mx exact {variant} {layout} {dt} G=3 M=300 N=384 K=1024")
        with Forced(variant, 1):
            y = mx_run(p, dt)
        mx_check(p, dt, y, exact=True)


@pytest.mark.parametrize("variant,split", [("t64x256", 4), ("t128x128", 3), ("t256x128p", 2),
                                           ("t256x256p", 8)])
def test_mx_bit_exact_split_k(variant, split):
    p = mx_problem(2, 200, 256, 1024, 32, "batch_first")
    say(f"mx exact {variant} split {split}")
    with Forced(variant, split):
        y = mx_run(p, "f32")
    mx_check(p, "f32", y, exact=True)


@pytest.mark.parametrize("M", [1, 9, 16])
def test_mx_bit_exact_skinny(M):
    for layout in ("m_major", "batch_first"):
        p = mx_problem(8, M, 1024, 1280, 33 + M, layout)
        say(f"mx exact skinny M={M} {layout}")
        mx_check(p, "bf16", mx_run(p, "bf16"), exact=True)


@pytest.mark.parametrize("grid", [0, 5, 64, 1024])
def test_mx_streamk_grids(grid):
    G, M, N, K = 4, 1024, 512, 2048
    p = mx_problem(G, M, N, K, 34, "batch_first")
    ws = torch.empty(1024 * 2 * (256 * 256 * 4 + 8), dtype=torch.uint8, device=DEV)
    say(f"mx exact stream-K grid {grid}")
    bsmm.bsmm_set_streamk_grid(grid)
    with Forced("t256x256skp", 0):
        y = mx_run(p, "bf16", workspace=ws)
    mx_check(p, "bf16", y, exact=True)


@pytest.mark.parametrize("variant,split", [(None, 0), ("t256x256p", 1), ("t128x128", 2),
                                           ("t256x256skp", 0), ("w256x256p", 1),
                                           ("s16x16", 0)])
@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
def test_mx_scales_land_on_their_own_blocks(variant, split, layout):
    """x_scale of one (batch, row, K block) raised by 20 (times 2**20) and
    w_scale of one (batch, column block, K block) lowered by 20."""
    G, M, N, K = 3, 16 if variant == "s16x16" else 300, 512, 1280
    base = mx_problem(G, M, N, K, 35, layout, codes="any", xs=(120, 134), ws=(120, 134))
    for g, m, kb, nb, kb2 in ((0, 0, 0, 0, 0), (2, M - 1, 9, 3, 9), (1, M // 2, 4, 2, 6)):
        p = dict(base, x_scale=base["x_scale"].copy(), w_scale=base["w_scale"].copy())
        if layout == "m_major":
            p["x_scale"][m, g, kb] += 20
        else:
            p["x_scale"][g, m, kb] += 20
        p["w_scale"][g, nb, kb2] -= 20
        say(f"mx own block {variant} split {split} {layout} g {g} row {m} kb {kb} nb {nb}")
        with Forced(variant, split):
            y = mx_run(p, "f32")
        mx_check(p, "f32", y)


@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
@pytest.mark.parametrize("xs,ws", [((60, 190), (97, 157)), ((97, 157), (60, 190)),
                                   ((0, 12), (242, 254)), ((242, 254), (0, 12))])
def test_mx_full_code_range_wide_e8m0(layout, xs, ws):
    """Codes over the whole E4M3 range and e8m0 bytes across 0..254, paired
    so that every scaled product and sum stays in the binary32 normal range
    (the scale product 2**(bx + bw - 254) within 2**+-97)."""
    p = mx_problem(2, 200, 384, 1280, 36, layout, codes="any", xs=xs, ws=ws)
    for variant in (None, "t128x128", "t256x256p", "s16x16"):
        q = p
        if variant == "s16x16":
            q = dict(p, x=p["x"][:16] if layout == "m_major" else p["x"][:, :16],
                     x_scale=p["x_scale"][:16] if layout == "m_major" else p["x_scale"][:, :16])
        say(f"mx wide e8m0 {layout} x {xs} w {ws} {variant}")
        with Forced(variant, 0):
            y = mx_run(q, "f32")
        mx_check(q, "f32", y)


@pytest.mark.parametrize("variant", [None, "t256x256p", "t64x128", "t256x256sk", "s16x16"])
def test_mx_zero_blocks_give_exact_zeros(variant):
    G, M, N, K = 2, 16 if variant == "s16x16" else 200, 384, 1024
    rng = np.random.default_rng(37)
    p = mx_problem(G, M, N, K, 37, "batch_first", codes="any", xs=(118, 136), ws=(118, 136))
    x, w = p["x"], p["w"]
    x[1, 3, :] = 0
    w[0, 200, :] = 0
    w[1, 0:128, 384:512] = 0
    for _ in range(20):
        x[rng.integers(0, G), rng.integers(0, M), 128 * rng.integers(0, 8) + np.arange(128)] = 0
    say(f"mx zero blocks {variant}")
    with Forced(variant, 0):
        y = mx_run(p, "bf16")
    res = S.fp8_mx_bmm(x, w, p["x_scale"], p["w_scale"], "batch_first", "bf16")
    got = host_out(y)
    assert (got[1, 3] & 0x7FFF == 0).all() and (got[0, :, 200] & 0x7FFF == 0).all()
    assert (got[res.bound == 0] & 0x7FFF == 0).all()
    mx_check(p, "bf16", y)


@pytest.mark.parametrize("variant,split", [(None, 0), ("t256x256p", 3), ("t256x256skp", 0),
                                           ("t64x256", 1), ("s16x16", 0)])
@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
def test_mx_guard_bands_ragged(variant, split, layout):
    """A ragged-M BMM written through strided views of a sentinel-filled
    buffer with a spare batch and spare rows and columns on every side, at a
    vector-aligned and an unaligned column offset."""
    G, M, N, K = 2, 9 if variant == "s16x16" else 300, 384, 768
    p = mx_problem(G, M, N, K, 38, layout, codes="any", xs=(122, 132), ws=(122, 132))
    for dt, c0 in (("f32", 4), ("bf16", 8), ("f32", 3), ("bf16", 2)):
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        if layout == "m_major":
            big = torch.full((M + 5, G + 1, N + 16), -7.0, dtype=tdt, device=DEV)
            view = big[2:2 + M, 1:1 + G, c0:c0 + N]
            sel = (slice(2, 2 + M), slice(1, 1 + G), slice(c0, c0 + N))
        else:
            big = torch.full((G + 1, M + 5, N + 16), -7.0, dtype=tdt, device=DEV)
            view = big[1:1 + G, 2:2 + M, c0:c0 + N]
            sel = (slice(1, 1 + G), slice(2, 2 + M), slice(c0, c0 + N))
        say(f"mx guard band {variant} split {split} {layout} {dt} column offset {c0}")
        with Forced(variant, split):
            mx_run(p, dt, out=view)
        h = host_out(big)
        mask = np.ones(h.shape, bool)
        mask[sel] = False
        sentinel = host_out(torch.full((1,), -7.0, dtype=tdt, device=DEV))[0]
        assert (h[mask] == sentinel).all()
        mx_check(p, dt, view)


def test_mx_batch_first_tail_guard_band_default_plan():
    """The c5 plan shape at reduced K: bulk launch over whole rounds plus a
    split-K tail of ragged rows, into a strided view."""
    G, M, N, K = 2, 9000, 2048, 1024
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX_BMM, G, M, N, K, "f32")
    say(f"mx batch-first tail plan {plan}")
    p = mx_problem(G, M, N, K, 39, "batch_first", codes="any", xs=(120, 134), ws=(120, 134))
    big = torch.full((G + 1, M + 40, N + 8), 9.0, dtype=torch.float32, device=DEV)
    view = big[0:G, 24:24 + M, 4:4 + N]
    mx_run(p, "f32", out=view)
    h = host_out(big)
    mask = np.ones(h.shape, bool)
    mask[0:G, 24:24 + M, 4:4 + N] = False
    assert (h[mask] == 9.0).all()
    rows = np.r_[0:4, 8185:8200, 8950:M]
    mx_check(p, "f32", view, rows=rows)


# ------------------------------------- own-block tests on M-split plans --

def test_blockwise_scales_land_on_their_own_blocks_bulk_and_split_tail():
    """The default plan of a call with a whole-rounds bulk launch and a
    split-K tail launch (both reading one packed copy of scale_a): a scale
    raised by 2**20 in the last bulk row, the first tail row and the last
    row, and one lowered by 2**-20 in several column blocks."""
    M, N, K = 16534, 1024, 2048
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_BLOCKWISE, 1, M, N, K, "f32")
    assert plan["m_split"] == 16384 and plan["tail_split_k"] > 1, plan
    base = bw_problem(M, N, K, 21, codes="any", scales=(-1, 1))
    for m, kb, nb, kb2 in ((16383, 3, 2, 3), (16384, 15, 7, 15), (M - 1, 0, 0, 8), (100, 7, 4, 2)):
        p = dict(base, scale_a=base["scale_a"].copy(), scale_b=base["scale_b"].copy())
        p["scale_a"][m, kb] *= np.float32(2.0**20)
        p["scale_b"][kb2, nb] *= np.float32(2.0**-20)
        say(f"blockwise own block, bulk + split tail: row {m} kb {kb} / kb {kb2} nb {nb}")
        y = bw_run(p, "f32")
        rows = np.array(sorted({0, m - 1, m, min(m + 1, M - 1), 16383, 16384, M - 1}))
        bw_check(p, "f32", y, rows=rows)


def test_mx_scales_land_on_their_own_blocks_bulk_and_split_tail():
    """The same for the mx BMM, batch-first, with the tail in both batches."""
    G, M, N, K = 2, 9000, 2048, 1024
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX_BMM, G, M, N, K, "f32")
    say(f"mx own block plan {plan}")
    base = mx_problem(G, M, N, K, 40, "batch_first", codes="any", xs=(120, 134), ws=(120, 134))
    for g, m, kb, nb, kb2 in ((0, 8191, 2, 3, 2), (1, 8192, 7, 15, 7), (1, M - 1, 0, 0, 5)):
        p = dict(base, x_scale=base["x_scale"].copy(), w_scale=base["w_scale"].copy())
        p["x_scale"][g, m, kb] += 20
        p["w_scale"][g, nb, kb2] -= 20
        say(f"mx own block, bulk + tail: g {g} row {m} kb {kb} / nb {nb} kb {kb2}")
        y = mx_run(p, "f32")
        rows = np.array(sorted({0, m - 1, m, min(m + 1, M - 1), 8191, 8192, M - 1}))
        mx_check(p, "f32", y, rows=rows)


# --------------------------------------------- the narrow kernel (M <= 128) --

NARROW_MS = [17, 100, 128]


@pytest.mark.parametrize("K", [384, 1280, 1408])
@pytest.mark.parametrize("M", NARROW_MS)
def test_narrow_mx_bit_exact(M, K):
    """The M <= 128 kernel: K from fewer blocks than its ring holds (3) to
    odd and even counts beyond it, both layouts, three batches."""
    for layout in ("m_major", "batch_first"):
        p = mx_problem(3, M, 384, K, 51 + M + K, layout)
        for dt in ("f32", "bf16"):
            say(f"narrow mx exact {layout} {dt} G=3 M={M} N=384 K={K}")
            with Forced("n128x32", 0):
                y = mx_run(p, dt)
            mx_check(p, dt, y, exact=True)


@pytest.mark.parametrize("M", NARROW_MS)
def test_narrow_blockwise_and_int8_and_scaled_mm_bit_exact(M):
    p = bw_problem(M, 512, 1280, 52 + M)
    for dt in ("f32", "bf16"):
        say(f"narrow blockwise exact {dt} M={M}")
        with Forced("n128x32", 0):
            y = bw_run(p, dt)
        bw_check(p, dt, y, exact=True)
    from synth import int8_rowwise_inputs
    from tests.gpu_util import check_int8, run_int8
    q = int8_rowwise_inputs(M, 352, 1280, 53 + M)
    for dt in ("i32", "f32", "bf16"):
        say(f"narrow int8 {dt} M={M}")
        with Forced("n128x32", 0):
            y = run_int8(q, dt)
        check_int8(q, dt, y)
    from synth import fp8_scaled_mm_inputs
    t = fp8_scaled_mm_inputs(M, 224, 1024, 54 + M, bias="f32")
    say(f"narrow scaled_mm f32 M={M}")
    with Forced("n128x32", 0):
        y = bsmm.bsmm_fp8_scaled_mm(dev(t["a"]), dev(t["b_nk"]).t(), dev(t["scale_a"]),
                                    dev(t["scale_b"]), bias=dev(t["bias"]), scale_result=0.5,
                                    out_dtype="f32")
    ref = S.fp8_scaled_mm(t["a"], t["b_nk"].T, t["scale_a"], t["scale_b"], bias=t["bias"],
                          scale_result=0.5, out_dtype="f32")
    rep = S.compare(as_f64(host_out(y)), ref)
    assert rep["ok"], rep


def test_narrow_falls_back_where_it_does_not_apply():
    """More K blocks than its scale region holds (blockwise K = 5120, 40
    blocks), more than 128 rows, N not a multiple of 32 (int8): the call
    runs another kernel and stays exact."""
    cases = [bw_problem(64, 256, 5120, 55), bw_problem(200, 256, 512, 56)]
    for p in cases:
        say(f"narrow fallback blockwise {p['a'].shape}")
        with Forced("n128x32", 0):
            y = bw_run(p, "f32")
        bw_check(p, "f32", y, exact=True)
    from synth import int8_rowwise_inputs
    from tests.gpu_util import check_int8, run_int8
    q = int8_rowwise_inputs(60, 200, 512, 57)
    say("narrow fallback int8 N=200")
    with Forced("n128x32", 0):
        y = run_int8(q, "i32")
    check_int8(q, "i32", y)


@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
def test_narrow_scales_land_on_their_own_blocks(layout):
    G, M, N, K = 3, 128, 512, 1280
    base = mx_problem(G, M, N, K, 58, layout, codes="any", xs=(120, 134), ws=(120, 134))
    for g, m, kb, nb, kb2 in ((0, 0, 0, 0, 0), (2, 127, 9, 3, 9), (1, 77, 4, 2, 6)):
        p = dict(base, x_scale=base["x_scale"].copy(), w_scale=base["w_scale"].copy())
        if layout == "m_major":
            p["x_scale"][m, g, kb] += 20
        else:
            p["x_scale"][g, m, kb] += 20
        p["w_scale"][g, nb, kb2] -= 20
        say(f"narrow mx own block {layout} g {g} row {m} kb {kb} nb {nb}")
        with Forced("n128x32", 0):
            y = mx_run(p, "f32")
        mx_check(p, "f32", y)
    q = bw_problem(100, 384, 1024, 59, codes="any", scales=(-1, 1))
    q["scale_a"][99, 7] *= np.float32(2.0**20)
    q["scale_b"][3, 2] *= np.float32(2.0**-20)
    say("narrow blockwise own block")
    with Forced("n128x32", 0):
        y = bw_run(q, "f32")
    bw_check(q, "f32", y)


@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
def test_narrow_guard_bands_and_full_range(layout):
    G, M, N, K = 2, 90, 384, 1280
    p = mx_problem(G, M, N, K, 60, layout, codes="any", xs=(60, 190), ws=(97, 157))
    for dt, c0 in (("f32", 4), ("bf16", 8), ("f32", 3), ("bf16", 2)):
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        if layout == "m_major":
            big = torch.full((M + 5, G + 1, N + 16), -7.0, dtype=tdt, device=DEV)
            view = big[2:2 + M, 1:1 + G, c0:c0 + N]
            sel = (slice(2, 2 + M), slice(1, 1 + G), slice(c0, c0 + N))
        else:
            big = torch.full((G + 1, M + 5, N + 16), -7.0, dtype=tdt, device=DEV)
            view = big[1:1 + G, 2:2 + M, c0:c0 + N]
            sel = (slice(1, 1 + G), slice(2, 2 + M), slice(c0, c0 + N))
        say(f"narrow guard band {layout} {dt} column offset {c0}")
        with Forced("n128x32", 0):
            mx_run(p, dt, out=view)
        h = host_out(big)
        mask = np.ones(h.shape, bool)
        mask[sel] = False
        sentinel = host_out(torch.full((1,), -7.0, dtype=tdt, device=DEV))[0]
        assert (h[mask] == sentinel).all()
        mx_check(p, dt, view)


@pytest.mark.parametrize("KB", [33, 56, 100, 156])
def test_narrow_mx_many_k_blocks(KB):
    """Scale staging in several rounds (more than 32 K blocks), up to the
    most K blocks the scale region holds; one more falls back."""
    G, M, N, K = 2, 100, 128, KB * 128
    p = mx_problem(G, M, N, K, 61 + KB, "m_major")
    say(f"narrow mx exact G={G} M={M} N={N} K={K}")
    with Forced("n128x32", 0):
        y = mx_run(p, "f32")
    mx_check(p, "f32", y, exact=True)
    q = mx_problem(G, M, N, K, 62 + KB, "batch_first", codes="any", xs=(120, 134),
                   ws=(120, 134))
    for g, m, kb, nb, kb2 in ((0, 0, KB - 1, 0, KB - 1), (1, 99, KB // 2, 0, min(33, KB - 1)), (1, 31, 32, 0, 0)):
        r = dict(q, x_scale=q["x_scale"].copy(), w_scale=q["w_scale"].copy())
        r["x_scale"][g, m, kb] += 20
        r["w_scale"][g, nb, kb2] -= 20
        say(f"narrow mx own block K={K} g {g} row {m} kb {kb} / kb {kb2}")
        with Forced("n128x32", 0):
            y = mx_run(r, "f32")
        mx_check(r, "f32", y)


def test_narrow_blockwise_most_k_blocks_and_beyond():
    """Blockwise at 33 and 39 K blocks (two staging rounds; 39 is the most
    the scale region holds) and its own-block placement there."""
    for KB in (33, 39):
        p = bw_problem(70, 256, KB * 128, 63 + KB)
        say(f"narrow blockwise exact K={KB * 128}")
        with Forced("n128x32", 0):
            y = bw_run(p, "bf16")
        bw_check(p, "bf16", y, exact=True)
        q = bw_problem(70, 256, KB * 128, 64 + KB, codes="any", scales=(-1, 1))
        q["scale_a"][69, KB - 1] *= np.float32(2.0**20)
        q["scale_a"][3, 32] *= np.float32(2.0**20)
        q["scale_b"][KB - 2, 1] *= np.float32(2.0**-20)
        with Forced("n128x32", 0):
            y = bw_run(q, "f32")
        bw_check(q, "f32", y)


# ------------------------- the narrow kernel: 64 columns and split K --

NARROW_PLANS = [("n128x32", 2), ("n128x32", 3), ("n128x64", 1), ("n128x64", 2), ("n128x64", 5)]


@pytest.mark.parametrize("variant,split", NARROW_PLANS)
def test_narrow_split_mx_bit_exact(variant, split):
    """Both widths, K split into 1 to 5 ranges added in the kernel (10 K
    blocks: ranges of 2 to 5 blocks, the last one shorter), both layouts,
    three batches."""
    for layout in ("m_major", "batch_first"):
        p = mx_problem(3, 100, 384, 1280, 70 + split, layout)
        for dt in ("f32", "bf16"):
            say(f"narrow mx exact {variant} split {split} {layout} {dt}")
            with Forced(variant, split):
                plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX_BMM, 3, 100, 384, 1280, dt)
                assert plan["variant"] == variant and plan["split_k"] == split, plan
                y = mx_run(p, dt)
            mx_check(p, dt, y, exact=True)


@pytest.mark.parametrize("variant,split", [("n128x64", 1), ("n128x64", 3), ("n128x32", 4)])
def test_narrow_split_blockwise_int8_scaled_mm_bit_exact(variant, split):
    p = bw_problem(77, 512, 1280, 71 + split)
    for dt in ("f32", "bf16"):
        say(f"narrow blockwise exact {variant} split {split} {dt}")
        with Forced(variant, split):
            y = bw_run(p, dt)
        bw_check(p, dt, y, exact=True)
    from synth import fp8_scaled_mm_inputs, int8_rowwise_inputs
    from tests.gpu_util import check_int8, run_int8
    q = int8_rowwise_inputs(77, 320, 1280, 72 + split)
    for dt in ("i32", "bf16"):
        say(f"narrow int8 {variant} split {split} {dt}")
        with Forced(variant, split):
            y = run_int8(q, dt)
        check_int8(q, dt, y)
    t = fp8_scaled_mm_inputs(77, 192, 1024, 73 + split, bias="f32")
    say(f"narrow scaled_mm {variant} split {split}")
    with Forced(variant, split):
        y = bsmm.bsmm_fp8_scaled_mm(dev(t["a"]), dev(t["b_nk"]).t(), dev(t["scale_a"]),
                                    dev(t["scale_b"]), bias=dev(t["bias"]), scale_result=0.5,
                                    out_dtype="f32")
    want = S.fp8_scaled_mm(t["a"], t["b_nk"].T, t["scale_a"], t["scale_b"], bias=t["bias"],
                           scale_result=0.5, out_dtype="f32")
    rep = S.compare(as_f64(host_out(y)), want)
    assert rep["ok"], rep


def test_narrow_split_scales_land_on_their_own_blocks():
    """10 K blocks split into 3 ranges (4, 4 and 2 blocks): a raised scale
    at the first and last block of every range shows only in its own
    block."""
    G, M, N, K = 2, 128, 256, 1280
    base = mx_problem(G, M, N, K, 74, "m_major", codes="any", xs=(120, 134), ws=(120, 134))
    for kb in (0, 3, 4, 7, 8, 9):
        p = dict(base, x_scale=base["x_scale"].copy(), w_scale=base["w_scale"].copy())
        p["x_scale"][kb * 11 % M, kb % G, kb] += 20
        p["w_scale"][(kb + 1) % G, kb % 2, kb] -= 20
        say(f"narrow split own block kb {kb}")
        with Forced("n128x64", 3):
            y = mx_run(p, "f32")
        mx_check(p, "f32", y)
    q = bw_problem(90, 256, 1280, 75, codes="any", scales=(-1, 1))
    q["scale_a"][89, 3] *= np.float32(2.0**20)
    q["scale_b"][6, 1] *= np.float32(2.0**-20)
    with Forced("n128x64", 3):
        y = bw_run(q, "f32")
    bw_check(q, "f32", y)


def test_narrow_split_counters_across_calls_and_small_workspace():
    """Launches in a row share the workspace's counters (each launch tags
    its own); a workspace too small for the split runs unsplit."""
    ps = [mx_problem(2, 90, 256, 1280, 76 + i, "batch_first") for i in range(3)]
    with Forced("n128x64", 4):
        plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX_BMM, 2, 90, 256, 1280, "f32")
        assert plan["variant"] == "n128x64" and plan["split_k"] == 4, plan
        ws = torch.empty(plan["workspace"], dtype=torch.uint8, device=DEV)
        ys = [mx_run(p, "f32", workspace=ws) for p in ps]
    for p, y in zip(ps, ys):
        mx_check(p, "f32", y, exact=True)
    small = torch.empty(1024, dtype=torch.uint8, device=DEV)
    with Forced("n128x64", 4):
        plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX_BMM, 2, 90, 256, 1280, "f32",
                                    workspace_bytes=1024)
        y = mx_run(ps[0], "f32", workspace=small)
    assert plan["split_k"] == 1, plan
    mx_check(ps[0], "f32", y, exact=True)
