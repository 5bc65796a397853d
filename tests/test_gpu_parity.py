"""GPU parity of the HIP path against the CPU oracle, at sizes that span
several tiles with ragged M and N tails: every kernel variant, forced split-K,
both mx layouts, strided and broadcast scales, guard bands around the output,
degenerate sizes and run-to-run determinism.

Bars: int8 path bit-exact (int32 accumulators, and the fp32/bf16 outputs,
which are the same binary32 operations in the same order); fp8 paths within
relative Frobenius error 1e-2 and |Y - C| <= 2^-7 * sum_k |a_deq||b_deq|
elementwise (Y exactly 0 where that sum is 0).
"""

import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsmm
from oracle import scaled_mm as S
from synth import fp8_blockwise_inputs, fp8_mx_bmm_inputs, int8_rowwise_inputs
from tests.gpu_util import (DEV, Forced, as_f64, check_blockwise, check_int8, check_mx,
                            dev, host_out, run_blockwise, run_int8, run_mx, say)

pytestmark = pytest.mark.gpu

VARIANTS = ["t256x256", "t256x128", "t128x256", "t128x128", "t64x256", "t64x128",
            "t256x256p", "t256x128p", "t128x256p", "w256x256", "w256x256p",
            "t256x256sk", "t256x128sk", "t128x128sk", "t256x256skp"]
SK_VARIANTS = ["t256x256sk", "t256x128sk", "t128x128sk", "t256x256skp"]
PACKED_VARIANTS = ["t256x256p", "t256x128p", "t128x256p", "t256x256skp", "w256x256p"]


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


# ------------------------------------------------------------------ int8 ----

@pytest.mark.parametrize("variant", VARIANTS)
def test_int8_variants_exact(variant):
    p = int8_rowwise_inputs(300, 384, 512, 101)
    for dt in ("i32", "f32", "bf16"):
        say(f"int8 {variant} {dt} M=300 N=384 K=512")
        with Forced(variant, 1):
            y = run_int8(p, dt)
        check_int8(p, dt, y)


def test_int8_tiny_workload_exact():
    """64x256 @ 256x128, codes uniform in [-127,127], scales in [1e-3,1e-2]:
    int32 accumulators bit-exact and the fp32 output bit-exact."""
    p = int8_rowwise_inputs(64, 128, 256, 1)
    say("int8 tiny i32 + f32")
    check_int8(p, "i32", run_int8(p, "i32"))
    check_int8(p, "f32", run_int8(p, "f32"))


@pytest.mark.parametrize("split", [2, 3, 4])
def test_int8_splitk_bit_identical(split):
    p = int8_rowwise_inputs(200, 256, 1024, 102)
    say(f"int8 split {split}")
    with Forced("t128x128", split):
        y = run_int8(p, "i32")
        yb = run_int8(p, "bf16")
    check_int8(p, "i32", y)
    check_int8(p, "bf16", yb)


def test_int8_tensorwise_and_extreme_values():
    """All codes at +-127 (largest accumulators) and tensorwise (0-d) scales."""
    M, N, K = 130, 160, 4096
    rng = np.random.default_rng(7)
    a = np.where(rng.random((M, K)) < 0.5, -127, 127).astype(np.int8)
    b = np.where(rng.random((N, K)) < 0.5, -127, 127).astype(np.int8)
    a[0, :] = 127
    b[0, :] = 127                                  # acc[0,0] = K * 127^2
    sa = np.float32(3e-3)
    sb = np.float32(7e-4)
    say("int8 tensorwise extreme")
    y = bsmm.bsmm_int8_rowwise(dev(a), dev(b).t(), torch.tensor(sa, device=DEV),
                               torch.tensor(sb, device=DEV), out_dtype="f32")
    yi = bsmm.bsmm_int8_rowwise(dev(a), dev(b).t(), out_dtype="i32")
    ref = S.int8_rowwise(a, b.T, np.full(M, sa), np.full(N, sb), "f32")
    assert S.compare(host_out(y), ref, exact=True)["ok"]
    refi = S.int8_rowwise(a, b.T, out_dtype="i32")
    assert S.compare(host_out(yi), refi, exact=True)["ok"]
    assert host_out(yi)[0, 0] == K * 127 * 127


def test_int8_guard_bands():
    """Output written through a strided view inside a sentinel-filled buffer:
    nothing outside [M, N] changes."""
    p = int8_rowwise_inputs(75, 200, 256, 103)
    big = torch.full((75 + 9, 256), -12345, dtype=torch.int32, device=DEV)
    view = big[3:78, 16:216]
    say("int8 guard bands")
    run_int8(p, "i32", out=view)
    h = host_out(big)
    check_int8(p, "i32", view)
    mask = np.ones_like(h, dtype=bool)
    mask[3:78, 16:216] = False
    assert (h[mask] == -12345).all()


# ------------------------------------------------------------ fp8 blockwise --

@pytest.mark.parametrize("variant", VARIANTS)
def test_blockwise_variants(variant):
    p = fp8_blockwise_inputs(300, 384, 640, 201)
    for dt in ("bf16", "f32"):
        say(f"blockwise {variant} {dt} M=300 N=384 K=640")
        with Forced(variant, 1):
            y = run_blockwise(p, dt)
        check_blockwise(p, dt, y)


@pytest.mark.parametrize("split", [2, 5])
def test_blockwise_splitk(split):
    p = fp8_blockwise_inputs(160, 256, 1280, 202)
    say(f"blockwise split {split}")
    with Forced("t128x256", split):
        y = run_blockwise(p, "f32")
    check_blockwise(p, "f32", y)


def test_blockwise_scale_layouts():
    """Column-major scale_a (stride along M = 1) and broadcast (stride 0)
    scale_b give the same results as their dense equivalents."""
    p = fp8_blockwise_inputs(96, 256, 512, 203)
    a = dev(p["a"])
    b = dev(p["b_nk"]).t()
    sa_cm = dev(np.ascontiguousarray(p["scale_a"].T)).t()          # [M, KB], stride (1, M)
    sb_one = torch.full((1, 1), 0.03125, device=DEV).expand(4, 2)  # stride (0, 0)
    say("blockwise strided scales")
    y = bsmm.bsmm_fp8_blockwise(a, b, sa_cm, sb_one, out_dtype="f32")
    ref = S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"],
                          np.full((4, 2), 0.03125, np.float32), "f32")
    assert S.compare(as_f64(host_out(y)), ref)["ok"]


def test_blockwise_guard_bands_and_m1():
    p = fp8_blockwise_inputs(1, 256, 256, 204)
    big = torch.full((4, 512), 7.0, dtype=torch.float32, device=DEV)
    view = big[1:2, 128:384]
    say("blockwise M=1 guard bands")
    run_blockwise(p, "f32", out=view)
    check_blockwise(p, "f32", view)
    h = host_out(big)
    mask = np.ones_like(h, dtype=bool)
    mask[1, 128:384] = False
    assert (h[mask] == 7.0).all()


# -------------------------------------------------------------------- mx ----

@pytest.mark.parametrize("layout", ["m_major", "batch_first"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_mx_variants(variant, layout):
    p = fp8_mx_bmm_inputs(3, 300, 384, 512, 301, layout=layout)
    say(f"mx {variant} {layout} G=3 M=300 N=384 K=512")
    with Forced(variant, 1):
        y = run_mx(p, "bf16")
    check_mx(p, "bf16", y)


@pytest.mark.parametrize("split", [2, 4])
def test_mx_splitk(split):
    p = fp8_mx_bmm_inputs(2, 70, 256, 1024, 302, layout="batch_first", dist="t")
    say(f"mx split {split}")
    with Forced("t64x256", split):
        y = run_mx(p, "f32")
    check_mx(p, "f32", y)


def test_mx_layouts_agree():
    """The same logical problem in m-major and batch-first storage gives the
    same bits (identical kernels, identical per-element order)."""
    p = fp8_mx_bmm_inputs(4, 130, 256, 512, 303, layout="m_major")
    q = dict(p)
    q["layout"] = "batch_first"
    q["x"] = np.ascontiguousarray(p["x"].transpose(1, 0, 2))
    q["x_scale"] = np.ascontiguousarray(p["x_scale"].transpose(1, 0, 2))
    say("mx layouts agree")
    y1 = host_out(run_mx(p, "f32"))
    y2 = host_out(run_mx(q, "f32"))
    assert np.array_equal(y1.transpose(1, 0, 2).view(np.uint32), y2.view(np.uint32))


# --------------------------------------------------------------- edges ----

def test_degenerate_sizes():
    say("degenerate sizes")
    z = torch.empty((0, 256), dtype=torch.uint8, device=DEV)
    b = torch.empty((256, 256), dtype=torch.uint8, device=DEV)
    y = bsmm.bsmm_fp8_blockwise(z, b.t(), torch.empty((0, 2), device=DEV),
                                torch.ones((2, 2), device=DEV), out_dtype="f32")
    assert y.shape == (0, 256)
    # K = 0: an empty sum is zero
    a0 = torch.empty((5, 0), dtype=torch.int8, device=DEV)
    b0 = torch.empty((0, 7), dtype=torch.int8, device=DEV)
    out = torch.full((5, 7), 99, dtype=torch.int32, device=DEV)
    bsmm.bsmm_int8_rowwise(a0, b0, out_dtype="i32", out=out)
    assert (host_out(out) == 0).all()


def test_determinism():
    p = fp8_blockwise_inputs(256, 512, 1024, 401)
    say("determinism")
    ys = [host_out(run_blockwise(p, "f32")).view(np.uint32) for _ in range(3)]
    assert all(np.array_equal(ys[0], y) for y in ys[1:])
    with Forced("t64x128", 3):
        z1 = host_out(run_blockwise(p, "f32")).view(np.uint32)
        z2 = host_out(run_blockwise(p, "f32")).view(np.uint32)
    assert np.array_equal(z1, z2)


# ------------------------------------------------------------- stream-K ----

@pytest.mark.parametrize("variant", SK_VARIANTS)
def test_streamk_many_segments(variant):
    """Few tiles, many workgroups: every tile is cut into several K
    segments whose partials the owning workgroup adds in K order."""
    p = int8_rowwise_inputs(300, 384, 1280, 501)
    q = fp8_blockwise_inputs(300, 384, 1280, 502)
    r = fp8_mx_bmm_inputs(2, 200, 256, 1280, 503, layout="m_major")
    say(f"stream-K {variant} many segments")
    with Forced(variant, 0):
        yi = run_int8(p, "i32")
        yb = run_blockwise(q, "f32")
        ym = run_mx(r, "bf16")
    check_int8(p, "i32", yi)
    check_blockwise(q, "f32", yb)
    check_mx(r, "bf16", ym)


def test_streamk_small_workspace_two_way_splits():
    """A workspace that holds three workgroups' slots: three workgroups,
    tiles split in two.  Results match the oracle and repeat bit for bit."""
    q = fp8_blockwise_inputs(520, 512, 1280, 504)
    a, b = dev(q["a"]), dev(q["b_nk"]).t()
    sa, sb = dev(q["scale_a"]), dev(q["scale_b"])
    ws = torch.empty(3 * 2 * (256 * 256 * 4 + 8), dtype=torch.uint8, device=DEV)
    say("stream-K 3-workgroup workspace")
    with Forced("t256x256sk", 0):
        y1 = bsmm.bsmm_fp8_blockwise(a, b, sa, sb, out_dtype="f32", workspace=ws)
        y2 = bsmm.bsmm_fp8_blockwise(a, b, sa, sb, out_dtype="f32", workspace=ws)
    check_blockwise(q, "f32", y1)
    assert np.array_equal(host_out(y1).view(np.uint32), host_out(y2).view(np.uint32))


def test_streamk_data_parallel_rounds_then_split_tiles():
    """A four-workgroup workspace over nine 256 x 256 tiles: one data-parallel
    round of four whole tiles, then the other five tiles' K blocks spread
    over the four workgroups (tiles split across two of them), for every
    operation, several mx batches included; repeatable bit for bit."""
    q = fp8_blockwise_inputs(600, 640, 1280, 505)
    p = int8_rowwise_inputs(600, 640, 1280, 506)
    r = fp8_mx_bmm_inputs(3, 300, 640, 1280, 507, layout="batch_first")
    ws = torch.empty(4 * 2 * (256 * 256 * 4 + 8), dtype=torch.uint8, device=DEV)
    a, b = dev(q["a"]), dev(q["b_nk"]).t()
    sa, sb = dev(q["scale_a"]), dev(q["scale_b"])
    say("stream-K data-parallel rounds + split tiles (4 workgroups)")
    with Forced("t256x256sk", 0):
        y1 = bsmm.bsmm_fp8_blockwise(a, b, sa, sb, out_dtype="bf16", workspace=ws)
        y2 = bsmm.bsmm_fp8_blockwise(a, b, sa, sb, out_dtype="bf16", workspace=ws)
        yi = bsmm.bsmm_int8_rowwise(dev(p["a"]), dev(p["b_nk"]).t(),
                                    dev(p["scale_a"]).reshape(-1, 1),
                                    dev(p["scale_b"]).reshape(1, -1), out_dtype="f32",
                                    workspace=ws)
        ym = bsmm.bsmm_fp8_mx_bmm(dev(r["x"]), dev(r["w"]), dev(r["x_scale"]), dev(r["w_scale"]),
                                  layout="batch_first", out_dtype="f32", workspace=ws)
    check_blockwise(q, "bf16", y1)
    assert np.array_equal(host_out(y1), host_out(y2))
    check_int8(p, "f32", yi)
    check_mx(r, "f32", ym)


# ------------------------------------------------------- packed scales ----

@pytest.mark.parametrize("variant", PACKED_VARIANTS)
def test_packed_scales_strided_and_ragged(variant):
    """Packed-scale kernels: scale_a repacked from a column-major (stride 1
    along M) tensor and from a broadcast one, M not a multiple of 64, mx
    with several batches in both layouts."""
    q = fp8_blockwise_inputs(300, 384, 640, 601)
    a, b = dev(q["a"]), dev(q["b_nk"]).t()
    sa_cm = dev(np.ascontiguousarray(q["scale_a"].T)).t()            # [M, KB], stride (1, M)
    sa_bc = torch.full((1, 1), 0.0625, device=DEV).expand(300, 5)     # stride (0, 0)
    say(f"packed {variant} blockwise strided / broadcast scale_a")
    with Forced(variant, 0):
        y1 = bsmm.bsmm_fp8_blockwise(a, b, sa_cm, dev(q["scale_b"]), out_dtype="f32")
        y2 = bsmm.bsmm_fp8_blockwise(a, b, sa_bc, dev(q["scale_b"]), out_dtype="bf16")
    check_blockwise(q, "f32", y1)
    q2 = dict(q)
    q2["scale_a"] = np.full((300, 5), 0.0625, np.float32)
    check_blockwise(q2, "bf16", y2)
    for layout in ("m_major", "batch_first"):
        r = fp8_mx_bmm_inputs(3, 300, 256, 640, 602, layout=layout)
        say(f"packed {variant} mx {layout} G=3 M=300")
        with Forced(variant, 0):
            ym = run_mx(r, "f32")
        check_mx(r, "f32", ym)


def test_packed_bulk_with_unpacked_tail():
    """The default plan for a large fp8 call: a packed 256-row bulk launch
    followed by a 64-row tail launch that reads scale_a directly."""
    M, N, K = 8232, 256, 512
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_BLOCKWISE, 1, M, N, K, "f32")
    assert plan["variant"].endswith("p") and plan["m_split"] == 8192, plan
    q = fp8_blockwise_inputs(M, N, K, 603)
    say("packed bulk + unpacked tail")
    y = run_blockwise(q, "f32")
    rows = np.r_[0:300, 8100:M]
    check_blockwise(q, "f32", y, rows=rows)


def test_whole_rounds_bulk_with_split_k_tail():
    """A call whose last round of 256-row tiles would leave most CUs idle:
    the bulk launch covers whole rounds and the remaining rows (ragged)
    run with split K, both from one packed copy of scale_a."""
    M, N, K = 16534, 1024, 2048
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_BLOCKWISE, 1, M, N, K, "bf16")
    assert plan["m_split"] == 16384 and plan["tail_split_k"] > 1, plan
    q = fp8_blockwise_inputs(M, N, K, 604)
    say("whole-rounds bulk + split-K tail")
    y = run_blockwise(q, "bf16")
    rows = np.r_[0:64, 16300:M]
    check_blockwise(q, "bf16", y, rows=rows)
    y2 = run_blockwise(q, "bf16")
    assert np.array_equal(host_out(y), host_out(y2))


# ------------------------------------------------------------- skinny M ----

@pytest.mark.parametrize("M", [1, 5, 16])
def test_skinny_all_ops(M):
    """The M <= 16 kernel (K split over the four waves of a workgroup, B
    read straight into registers): the default plan for these M, with K
    blocks not a multiple of four, a ragged int8 N and several mx batches in
    both layouts."""
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX_BMM, 3, M, 384, 640, "bf16")
    assert plan["variant"] == "s16x16", plan
    p = int8_rowwise_inputs(M, 200, 640, 701 + M)
    for dt in ("i32", "f32", "bf16"):
        say(f"skinny int8 {dt} M={M} N=200 K=640")
        check_int8(p, dt, run_int8(p, dt))
    q = fp8_blockwise_inputs(M, 384, 896, 711 + M)
    for dt in ("bf16", "f32"):
        say(f"skinny blockwise {dt} M={M} N=384 K=896")
        check_blockwise(q, dt, run_blockwise(q, dt))
    for layout in ("m_major", "batch_first"):
        r = fp8_mx_bmm_inputs(3, M, 384, 640, 721 + M, layout=layout, dist="t")
        say(f"skinny mx {layout} G=3 M={M} N=384 K=640")
        check_mx(r, "bf16", run_mx(r, "bf16"))
        check_mx(r, "f32", run_mx(r, "f32"))


def test_skinny_short_k_and_guard_bands():
    """One and two K blocks (three or two waves with no K work) and a
    strided output inside a sentinel buffer."""
    for K in (128, 256):
        p = int8_rowwise_inputs(3, 130, K, 731)
        say(f"skinny int8 K={K}")
        check_int8(p, "i32", run_int8(p, "i32"))
        r = fp8_mx_bmm_inputs(2, 9, 256, K, 732, layout="m_major")
        say(f"skinny mx K={K}")
        check_mx(r, "f32", run_mx(r, "f32"))
    q = fp8_blockwise_inputs(7, 256, 512, 733)
    big = torch.full((12, 512), 7.0, dtype=torch.float32, device=DEV)
    view = big[2:9, 128:384]
    say("skinny blockwise guard bands")
    run_blockwise(q, "f32", out=view)
    check_blockwise(q, "f32", view)
    h = host_out(big)
    mask = np.ones_like(h, dtype=bool)
    mask[2:9, 128:384] = False
    assert (h[mask] == 7.0).all()


def test_skinny_forced_on_tall_m_falls_back():
    """Forcing the skinny kernel on M > 16 takes the regular plan."""
    p = int8_rowwise_inputs(40, 256, 512, 741)
    say("skinny forced on M=40")
    with Forced("s16x16", 0):
        plan = bsmm.bsmm_query_plan(bsmm.OP_INT8_ROWWISE, 1, 40, 256, 512, "i32")
        y = run_int8(p, "i32")
    assert plan["variant"] != "s16x16", plan
    check_int8(p, "i32", y)


# ----------------------------------------- stream-K grids, two streams ----

@pytest.mark.parametrize("grid", [0, 5, 600])
def test_int8_streamk_any_grid_exact(grid):
    """The int8 stream-K kernel (the dispatcher's choice for the 8192 x 4096
    x 4096 linear) at its default grid, at 5 workgroups and at 600, more
    than the device holds at once: split tiles are added up by the last of
    their segments to finish, so the int32 accumulators are bit-exact
    whatever the grid."""
    p = int8_rowwise_inputs(1024, 1024, 4096, 510)
    a, b = dev(p["a"]), dev(p["b_nk"]).t()
    sa, sb = dev(p["scale_a"]).reshape(-1, 1), dev(p["scale_b"]).reshape(1, -1)
    ws = torch.empty(600 * 2 * (256 * 256 * 4 + 8), dtype=torch.uint8, device=DEV)
    say(f"int8 stream-K grid {grid}")
    bsmm.bsmm_set_streamk_grid(grid)
    try:
        with Forced("t256x256skp", 0):
            yi = bsmm.bsmm_int8_rowwise(a, b, out_dtype="i32", workspace=ws)
            yb = bsmm.bsmm_int8_rowwise(a, b, sa, sb, out_dtype="bf16", workspace=ws)
    finally:
        bsmm.bsmm_set_streamk_grid(0)
    rows = np.r_[0:16, 500:520, 1000:1024]
    check_int8(p, "i32", yi, rows=rows)
    check_int8(p, "bf16", yb, rows=rows)


def test_two_streams_get_their_own_workspace():
    """Two split-K calls of the same shape queued on two streams at once:
    the binding gives each stream its own cached workspace, so their
    partial sums do not mix."""
    M, N, K = 256, 512, 4096
    plan = bsmm.bsmm_query_plan(bsmm.OP_FP8_BLOCKWISE, 1, M, N, K, "f32")
    assert plan["split_k"] > 1 and plan["workspace"] > 0, plan
    ps = [fp8_blockwise_inputs(M, N, K, 530 + i) for i in range(2)]
    ins = [(dev(q["a"]), dev(q["b_nk"]).t(), dev(q["scale_a"]), dev(q["scale_b"])) for q in ps]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    say("two streams, one shape, split-K")
    outs = [[], []]
    for _ in range(4):
        for i, s in enumerate(streams):
            outs[i].append(bsmm.bsmm_fp8_blockwise(*ins[i], out_dtype="f32", stream=s))
    torch.cuda.synchronize()
    for i, q in enumerate(ps):
        for y in outs[i]:
            check_blockwise(q, "f32", y)
