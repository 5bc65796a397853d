"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before any HIP call.  Also the
host-side plan selection and the dispatch table.  Pointers used here are
never dereferenced: every call fails validation (or is a no-op) first.
"""

import ctypes
import os
import re

import pytest

import block_scaled_precision_gemm_amd as bsmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsmm.h")
TABLE = os.path.join(ROOT, "block_scaled_precision_gemm_amd", "csrc", "bsmm_tuned_table.inc")

OK, NULL, SHAPE, SCALE, LAYOUT, ALIGN, DTYPE, UNSUP = 0, 1, 2, 3, 4, 5, 6, 7
P = 0x10000          # a fake, 16-byte-aligned "device pointer" (never touched)


@pytest.fixture(scope="module")
def L():
    return bsmm.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsmm_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "bsmm_fp8_blockwise" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"missing export {n}"
    assert bsmm.bsmm_version() == 1


def test_status_strings(L):
    for code, name in bsmm.STATUS.items():
        assert L.bsmm_status_string(code).decode() == name


def i8(*, a=P, lda=256, b=P, ldb=256, sa=P, sa_m=1, sb=P, sb_n=1, out=P, ldo=128,
       dt=bsmm.F32, M=64, N=128, K=256, ws=None, wsb=0):
    L = bsmm.load()
    return L.bsmm_int8_rowwise(a, lda, b, ldb, sa, sa_m, sb, sb_n, out, ldo, dt,
                               M, N, K, ws, wsb, None)


def bw(*, a=P, lda=256, b=P, ldb=256, sa=P, sa_m=2, sa_kb=1, sb=P, sb_kb=1, sb_nb=2,
       out=P, ldo=256, dt=bsmm.BF16, M=64, N=256, K=256):
    L = bsmm.load()
    return L.bsmm_fp8_blockwise(a, lda, b, ldb, sa, sa_m, sa_kb, sb, sb_kb, sb_nb,
                                out, ldo, dt, M, N, K, None, 0, None)


def bws(*, a=P, lda=256, b=P, ldb=256, sa=P, sa_m=2, sa_kb=1, sb=P, sb_kb=1, sb_nb=2,
        out=P, ldo=256, dt=bsmm.BF16, M=64, N=256, K=256):
    L = bsmm.load()
    return L.bsmm_fp8_blockwise_scratch(a, lda, b, ldb, sa, sa_m, sa_kb, sb, sb_kb, sb_nb,
                                        out, ldo, dt, M, N, K, None)


def test_blockwise_scratch_rejects_like_blockwise_and_beyond_the_scratch():
    """The allocation-free entry validates as bsmm_fp8_blockwise does, and
    rejects a problem whose plan wants more than the 64 MiB static scratch
    (2048 x 3840 x 8192: 120 tiles, split K 3, 90.5 MiB of partials) before
    any HIP call, naming the size."""
    for kw, status in ((dict(dt=bsmm.I32), DTYPE), (dict(N=200, ldo=256), UNSUP),
                       (dict(sa=None), NULL), (dict(ldb=255), SHAPE), (dict(b=P + 4), ALIGN)):
        assert bws(**kw) == status == bw(**kw)
    assert bws(M=0) == OK
    need = bsmm.bsmm_workspace_bytes(bsmm.OP_FP8_BLOCKWISE, 1, 2048, 3840, 8192, bsmm.BF16)
    assert need > 64 << 20
    st = bws(M=2048, N=3840, K=8192, lda=8192, ldb=8192, ldo=3840, sa_m=64, sb_nb=64)
    assert st == UNSUP
    msg = bsmm.load().bsmm_last_error().decode()
    assert str(need) in msg and str(64 << 20) in msg


def mx(*, x=P, x_sg=512, x_sm=4096, w=P, w_sg=1 << 20, w_sn=512, xs=P, xs_sg=4,
       xs_sm=32, ws=P, ws_sg=64, ws_snb=4, out=P, o_sg=256, o_sm=2048,
       dt=bsmm.BF16, G=8, M=16, N=256, K=512):
    L = bsmm.load()
    return L.bsmm_fp8_mx_bmm(x, x_sg, x_sm, w, w_sg, w_sn, xs, xs_sg, xs_sm, ws, ws_sg,
                             ws_snb, out, o_sg, o_sm, dt, G, M, N, K, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), SHAPE), (dict(N=-5), SHAPE), (dict(K=-128), SHAPE),
    (dict(K=200), UNSUP), (dict(K=2**31), UNSUP), (dict(K=133248, lda=133248, ldb=133248), UNSUP),
    # int8 codes include -128: K * 2^14 must stay below 2^31, so 130944 is the
    # largest K (passes the size check and fails on the NULL output instead)
    (dict(K=131072, lda=131072, ldb=131072), UNSUP),
    (dict(K=130944, lda=130944, ldb=130944, out=None), NULL),
    (dict(dt=7), DTYPE),
    (dict(out=None), NULL), (dict(a=None), NULL), (dict(sa=None), NULL),
    (dict(sa_m=-1), SCALE), (dict(sb_n=-2), SCALE),
    (dict(lda=128), SHAPE), (dict(ldo=100), SHAPE),
    (dict(lda=264), ALIGN), (dict(a=P + 8), ALIGN), (dict(sa=P + 2), ALIGN),
    (dict(lda=1 << 24, ldb=1 << 24), UNSUP),
])
def test_int8_rejects(kw, status):
    assert i8(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


def test_int8_noops_and_int32_mode_without_scales():
    assert i8(M=0) == OK            # nothing to compute: returns before any launch
    assert i8(N=0, a=None, b=None, out=None) == OK
    # int32 mode ignores the scales: NULL scales pass validation (then M=0)
    assert i8(M=0, sa=None, sb=None, dt=bsmm.I32) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(dt=bsmm.I32), DTYPE), (dict(N=200, ldo=256), UNSUP), (dict(K=100), UNSUP),
    (dict(sa=None), NULL), (dict(sb=None), NULL), (dict(out=None), NULL),
    (dict(sa_kb=-1), SCALE), (dict(sb_nb=-1), SCALE),
    (dict(ldb=255), SHAPE), (dict(ldb=264), ALIGN), (dict(b=P + 4), ALIGN),
    (dict(sa_m=1 << 30), UNSUP),
])
def test_blockwise_rejects(kw, status):
    assert bw(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(G=-1), SHAPE), (dict(dt=bsmm.I32), DTYPE), (dict(N=192, o_sm=192), UNSUP),
    (dict(x_sm=256), LAYOUT), (dict(w_sn=100), LAYOUT), (dict(o_sm=100), LAYOUT),
    (dict(x_sg=-512), LAYOUT), (dict(xs_sm=-1), SCALE), (dict(x_sm=4104), ALIGN),
    (dict(w_sg=8), ALIGN), (dict(xs=None), NULL), (dict(w=None), NULL),
])
def test_mx_rejects(kw, status):
    assert mx(**kw) == status


def test_mx_noops():
    assert mx(G=0) == OK and mx(M=0) == OK and mx(N=0) == OK


def smm(*, a=P, lda=256, b=P, ldb=256, sa=P, sa_m=1, sb=P, sb_n=1, bias=None,
        bdt=bsmm.F32, sr=None, out=P, ldo=128, dt=bsmm.BF16, M=64, N=128, K=256):
    return bsmm.load().bsmm_fp8_scaled_mm(a, lda, b, ldb, sa, sa_m, sb, sb_n, bias, bdt, sr,
                                          out, ldo, dt, M, N, K, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), SHAPE), (dict(dt=bsmm.I32), DTYPE), (dict(dt=9), DTYPE), (dict(K=200), UNSUP),
    (dict(out=None), NULL), (dict(sa=None), NULL), (dict(sb=None), NULL), (dict(a=None), NULL),
    (dict(sa_m=-1), SCALE), (dict(sb_n=-1), SCALE), (dict(ldo=100), SHAPE),
    (dict(lda=128), SHAPE), (dict(ldb=264), ALIGN), (dict(b=P + 4), ALIGN),
    (dict(sa=P + 2), ALIGN), (dict(bias=P, bdt=bsmm.I32), DTYPE),
    (dict(bias=P + 2, bdt=bsmm.F32), ALIGN), (dict(sr=P + 1), ALIGN),
    (dict(out=P + 1, dt=bsmm.BF16), ALIGN), (dict(sa_m=1 << 30), UNSUP),
])
def test_scaled_mm_rejects(kw, status):
    assert smm(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


def test_scaled_mm_noops_and_plans():
    assert smm(M=0) == OK and smm(N=0, a=None, b=None, out=None) == OK
    # an odd byte address is fine for e4m3 output and a bf16 bias; M=0 keeps
    # the call from launching
    assert smm(M=0, out=P + 1, dt=bsmm.E4M3, bias=P + 2, bdt=bsmm.BF16) == OK
    # no scales in the K loop: never a packed-scale plan, no packing workspace
    p = bsmm.bsmm_query_plan(bsmm.OP_FP8_SCALED_MM, 1, 16640, 5120, 8192, "bf16")
    assert not p["variant"].endswith("p") and p["tail_split_k"] >= 2
    assert bsmm.bsmm_query_plan(bsmm.OP_FP8_SCALED_MM, 1, 8, 300, 1024, "e4m3")["variant"] == \
        "s16x16"
    p = bsmm.bsmm_query_plan(bsmm.OP_FP8_SCALED_MM, 1, 4096, 4096, 4096, "f32")
    assert p["workspace"] == 0 and not p["variant"].endswith("p")


def mx32(*, a=P, lda=256, b=P, ldb=256, sa=P, as_m=8, sb=P, bs_n=8, out=P, ldo=128,
         dt=bsmm.BF16, M=64, N=128, K=256):
    return bsmm.load().bsmm_fp8_mx32_mm(a, lda, b, ldb, sa, as_m, sb, bs_n, out, ldo, dt, M, N,
                                        K, None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), SHAPE), (dict(dt=bsmm.I32), DTYPE), (dict(dt=bsmm.E4M3), DTYPE),
    (dict(K=96), UNSUP), (dict(out=None), NULL), (dict(sa=None), NULL), (dict(b=None), NULL),
    (dict(as_m=7), SCALE), (dict(bs_n=-1), SCALE), (dict(ldo=100), SHAPE), (dict(lda=128), SHAPE),
    (dict(ldb=264), ALIGN), (dict(a=P + 4), ALIGN), (dict(out=P + 2), ALIGN),
    (dict(as_m=1 << 26), UNSUP),
])
def test_mx32_rejects(kw, status):
    assert mx32(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


def test_mx32_noops_and_plans():
    assert mx32(M=0) == OK and mx32(N=0) == OK
    # byte scales need no alignment
    assert mx32(M=0, sa=P + 1, sb=P + 3) == OK
    # the tile kernels read packed scales: A [K/32][M rounded to 256] bytes,
    # then B [K/32][N rounded to 256] bytes, before the split-K partials
    M, N, K = 16640, 5120, 8192
    p = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX32_MM, 1, M, N, K, "bf16")
    assert p["variant"] == "t256x256p" and p["m_split"] == 16384
    pack = (K // 32) * 16640 + (K // 32) * 5120
    assert p["workspace"] == pack + p["tail_split_k"] * 256 * N * 4
    q = bsmm.bsmm_query_plan(bsmm.OP_FP8_MX32_MM, 1, 200, 384, 512, "bf16", workspace_bytes=0)
    assert q["variant"] == "t256x128" and q["workspace"] == 0      # no workspace: unpacked
    assert bsmm.bsmm_query_plan(bsmm.OP_FP8_MX32_MM, 1, 3, 256, 512, "f32")["variant"] == "s16x16"


def gw(*, a=P, lda=256, b=P, ldb=256, sa=P, sa_m=2, sa_kb=1, sb=P, sb_kb=200, sb_n=1, out=P,
       ldo=200, dt=bsmm.BF16, M=64, N=200, K=256, ws=None, wsn=0):
    return bsmm.load().bsmm_fp8_groupwise(a, lda, b, ldb, sa, sa_m, sa_kb, sb, sb_kb, sb_n, out,
                                          ldo, dt, M, N, K, ws, wsn, None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), SHAPE), (dict(dt=bsmm.I32), DTYPE), (dict(dt=bsmm.E4M3), DTYPE),
    (dict(K=200), UNSUP), (dict(out=None), NULL), (dict(sa=None), NULL), (dict(sb=None), NULL),
    (dict(a=None), NULL), (dict(sa_kb=-1), SCALE), (dict(sb_n=-1), SCALE),
    (dict(ldo=100), SHAPE), (dict(lda=128), SHAPE), (dict(ldb=264), ALIGN),
    (dict(b=P + 4), ALIGN), (dict(sa=P + 2), ALIGN), (dict(out=P + 2), ALIGN),
    (dict(sb_n=1 << 30), UNSUP), (dict(K=128 * 70000, lda=128 * 70000, ldb=128 * 70000), UNSUP),
])
def test_groupwise_rejects(kw, status):
    assert gw(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


def test_groupwise_noops_and_needs_a_workspace():
    assert gw(M=0) == OK and gw(N=0) == OK
    # N need not be a multiple of 128 (one scale per column); without a
    # workspace for the packed scales the call is refused before any launch
    assert gw() == 9
    assert "workspace" in bsmm.load().bsmm_last_error().decode()
    need = bsmm.bsmm_workspace_bytes(bsmm.OP_FP8_GROUPWISE, 1, 64, 200, 256, "bf16")
    assert need == 2 * (2 * 256 * 4)       # K/128 blocks x rows / columns padded to 256
    assert gw(ws=P, wsn=need - 256) == 9


def test_groupwise_plans():
    # the weight gradient of the 16640 x 8192 -> 5120 layer: dW [5120, 8192]
    # over 16640 tokens; two whole rounds of 256 x 256 tiles, the last 1024
    # rows split K two ways
    M, N, K = 5120, 8192, 16640
    p = bsmm.bsmm_query_plan(bsmm.OP_FP8_GROUPWISE, 1, M, N, K, "bf16")
    assert p["variant"] == "t256x256p" and p["m_split"] == 4096 and p["tail_split_k"] == 2
    pack = (K // 128) * M * 4 + (K // 128) * N * 4
    assert p["workspace"] == pack + 2 * 1024 * N * 4
    # only packed-scale kernels, at every M (no skinny or 64-row kernel)
    for m, n in ((1, 256), (16, 384), (64, 200), (128, 512), (300, 640)):
        v = bsmm.bsmm_query_plan(bsmm.OP_FP8_GROUPWISE, 1, m, n, 1024, "f32")["variant"]
        assert v.endswith("p"), (m, n, v)


def qi8(*, x=P, ldx=256, xdt=bsmm.BF16, q=P, ldq=256, sc=P, s_m=1, M=64, K=256):
    return bsmm.load().bsmm_quant_int8_rowwise(x, ldx, xdt, q, ldq, sc, s_m, M, K, None)


def qbw(*, fn="bsmm_quant_fp8_blockwise", x=P, ldx=256, xdt=bsmm.F32, q=P, ldq=256, sc=P,
        s_m=2, s_kb=1, M=64, K=256):
    return getattr(bsmm.load(), fn)(x, ldx, xdt, q, ldq, sc, s_m, s_kb, M, K, None)


@pytest.mark.parametrize("kw,status", [
    (dict(xdt=bsmm.I32), DTYPE), (dict(M=-1), SHAPE), (dict(K=-8), SHAPE),
    (dict(K=100), UNSUP), (dict(M=(1 << 26) + 1), UNSUP), (dict(K=2**31), UNSUP),
    (dict(sc=None), NULL), (dict(x=None), NULL), (dict(q=None), NULL),
    (dict(s_m=-1), SCALE), (dict(s_m=0), SCALE),
    (dict(ldx=128), SHAPE), (dict(ldq=128), SHAPE), (dict(ldx=260), ALIGN),
    (dict(ldq=260), ALIGN), (dict(x=P + 8), ALIGN), (dict(q=P + 4), ALIGN),
    (dict(sc=P + 2), ALIGN),
])
def test_quant_int8_rejects(kw, status):
    assert qi8(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


def test_quant_mx32_rejects_and_noops():
    L = bsmm.load()
    call = lambda **kw: L.bsmm_quant_fp8_mx32(
        kw.get("x", P), kw.get("ldx", 256), kw.get("xdt", bsmm.BF16), kw.get("q", P),
        kw.get("ldq", 256), kw.get("sc", P), kw.get("s_m", 8), kw.get("s_kb", 1),
        kw.get("M", 64), kw.get("K", 256), None)
    assert call(K=48) == UNSUP                    # not a multiple of 32
    assert call(K=96, s_m=3, M=0) == OK           # 32-element blocks: K = 96 is fine
    assert call(s_m=7) == SCALE                   # rows of 8 scales overlap
    assert call(xdt=bsmm.I32) == DTYPE
    assert call(K=0, x=None, q=None, sc=None) == OK


@pytest.mark.parametrize("fn", ["bsmm_quant_fp8_blockwise", "bsmm_quant_fp8_mx"])
@pytest.mark.parametrize("kw,status", [
    (dict(xdt=7), DTYPE), (dict(K=200), UNSUP), (dict(M=1 << 23, K=1 << 14, ldx=1 << 14,
                                                          ldq=1 << 14, s_m=128), UNSUP),
    (dict(sc=None), NULL), (dict(x=None), NULL),
    (dict(s_kb=-1), SCALE), (dict(s_m=1, s_kb=1), SCALE), (dict(s_m=0), SCALE),
    (dict(s_kb=0), SCALE), (dict(s_m=1, s_kb=63), SCALE),
    (dict(ldq=255), SHAPE), (dict(ldx=260), ALIGN), (dict(q=P + 4), ALIGN),
    (dict(ldq=260), ALIGN),
])
def test_quant_fp8_rejects(fn, kw, status):
    assert qbw(fn=fn, **kw) == status


def test_quant_noops_and_scale_layouts():
    assert qi8(M=0, x=None, q=None, sc=None) == OK
    # fp8 with K == 0 has no blocks: nothing is read or written
    for fn in ("bsmm_quant_fp8_blockwise", "bsmm_quant_fp8_mx"):
        assert qbw(fn=fn, K=0, x=None, q=None, sc=None) == OK
        assert qbw(fn=fn, M=0) == OK
        # the column-major scale layout (s_m = 1, s_kb = M) passes validation;
        # M = 0 keeps the call from launching
        assert qbw(fn=fn, M=0, s_m=1, s_kb=64) == OK
    assert bsmm.load().bsmm_quant_fp8_mx(P, 256, bsmm.F32, P, 256, P + 1, 2, 1, 0, 256,
                                         None) == OK   # byte scales need no alignment


# ----------------------------------------------------------------- binding --

def qcol(*, x=P, ldx=256, xdt=bsmm.BF16, qt=P, ldqt=256, sc=P, s_g=256, s_c=1, R=256, C=256):
    return bsmm.load().bsmm_quant_fp8_columns(x, ldx, xdt, qt, ldqt, sc, s_g, s_c, R, C, None)


def qw(*, w=P, ldw=256, wdt=bsmm.F32, q=P, ldq=256, qt=P, ldqt=256, sc=P, s_r=2, s_c=1, R=256,
       C=256):
    return bsmm.load().bsmm_quant_fp8_weight(w, ldw, wdt, q, ldq, qt, ldqt, sc, s_r, s_c, R, C,
                                             None)


@pytest.mark.parametrize("kw,status", [
    (dict(xdt=bsmm.I32), DTYPE), (dict(R=-128), SHAPE), (dict(R=200), UNSUP), (dict(C=100), UNSUP),
    (dict(R=128 * 65536, ldqt=128 * 65536), UNSUP), (dict(sc=None), NULL), (dict(x=None), NULL),
    (dict(qt=None), NULL), (dict(s_g=-1), SCALE), (dict(s_g=100), SCALE), (dict(s_c=0), SCALE),
    (dict(ldx=128), SHAPE), (dict(ldqt=128), SHAPE), (dict(ldx=260), ALIGN),
    (dict(ldqt=264), ALIGN), (dict(x=P + 8), ALIGN), (dict(qt=P + 8), ALIGN), (dict(sc=P + 2), ALIGN),
])
def test_quant_columns_rejects(kw, status):
    assert qcol(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(wdt=bsmm.BF16 + 5), DTYPE), (dict(C=200, ldw=256, ldq=256), UNSUP), (dict(R=192), UNSUP),
    (dict(q=None, qt=None), NULL), (dict(sc=None), NULL), (dict(w=None), NULL),
    (dict(s_r=1, s_c=1), SCALE), (dict(ldq=128), SHAPE), (dict(ldq=260), ALIGN),
    (dict(q=P + 4), ALIGN), (dict(ldqt=255), SHAPE), (dict(qt=P + 8), ALIGN),
])
def test_quant_weight_rejects(kw, status):
    assert qw(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


def qrc(*, x=P, ldx=256, xdt=bsmm.BF16, q=P, ldq=256, sr=P, sr_m=2, sr_kb=1, qt=P, ldqt=256,
        sc=P, sc_g=256, sc_c=1, R=256, C=256):
    return bsmm.load().bsmm_quant_fp8_blockwise_columns(x, ldx, xdt, q, ldq, sr, sr_m, sr_kb, qt,
                                                        ldqt, sc, sc_g, sc_c, R, C, None)


@pytest.mark.parametrize("kw,status", [
    (dict(xdt=bsmm.I32), DTYPE), (dict(R=200), UNSUP), (dict(C=200, ldx=256, ldq=256), UNSUP),
    (dict(q=None), NULL), (dict(qt=None), NULL), (dict(sr=None), NULL), (dict(sc=None), NULL),
    (dict(sr_m=1, sr_kb=1), SCALE), (dict(sr_m=-1), SCALE), (dict(sc_c=0), SCALE),
    (dict(ldq=128), SHAPE), (dict(ldq=260), ALIGN), (dict(ldqt=128), SHAPE),
    (dict(qt=P + 8), ALIGN), (dict(sr=P + 2), ALIGN), (dict(x=P + 8), ALIGN),
])
def test_quant_blockwise_columns_rejects(kw, status):
    assert qrc(**kw) == status
    assert bsmm.load().bsmm_last_error().decode()


def test_quant_backward_noops_and_single_outputs():
    assert qcol(R=0) == OK and qcol(C=0) == OK and qw(R=0) == OK and qw(C=0) == OK
    assert qrc(R=0) == OK and qrc(C=0) == OK
    # C need only be a multiple of 8 for the column groups; either output
    # of the weight quantiser alone is fine (M = 0 rows keeps it from launching)
    assert qcol(C=200, ldx=200 + 8, R=0) == OK
    assert qw(q=None, R=0) == OK and qw(qt=None, R=0) == OK


def test_binding_scale_shape_rules_follow_the_page():
    """The rowwise/tensorwise message and the blockwise shapes of the PyTorch
    blockwise _scaled_mm issue: (16640, 64) / (64, 40) for M=16640, K=8192,
    N=5120 are the blockwise scales; rowwise-shaped scales are rejected."""
    import torch
    M, N, K = 16640, 5120, 8192
    a = torch.empty((M, K), dtype=torch.float8_e4m3fn)
    b = torch.empty((N, K), dtype=torch.float8_e4m3fn).t()
    with pytest.raises(ValueError, match=r"scale_a should be \(16640, 64\)"):
        bsmm.bsmm_fp8_blockwise(a, b, torch.empty(M, 1), torch.empty(1, N))
    ai = torch.empty((M, K), dtype=torch.int8)
    bi = torch.empty((N, K), dtype=torch.int8).t()
    with pytest.raises(ValueError, match=r"rowwise scaling, scale_a should be \(16640, 1\)"):
        bsmm.bsmm_int8_rowwise(ai, bi, torch.empty(M, 64), torch.empty(64, 40))
    with pytest.raises(ValueError, match="column-major"):
        bsmm.bsmm_int8_rowwise(ai, torch.empty((K, N), dtype=torch.int8),
                               torch.empty(M, 1), torch.empty(1, N))
    x = torch.empty((4, 8, 512), dtype=torch.uint8)
    w = torch.empty((8, 256, 512), dtype=torch.uint8)
    with pytest.raises(ValueError, match="x_scale should be"):
        bsmm.bsmm_fp8_mx_bmm(x, w, torch.empty((4, 8, 3), dtype=torch.uint8),
                             torch.empty((8, 2, 4), dtype=torch.uint8))


# ---------------------------------------------------------------- dispatch --

def test_plan_heuristics():
    q = bsmm.bsmm_query_plan
    p = q(bsmm.OP_FP8_BLOCKWISE, 1, 16640, 5120, 8192, "bf16")
    assert p["tile_m"] in (128, 256) and p["split_k"] >= 1
    # (a shape with no tuned-table entry, so the heuristic decides)
    small = q(bsmm.OP_FP8_MX_BMM, 8, 40, 2048, 4096, "bf16")
    assert small["source"] == 2
    assert small["tile_m"] == 64 and small["split_k"] > 1
    assert small["workspace"] == small["split_k"] * 8 * 40 * 2048 * 4
    # without workspace the same problem runs unsplit
    nows = q(bsmm.OP_FP8_MX_BMM, 8, 40, 2048, 4096, "bf16", workspace_bytes=0)
    assert nows["split_k"] == 1 and nows["workspace"] == 0
    assert bsmm.bsmm_workspace_bytes(bsmm.OP_FP8_MX_BMM, 8, 40, 2048, 4096, "bf16") == \
        small["workspace"]


def test_plan_skinny_m():
    """M <= 16 runs the skinny kernel for every operation, unsplit and
    without workspace; M = 17 does not, and forcing it on a taller M falls
    back to the regular plan."""
    q = bsmm.bsmm_query_plan
    for op in (bsmm.OP_INT8_ROWWISE, bsmm.OP_FP8_BLOCKWISE, bsmm.OP_FP8_MX_BMM):
        for M in (1, 16):
            p = q(op, 8 if op == bsmm.OP_FP8_MX_BMM else 1, M, 1024, 4096, "bf16")
            assert p["variant"] == "s16x16" and p["split_k"] == 1 and p["workspace"] == 0, p
            assert p["m_split"] == 0
        assert q(op, 1, 17, 1024, 4096, "bf16")["variant"] != "s16x16"
    try:
        bsmm.bsmm_set_override("s16x16", 4)
        assert q(bsmm.OP_INT8_ROWWISE, 1, 8, 1024, 4096, "bf16")["split_k"] == 1
        assert q(bsmm.OP_INT8_ROWWISE, 1, 40, 1024, 4096, "bf16")["variant"] != "s16x16"
    finally:
        bsmm.bsmm_set_override(None, 0)


def test_tuned_table_exact_and_padded_m():
    """A tuned entry serves its exact shape (source 0) and, as the padded-M
    bucket, smaller M of the same (op, dtype, G, N, K) (source 1), but never
    M <= 16, which keeps the skinny kernel (groupwise has none), and never
    for stream-K entries."""
    rows = parse_table()
    q = bsmm.bsmm_query_plan
    dts = {0: "i32", 1: "f32", 2: "bf16"}
    for f in rows:
        op, dt, G, M, N, K = (int(x) for x in f[:6])
        assert q(op, G, M, N, K, dts[dt])["source"] == 0
        if M > 17:
            below = q(op, G, M - 1, N, K, dts[dt])
            if "sk" in f[6]:      # stream-K entries serve their exact shape only
                assert below["source"] == 2
            else:
                assert below["source"] == 1 and below["variant"] == f[6]
            if op != bsmm.OP_FP8_GROUPWISE:
                assert q(op, G, 8, N, K, dts[dt])["variant"] == "s16x16"


def test_override_roundtrip():
    try:
        bsmm.bsmm_set_override("t128x128", 3)
        p = bsmm.bsmm_query_plan(bsmm.OP_INT8_ROWWISE, 1, 4096, 4096, 4096, "bf16")
        assert p["variant"] == "t128x128" and p["split_k"] == 3 and p["source"] == 3
        with pytest.raises(bsmm.BsmmError):
            bsmm.bsmm_set_override("no_such_variant", 0)
    finally:
        bsmm.bsmm_set_override(None, 0)
    p = bsmm.bsmm_query_plan(bsmm.OP_INT8_ROWWISE, 1, 4096, 4096, 4096, "bf16")
    assert p["source"] != 3


def parse_table():
    rows = []
    for line in open(TABLE):
        line = line.split("//")[0].strip()
        if not line:
            continue
        m = re.match(r"\{(.*)\},?$", line)
        assert m, line
        f = [x.strip().strip('"') for x in m.group(1).split(",")]
        rows.append(f)
    return rows


def test_dispatch_table_keys_unique_and_variants_exist():
    names = set(bsmm.bsmm_variant_names())
    keys = set()
    for f in parse_table():
        key = tuple(int(x) for x in f[:6])
        assert key not in keys, f"duplicate dispatch key {key}"
        keys.add(key)
        assert f[6] in names
        if int(f[8]):
            assert f[9] in names
    # every table entry is what the dispatcher returns for its key
    for f in parse_table():
        op, dt, G, M, N, K = (int(x) for x in f[:6])
        p = bsmm.bsmm_query_plan(op, G, M, N, K, {0: "i32", 1: "f32", 2: "bf16"}[dt])
        assert p["source"] == 0 and p["variant"] == f[6]


def test_int8_packed_variant_needs_no_workspace():
    """Packed variants only repack fp8 scales: an int8 plan on one needs no
    workspace."""
    import block_scaled_precision_gemm_amd as b
    b.bsmm_set_override("t256x256p", 0)
    try:
        assert b.bsmm_query_plan(b.OP_INT8_ROWWISE, 1, 4096, 4096, 4096, "bf16")["workspace"] == 0
        assert b.bsmm_query_plan(b.OP_FP8_BLOCKWISE, 1, 4096, 4096, 4096, "bf16")["workspace"] > 0
    finally:
        b.bsmm_set_override(None, 0)


def test_timing_hook_host_paths(L):
    """Timing hook without a GPU: enabling clears the record, reading an empty
    record returns zero launches, NULL outputs are rejected."""
    bsmm.bsmm_timing_enable(True)
    assert bsmm.bsmm_timing_read() == (0.0, 0, "")
    bsmm.bsmm_timing_enable(False)
    assert L.bsmm_timing_read(None, None, None, 0) == 1   # BSMM_ERR_NULL


def test_tuner_candidates_and_table_format(tmp_path, monkeypatch):
    """The tuning tool's host side: shape parsing, the distinct plans the
    override yields (every one a known variant, skinny only for M <= 16),
    and a table it writes parses back with unique keys."""
    from block_scaled_precision_gemm_amd import tune
    sh = tune.parse_shape("mx,bf16,8,128,1024,4096,m_major")
    assert (sh["G"], sh["M"], sh["N"], sh["K"], sh["layout"]) == (8, 128, 1024, 4096, "m_major")
    names = set(bsmm.bsmm_variant_names())
    cands = tune.candidates(sh)
    assert len(cands) > 5 and all(c[0] in names for c in cands)
    assert all(c[0] != "s16x16" for c in cands) and all(c[2] == 0 for c in cands)
    assert ("s16x16", 1, 0, "", 1) in tune.candidates(tune.parse_shape("int8,bf16,1,4,4096,4096"))
    # a shape the dispatcher splits in M also gets bulk + tail candidates,
    # each one a plan the forced override really produces
    c3 = tune.parse_shape("fp8_blockwise,bf16,1,16640,5120,8192")
    tails = [c for c in tune.candidates(c3) if c[2]]
    assert len(tails) > 20 and {c[2] for c in tails} == {16384, 16128}
    assert all(c[3] in names and not c[3].startswith("s") for c in tails)
    try:
        tune.set_plan(tails[0])
        p = bsmm.bsmm_query_plan(bsmm.OP_FP8_BLOCKWISE, 1, 16640, 5120, 8192, "bf16")
        assert (p["m_split"], p["tail_variant"], p["source"]) == (tails[0][2], tails[0][3], 3)
    finally:
        tune.clear_plan()
    monkeypatch.setattr(tune, "TABLE", str(tmp_path / "t.inc"))
    rows = {(2, 2, 8, 128, 1024, 4096): '{2, 2, 8, 128, 1024, 4096, "t128x128", 4, 0, "", 1}'}
    tune.write_table(rows)
    assert tune.read_table() == rows
    with pytest.raises(SystemExit):
        tune.parse_shape("fp16,bf16,1,2,3,4")
