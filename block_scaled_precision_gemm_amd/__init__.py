"""Python binding of libbsmm (the block-scaled matmul for MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libbsmm.so``.  The functions take PyTorch tensors (PyTorch is
used for device memory and streams), check shapes the way ``_scaled_mm``
states its scaling rules (ValueError), and pass raw pointers, strides and the
current HIP stream to the C ABI in ``include/bsmm.h``.  There is no fallback:
if the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "load", "lib_path", "BsmmError",
    "bsmm_int8_rowwise", "bsmm_fp8_blockwise", "bsmm_fp8_blockwise_scratch",
    "bsmm_fp8_mx_bmm", "bsmm_fp8_scaled_mm",
    "bsmm_fp8_mx32_mm", "OP_FP8_MX32_MM", "bsmm_fp8_groupwise", "OP_FP8_GROUPWISE",
    "bsmm_quant_int8_rowwise", "bsmm_quant_fp8_blockwise", "bsmm_quant_fp8_mx",
    "bsmm_quant_fp8_columns", "bsmm_quant_fp8_weight", "bsmm_quant_fp8_blockwise_columns",
    "bsmm_workspace_bytes", "bsmm_query_plan", "bsmm_set_override", "bsmm_set_override_tail", "bsmm_set_streamk_grid", "bsmm_mfma_probe",
    "bsmm_variant_names", "bsmm_version", "bsmm_timing_enable", "bsmm_timing_read",
    "I32", "F32", "BF16", "E4M3", "OP_INT8_ROWWISE", "OP_FP8_BLOCKWISE", "OP_FP8_MX_BMM",
    "OP_FP8_SCALED_MM",
    "STATUS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# BSMM_LIB_PATH: another build of the same library (the sanitized host
# build) in place of the in-tree one
lib_path = os.environ.get("BSMM_LIB_PATH") or os.path.join(_PKG, "libbsmm.so")

I32, F32, BF16, E4M3 = 0, 1, 2, 3
OP_INT8_ROWWISE, OP_FP8_BLOCKWISE, OP_FP8_MX_BMM, OP_FP8_SCALED_MM, OP_FP8_MX32_MM = 0, 1, 2, 3, 4
OP_FP8_GROUPWISE = 5
STATUS = {0: "BSMM_OK", 1: "BSMM_ERR_NULL", 2: "BSMM_ERR_SHAPE",
          3: "BSMM_ERR_SCALE_SHAPE", 4: "BSMM_ERR_LAYOUT", 5: "BSMM_ERR_ALIGN",
          6: "BSMM_ERR_DTYPE", 7: "BSMM_ERR_UNSUPPORTED", 8: "BSMM_ERR_HIP",
          9: "BSMM_ERR_ARG"}

_lib = None


class BsmmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_char * 48), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("m_split", ctypes.c_int32), ("workspace", ctypes.c_int64),
                ("source", ctypes.c_int32), ("tail_variant", ctypes.c_char * 48),
                ("tail_split_k", ctypes.c_int32)]


def load():
    """Load the in-tree libbsmm.so (once) and declare its prototypes.

    PyTorch is imported first: its HIP runtime must be the one in the
    process before the library's own dependency on a HIP runtime is
    resolved, or the library would bring in a second runtime whose launches
    and allocations do not mix with torch's.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise RuntimeError(f"{lib_path} is not built; run __graft_entry__.build()")
    import torch  # noqa: F401  (see above)
    L = ctypes.CDLL(lib_path)
    i64, vp, sz, st = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.bsmm_int8_rowwise.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, st,
                                    i64, i64, i64, vp, sz, vp]
    L.bsmm_fp8_blockwise.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp, i64, i64,
                                     vp, i64, st, i64, i64, i64, vp, sz, vp]
    L.bsmm_fp8_groupwise.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp, i64, i64,
                                     vp, i64, st, i64, i64, i64, vp, sz, vp]
    L.bsmm_fp8_blockwise_scratch.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp, i64, i64,
                                             vp, i64, st, i64, i64, i64, vp]
    L.bsmm_fp8_mx_bmm.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64,
                                  i64, vp, i64, i64, st, i64, i64, i64, i64, vp, sz, vp]
    L.bsmm_fp8_scaled_mm.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, st, vp,
                                     vp, i64, st, i64, i64, i64, vp, sz, vp]
    L.bsmm_fp8_mx32_mm.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, vp, i64, st, i64, i64,
                                   i64, vp, sz, vp]
    L.bsmm_quant_int8_rowwise.argtypes = [vp, i64, st, vp, i64, vp, i64, i64, i64, vp]
    L.bsmm_quant_fp8_blockwise.argtypes = [vp, i64, st, vp, i64, vp, i64, i64, i64, i64, vp]
    L.bsmm_quant_fp8_mx.argtypes = [vp, i64, st, vp, i64, vp, i64, i64, i64, i64, vp]
    L.bsmm_quant_fp8_mx32.argtypes = [vp, i64, st, vp, i64, vp, i64, i64, i64, i64, vp]
    L.bsmm_quant_fp8_columns.argtypes = [vp, i64, st, vp, i64, vp, i64, i64, i64, i64, vp]
    L.bsmm_quant_fp8_weight.argtypes = [vp, i64, st, vp, i64, vp, i64, vp, i64, i64, i64, i64,
                                        vp]
    L.bsmm_quant_fp8_blockwise_columns.argtypes = [vp, i64, st, vp, i64, vp, i64, i64, vp, i64,
                                                   vp, i64, i64, i64, i64, vp]
    for f in ("bsmm_int8_rowwise", "bsmm_fp8_blockwise", "bsmm_fp8_blockwise_scratch",
              "bsmm_fp8_mx_bmm", "bsmm_fp8_scaled_mm",
              "bsmm_fp8_mx32_mm",
              "bsmm_quant_int8_rowwise", "bsmm_quant_fp8_blockwise", "bsmm_quant_fp8_mx",
              "bsmm_quant_fp8_mx32", "bsmm_quant_fp8_columns", "bsmm_quant_fp8_weight",
              "bsmm_quant_fp8_blockwise_columns"):
        getattr(L, f).restype = st
    L.bsmm_workspace_bytes.argtypes = [st, i64, i64, i64, i64, st]
    L.bsmm_workspace_bytes.restype = sz
    L.bsmm_query_plan.argtypes = [st, i64, i64, i64, i64, st, sz, ctypes.POINTER(PlanInfo)]
    L.bsmm_query_plan.restype = st
    L.bsmm_set_override.argtypes = [ctypes.c_char_p, st]
    L.bsmm_set_override.restype = st
    L.bsmm_set_override_tail.argtypes = [st, ctypes.c_char_p, st]
    L.bsmm_set_override_tail.restype = st
    L.bsmm_set_streamk_grid.argtypes = [st]
    L.bsmm_set_streamk_grid.restype = st
    L.bsmm_mfma_probe.argtypes = [st, st, st, vp, vp]
    L.bsmm_mfma_probe.restype = st
    L.bsmm_variant_names.restype = ctypes.c_char_p
    L.bsmm_status_string.argtypes = [st]
    L.bsmm_status_string.restype = ctypes.c_char_p
    L.bsmm_last_error.restype = ctypes.c_char_p
    L.bsmm_version.restype = st
    L.bsmm_timing_enable.argtypes = [ctypes.c_int]
    L.bsmm_timing_enable.restype = st
    L.bsmm_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64),
                                   ctypes.c_char_p, sz]
    L.bsmm_timing_read.restype = st
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise BsmmError(status, load().bsmm_last_error().decode())


# ----------------------------------------------------------------- helpers --

def _torch():
    import torch
    return torch


_RAW_STREAM = []


def _stream(stream):
    """The HIP stream handle of ``stream``, or of the current stream of the
    current device (read without building a Stream object: the per-call
    host cost matters for decode-sized calls)."""
    torch = _torch()
    if stream is not None:
        return stream.cuda_stream
    if not _RAW_STREAM:
        _RAW_STREAM.append(getattr(torch._C, "_cuda_getCurrentRawStream", None))
    raw = _RAW_STREAM[0]
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


_WS = {}          # workspace buffer per (device, stream handle)
_WS_NEED = {}     # workspace bytes per (op, G, M, N, K, out dtype); cleared by the override


def _workspace(op, G, M, N, K, out_dtype, device, stream, handle):
    """Workspace for the fastest plan, cached per (device, stream) and grown
    when a call needs more.  Calls on one stream run in order, so they may
    share a buffer; calls on different streams get different buffers.  A
    buffer is allocated while its stream is current, so the caching
    allocator hands its memory to no other stream before the work queued on
    that stream has finished, even once the buffer is replaced by a larger
    one."""
    key = (op, G, M, N, K, out_dtype)
    need = _WS_NEED.get(key)
    if need is None:
        need = load().bsmm_workspace_bytes(op, G, M, N, K, out_dtype)
        _WS_NEED[key] = need
    if need == 0:
        return None, 0
    wkey = (device, handle)
    buf = _WS.get(wkey)
    if buf is None or buf.numel() < need:
        torch = _torch()
        if stream is None:
            buf = torch.empty(need, dtype=torch.uint8, device=device)
        else:
            with torch.cuda.stream(stream):
                buf = torch.empty(need, dtype=torch.uint8, device=device)
        _WS[wkey] = buf
    return buf, buf.numel()


def _dtype_code(dt):
    torch = _torch()
    if isinstance(dt, int) and not isinstance(dt, bool) and dt in (I32, F32, BF16, E4M3):
        return dt
    if dt in (torch.int32, "i32"):
        return I32
    if dt in (torch.float32, "f32"):
        return F32
    if dt in (torch.bfloat16, "bf16"):
        return BF16
    if dt in (torch.float8_e4m3fn, "e4m3"):
        return E4M3
    raise ValueError(f"unsupported output dtype {dt}")


def _torch_dtype(code):
    torch = _torch()
    return {I32: torch.int32, F32: torch.float32, BF16: torch.bfloat16,
            E4M3: torch.float8_e4m3fn}[code]


def _bytes_view(t, name):
    torch = _torch()
    if t.dtype in (torch.int8, torch.uint8):
        return t
    if t.dtype in (torch.float8_e4m3fn, torch.float8_e8m0fnu):
        return t.view(torch.uint8)
    raise ValueError(f"{name}: expected 1-byte codes, got {t.dtype}")


def _out(out, shape, code, device):
    torch = _torch()
    dt = _torch_dtype(code)
    if out is None:
        return torch.empty(shape, dtype=dt, device=device)
    if tuple(out.shape) != tuple(shape) or out.dtype != dt:
        raise ValueError(f"out must be {tuple(shape)} {dt}, got {tuple(out.shape)} {out.dtype}")
    return out


def _ws_args(workspace, op, G, M, N, K, code, device, stream, handle):
    if workspace is False:
        return None, 0
    if workspace is None:
        buf, n = _workspace(op, G, M, N, K, code, device, stream, handle)
        return (buf.data_ptr() if buf is not None else None), n
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


# ------------------------------------------------------------ entry points --

def bsmm_int8_rowwise(a, b, scale_a=None, scale_b=None, *, out_dtype="bf16",
                      out=None, workspace=None, stream=None):
    """int8 rowwise scaled matmul.

    a: int8 [M, K] with unit stride along K.  b: int8 [K, N] column-major
    (b.stride(0) == 1), e.g. ``b_nk.t()``.  scale_a: fp32 [M, 1] / [M] or a
    0-d scalar (tensorwise); scale_b: fp32 [1, N] / [N] or 0-d.  out_dtype
    "i32" returns the raw int32 accumulators and ignores the scales.
    """
    torch = _torch()
    code = _dtype_code(out_dtype)
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if a.dtype != torch.int8 or b.dtype != torch.int8:
        raise ValueError("a and b must be int8")
    if K and a.stride(1) != 1:
        raise ValueError(f"a must be row-major, got stride {a.stride()}")
    if K and b.stride(0) != 1:
        raise ValueError(f"b must be column-major, got stride {b.stride()}")
    sa_m = sb_n = 0
    if code != I32:
        if scale_a is None or scale_b is None:
            raise ValueError("scale_a and scale_b are required unless out_dtype is int32")
        if scale_a.dtype != torch.float32 or scale_b.dtype != torch.float32:
            raise ValueError("scales must be fp32")
        if scale_a.dim() == 0 and scale_b.dim() == 0:
            pass                                     # tensorwise
        elif (tuple(scale_a.shape) in ((M, 1), (M,)) and tuple(scale_b.shape) in ((1, N), (N,))):
            sa_m = scale_a.stride(0)
            sb_n = scale_b.stride(-1)
        else:
            raise ValueError(
                "Invalid scaling configuration. For tensorwise scaling, both scales "
                f"should be scalar. For rowwise scaling, scale_a should be ({M}, 1), "
                f"scale_b should be (1, {N}). Got scale_a.size()={tuple(scale_a.shape)} "
                f"and scale_b.size()={tuple(scale_b.shape)}")
    o = _out(out, (M, N), code, a.device)
    hs = _stream(stream)
    wsp, wsn = _ws_args(workspace, OP_INT8_ROWWISE, 1, M, N, K, code, a.device, stream, hs)
    _check(load().bsmm_int8_rowwise(
        a.data_ptr(), a.stride(0), b.data_ptr(), b.stride(1),
        scale_a.data_ptr() if scale_a is not None else None, sa_m,
        scale_b.data_ptr() if scale_b is not None else None, sb_n,
        o.data_ptr(), o.stride(0), code, M, N, K, wsp, wsn, hs))
    return o


def bsmm_fp8_blockwise(a, b, scale_a, scale_b, *, out_dtype="bf16", out=None,
                       workspace=None, stream=None):
    """fp8 E4M3 blockwise scaled matmul.

    a: [M, K] E4M3 codes (float8_e4m3fn or uint8), row-major.  b: [K, N]
    column-major.  scale_a: fp32 [M, K/128]; scale_b: fp32 [K/128, N/128]
    (any strides).
    """
    torch = _torch()
    code = _dtype_code(out_dtype)
    a8, b8 = _bytes_view(a, "a"), _bytes_view(b, "b")
    M, K = a8.shape
    K2, N = b8.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if K and a8.stride(1) != 1:
        raise ValueError(f"a must be row-major, got stride {a8.stride()}")
    if K and b8.stride(0) != 1:
        raise ValueError(f"b must be column-major, got stride {b8.stride()}")
    KB, NB = -(-K // 128), -(-N // 128)
    if scale_a.dtype != torch.float32 or scale_b.dtype != torch.float32:
        raise ValueError("blockwise scales must be fp32")
    if tuple(scale_a.shape) != (M, KB) or tuple(scale_b.shape) != (KB, NB):
        raise ValueError(
            "Invalid scaling configuration. For blockwise scaling, scale_a should be "
            f"({M}, {KB}) and scale_b should be ({KB}, {NB}). Got "
            f"scale_a.size()={tuple(scale_a.shape)} and scale_b.size()={tuple(scale_b.shape)}")
    o = _out(out, (M, N), code, a8.device)
    hs = _stream(stream)
    wsp, wsn = _ws_args(workspace, OP_FP8_BLOCKWISE, 1, M, N, K, code, a8.device, stream, hs)
    _check(load().bsmm_fp8_blockwise(
        a8.data_ptr(), a8.stride(0), b8.data_ptr(), b8.stride(1),
        scale_a.data_ptr(), scale_a.stride(0), scale_a.stride(1),
        scale_b.data_ptr(), scale_b.stride(0), scale_b.stride(1),
        o.data_ptr(), o.stride(0), code, M, N, K, wsp, wsn, hs))
    return o


def bsmm_fp8_blockwise_scratch(a, b, scale_a, scale_b, *, out_dtype="bf16", out=None,
                               stream=None):
    """bsmm_fp8_blockwise with the library's static device scratch as its
    workspace: the library allocates nothing (pass ``out`` to allocate
    nothing here either).  Same arguments and results; problems whose plan
    needs more than the scratch holds raise BsmmError (BSMM_ERR_UNSUPPORTED).
    Calls that overlap on one GPU race on its scratch."""
    torch = _torch()
    code = _dtype_code(out_dtype)
    a8, b8 = _bytes_view(a, "a"), _bytes_view(b, "b")
    M, K = a8.shape
    K2, N = b8.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if K and a8.stride(1) != 1:
        raise ValueError(f"a must be row-major, got stride {a8.stride()}")
    if K and b8.stride(0) != 1:
        raise ValueError(f"b must be column-major, got stride {b8.stride()}")
    KB, NB = -(-K // 128), -(-N // 128)
    if scale_a.dtype != torch.float32 or scale_b.dtype != torch.float32:
        raise ValueError("blockwise scales must be fp32")
    if tuple(scale_a.shape) != (M, KB) or tuple(scale_b.shape) != (KB, NB):
        raise ValueError(
            "Invalid scaling configuration. For blockwise scaling, scale_a should be "
            f"({M}, {KB}) and scale_b should be ({KB}, {NB}). Got "
            f"scale_a.size()={tuple(scale_a.shape)} and scale_b.size()={tuple(scale_b.shape)}")
    o = _out(out, (M, N), code, a8.device)
    _check(load().bsmm_fp8_blockwise_scratch(
        a8.data_ptr(), a8.stride(0), b8.data_ptr(), b8.stride(1),
        scale_a.data_ptr(), scale_a.stride(0), scale_a.stride(1),
        scale_b.data_ptr(), scale_b.stride(0), scale_b.stride(1),
        o.data_ptr(), o.stride(0), code, M, N, K, _stream(stream)))
    return o


def bsmm_fp8_groupwise(a, b, scale_a, scale_b, *, out_dtype="bf16", out=None,
                       workspace=None, stream=None):
    """fp8 E4M3 matmul with 1 x 128 groups on both operands (the weight
    gradient of a blockwise fp8 linear layer).

    a: [M, K] E4M3 codes, row-major.  b: [K, N] column-major.  scale_a: fp32
    [M, K/128] (per row of a and K block); scale_b: fp32 [K/128, N] (per K
    block and column of b); any strides.  The call needs a workspace (the
    default allocates one); ``workspace=False`` is rejected by the library.
    """
    torch = _torch()
    code = _dtype_code(out_dtype)
    a8, b8 = _bytes_view(a, "a"), _bytes_view(b, "b")
    M, K = a8.shape
    K2, N = b8.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if K and a8.stride(1) != 1:
        raise ValueError(f"a must be row-major, got stride {a8.stride()}")
    if K and b8.stride(0) != 1:
        raise ValueError(f"b must be column-major, got stride {b8.stride()}")
    KB = -(-K // 128)
    if scale_a.dtype != torch.float32 or scale_b.dtype != torch.float32:
        raise ValueError("groupwise scales must be fp32")
    if tuple(scale_a.shape) != (M, KB) or tuple(scale_b.shape) != (KB, N):
        raise ValueError(
            "Invalid scaling configuration. For groupwise (1x128 x 128x1) scaling, scale_a "
            f"should be ({M}, {KB}) and scale_b should be ({KB}, {N}). Got "
            f"scale_a.size()={tuple(scale_a.shape)} and scale_b.size()={tuple(scale_b.shape)}")
    o = _out(out, (M, N), code, a8.device)
    hs = _stream(stream)
    wsp, wsn = _ws_args(workspace, OP_FP8_GROUPWISE, 1, M, N, K, code, a8.device, stream, hs)
    _check(load().bsmm_fp8_groupwise(
        a8.data_ptr(), a8.stride(0), b8.data_ptr(), b8.stride(1),
        scale_a.data_ptr(), scale_a.stride(0), scale_a.stride(1),
        scale_b.data_ptr(), scale_b.stride(0), scale_b.stride(1),
        o.data_ptr(), o.stride(0), code, M, N, K, wsp, wsn, hs))
    return o


def bsmm_fp8_mx_bmm(x, w, x_scale, w_scale, *, layout="m_major", out_dtype="bf16",
                    out=None, workspace=None, stream=None):
    """fp8 E4M3 batched matmul with e8m0 per-128-K-block scales.

    layout "m_major": x [M, G, K], x_scale [M, G, K/128], out [M, G, N].
    layout "batch_first": x [G, M, K], x_scale [G, M, K/128], out [G, M, N].
    w [G, N, K] and w_scale [G, N/128, K/128] in both.  Arbitrary strides
    with unit stride along K.
    """
    code = _dtype_code(out_dtype)
    x8, w8 = _bytes_view(x, "x"), _bytes_view(w, "w")
    xs8, ws8 = _bytes_view(x_scale, "x_scale"), _bytes_view(w_scale, "w_scale")
    if x8.dim() != 3 or w8.dim() != 3:
        raise ValueError("x and w must be 3-D")
    if layout == "m_major":
        M, G, K = x8.shape
        x_sg, x_sm = x8.stride(1), x8.stride(0)
    elif layout == "batch_first":
        G, M, K = x8.shape
        x_sg, x_sm = x8.stride(0), x8.stride(1)
    else:
        raise ValueError(f"unknown layout {layout}")
    G2, N, K2 = w8.shape
    if G2 != G or K2 != K:
        raise ValueError(f"x {tuple(x8.shape)} and w {tuple(w8.shape)} disagree")
    if K and (x8.stride(2) != 1 or w8.stride(2) != 1):
        raise ValueError("x and w must be contiguous along K")
    KB, NB = -(-K // 128), -(-N // 128)
    want_xs = (M, G, KB) if layout == "m_major" else (G, M, KB)
    if tuple(xs8.shape) != want_xs or tuple(ws8.shape) != (G, NB, KB):
        raise ValueError(
            f"Invalid scaling configuration. For mxscale BMM ({layout}), x_scale should be "
            f"{want_xs} and w_scale should be {(G, NB, KB)}. Got x_scale.size()="
            f"{tuple(xs8.shape)} and w_scale.size()={tuple(ws8.shape)}")
    if KB and (xs8.stride(2) != 1 or ws8.stride(2) != 1):
        raise ValueError("scales must be contiguous along K/128")
    if layout == "m_major":
        xs_sg, xs_sm = xs8.stride(1), xs8.stride(0)
        oshape = (M, G, N)
    else:
        xs_sg, xs_sm = xs8.stride(0), xs8.stride(1)
        oshape = (G, M, N)
    o = _out(out, oshape, code, x8.device)
    if layout == "m_major":
        o_sg, o_sm = o.stride(1), o.stride(0)
    else:
        o_sg, o_sm = o.stride(0), o.stride(1)
    if o.stride(2) != 1:
        raise ValueError("out must be contiguous along N")
    hs = _stream(stream)
    wsp, wsn = _ws_args(workspace, OP_FP8_MX_BMM, G, M, N, K, code, x8.device, stream, hs)
    _check(load().bsmm_fp8_mx_bmm(
        x8.data_ptr(), x_sg, x_sm, w8.data_ptr(), w8.stride(0), w8.stride(1),
        xs8.data_ptr(), xs_sg, xs_sm, ws8.data_ptr(), ws8.stride(0), ws8.stride(1),
        o.data_ptr(), o_sg, o_sm, code, G, M, N, K, wsp, wsn, hs))
    return o


def bsmm_fp8_scaled_mm(a, b, scale_a, scale_b, *, bias=None, scale_result=None,
                       out_dtype="bf16", out=None, workspace=None, stream=None):
    """fp8 E4M3 scaled matmul with tensorwise or rowwise fp32 scales.

    a: [M, K] E4M3 codes, row-major; b: [K, N] column-major.  Tensorwise:
    scale_a and scale_b one element each (shape () or (1, 1)); rowwise:
    scale_a (M, 1), scale_b (1, N).  bias: optional [N] fp32 or bf16.
    scale_result: optional one-element fp32 tensor (or a float).  out_dtype:
    "f32", "bf16" or "e4m3" (torch.float8_e4m3fn).
    """
    torch = _torch()
    code = _dtype_code(out_dtype)
    if code == I32:
        raise ValueError("fp8 scaled_mm writes f32, bf16 or e4m3")
    a8, b8 = _bytes_view(a, "a"), _bytes_view(b, "b")
    M, K = a8.shape
    K2, N = b8.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if K and a8.stride(1) != 1:
        raise ValueError(f"a must be row-major, got stride {a8.stride()}")
    if K and b8.stride(0) != 1:
        raise ValueError(f"b must be column-major, got stride {b8.stride()}")
    if scale_a.dtype != torch.float32 or scale_b.dtype != torch.float32:
        raise ValueError("scale_a and scale_b must be fp32")
    if scale_a.numel() == 1 and scale_b.numel() == 1:      # tensorwise: one value each
        sa_m, sb_n = 0, 0
    elif tuple(scale_a.shape) == (M, 1) and tuple(scale_b.shape) == (1, N):
        sa_m, sb_n = scale_a.stride(0), scale_b.stride(1)
    else:
        raise ValueError(
            f"scale shapes: tensorwise takes two scalars, rowwise scale_a ({M}, 1) and "
            f"scale_b (1, {N}); got {tuple(scale_a.shape)} and {tuple(scale_b.shape)}")
    bias_ptr, bias_code = None, F32
    if bias is not None:
        if bias.dtype not in (torch.float32, torch.bfloat16) or bias.dim() != 1 or \
                bias.shape[0] != N or (N and bias.stride(0) != 1):
            raise ValueError(f"bias must be a contiguous [N={N}] fp32 or bf16 tensor")
        bias_ptr, bias_code = bias.data_ptr(), _dtype_code(bias.dtype)
    sr_ptr = None
    if scale_result is not None:
        if not isinstance(scale_result, torch.Tensor):
            scale_result = torch.tensor([float(scale_result)], dtype=torch.float32,
                                        device=a8.device)
        if scale_result.dtype != torch.float32 or scale_result.numel() != 1:
            raise ValueError("scale_result must be one fp32 value")
        sr_ptr = scale_result.data_ptr()
    o = _out(out, (M, N), code, a8.device)
    o8 = o.view(torch.uint8) if code == E4M3 else o
    hs = _stream(stream)
    wsp, wsn = _ws_args(workspace, OP_FP8_SCALED_MM, 1, M, N, K, code, a8.device, stream, hs)
    _check(load().bsmm_fp8_scaled_mm(
        a8.data_ptr(), a8.stride(0), b8.data_ptr(), b8.stride(1),
        scale_a.data_ptr(), sa_m, scale_b.data_ptr(), sb_n, bias_ptr, bias_code, sr_ptr,
        o8.data_ptr(), o.stride(0), code, M, N, K, wsp, wsn, hs))
    return o


def bsmm_fp8_mx32_mm(a, b, a_scale, b_scale, *, out_dtype="bf16", out=None, workspace=None,
                     stream=None):
    """fp8 E4M3 matmul with e8m0 scales on 32-element K blocks (MX).

    a: [M, K] E4M3 codes, row-major; b: [K, N] column-major; a_scale
    [M, K/32] and b_scale [N, K/32] e8m0 bytes (uint8 or float8_e8m0fnu)
    with contiguous rows.
    """
    code = _dtype_code(out_dtype)
    if code not in (F32, BF16):
        raise ValueError("fp8 mx32 writes f32 or bf16")
    a8, b8 = _bytes_view(a, "a"), _bytes_view(b, "b")
    sa8, sb8 = _bytes_view(a_scale, "a_scale"), _bytes_view(b_scale, "b_scale")
    M, K = a8.shape
    K2, N = b8.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if K and a8.stride(1) != 1:
        raise ValueError(f"a must be row-major, got stride {a8.stride()}")
    if K and b8.stride(0) != 1:
        raise ValueError(f"b must be column-major, got stride {b8.stride()}")
    KC = -(-K // 32)
    if tuple(sa8.shape) != (M, KC) or tuple(sb8.shape) != (N, KC):
        raise ValueError(f"MX scales: a_scale should be ({M}, {KC}) and b_scale ({N}, {KC}); "
                         f"got {tuple(sa8.shape)} and {tuple(sb8.shape)}")
    if KC and (sa8.stride(1) != 1 or sb8.stride(1) != 1):
        raise ValueError("scale rows must be contiguous")
    o = _out(out, (M, N), code, a8.device)
    hs = _stream(stream)
    wsp, wsn = _ws_args(workspace, OP_FP8_MX32_MM, 1, M, N, K, code, a8.device, stream, hs)
    _check(load().bsmm_fp8_mx32_mm(
        a8.data_ptr(), a8.stride(0), b8.data_ptr(), b8.stride(1),
        sa8.data_ptr(), sa8.stride(0), sb8.data_ptr(), sb8.stride(0),
        o.data_ptr(), o.stride(0), code, M, N, K, wsp, wsn, hs))
    return o


def _quant_input(x, name="x"):
    """A bf16 / fp32 tensor as rows of K: (rows view, input dtype code)."""
    torch = _torch()
    if x.dtype == torch.bfloat16:
        code = BF16
    elif x.dtype == torch.float32:
        code = F32
    else:
        raise ValueError(f"{name}: expected bf16 or fp32, got {x.dtype}")
    if x.dim() < 2:
        raise ValueError(f"{name} must have at least 2 dimensions")
    K = x.shape[-1]
    if K and x.stride(-1) != 1:
        raise ValueError(f"{name} must be contiguous along its last dimension")
    if x.dim() == 2:
        return x, code
    if K == 0:
        n = 1
        for d in x.shape[:-1]:
            n *= d
        return x.new_empty((n, 0)), code
    try:
        rows = x.view(-1, K)
    except RuntimeError as e:
        raise ValueError(f"{name}: leading dimensions do not form rows of one stride") from e
    return rows, code


def _quant_out(t, shape, dtype, name, device):
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")
    return t


def bsmm_quant_int8_rowwise(x, *, q=None, scale=None, stream=None):
    """Per-row symmetric int8 quantisation of x [M, K] (bf16 or fp32).

    Returns (q int8 [M, K], scale fp32 [M, 1]) with x ~ q * scale: the
    operand and scale_a of bsmm_int8_rowwise.
    """
    torch = _torch()
    x2, code = _quant_input(x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x2.shape
    q = _quant_out(q, (M, K), torch.int8, "q", x.device)
    scale = _quant_out(scale, (M, 1), torch.float32, "scale", x.device)
    if K and q.stride(1) != 1:
        raise ValueError("q must be row-major")
    _check(load().bsmm_quant_int8_rowwise(
        x2.data_ptr(), x2.stride(0), code, q.data_ptr(), q.stride(0),
        scale.data_ptr(), scale.stride(0), M, K, _stream(stream)))
    return q, scale


def bsmm_quant_fp8_blockwise(x, *, q=None, scale=None, stream=None):
    """fp8 E4M3 quantisation of x [M, K] with one fp32 scale per 1 x 128 block.

    Returns (q float8_e4m3fn [M, K], scale fp32 [M, K/128]); a given
    ``scale`` may have any strides (e.g. the column-major transpose).
    """
    torch = _torch()
    x2, code = _quant_input(x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x2.shape
    KB = K // 128
    q = _quant_out(q, (M, K), torch.float8_e4m3fn, "q", x.device)
    scale = _quant_out(scale, (M, KB), torch.float32, "scale", x.device)
    if K and q.stride(1) != 1:
        raise ValueError("q must be row-major")
    q8 = q.view(torch.uint8)
    _check(load().bsmm_quant_fp8_blockwise(
        x2.data_ptr(), x2.stride(0), code, q8.data_ptr(), q8.stride(0),
        scale.data_ptr(), scale.stride(0), scale.stride(1), M, K, _stream(stream)))
    return q, scale


def bsmm_quant_fp8_columns(x, *, q_t=None, scale=None, stream=None):
    """fp8 E4M3 quantisation of x [R, C] (bf16 or fp32; R a multiple of 128,
    C of 8) in groups of 128 consecutive rows of one column, one fp32 scale
    each: the operands of the weight-gradient GEMM bsmm_fp8_groupwise, which
    contracts over the R tokens.

    Returns (q_t float8_e4m3fn [C, R], the codes transposed, and scale fp32
    [R/128, C]).  With dY [R, N] and X [R, K] quantised this way,
    ``bsmm_fp8_groupwise(dYq_t, Xq_t.t(), s_dy.t(), s_x)`` is dW [N, K].
    """
    torch = _torch()
    x2, code = _quant_input(x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [R, C]")
    R, C = x2.shape
    q_t = _quant_out(q_t, (C, R), torch.float8_e4m3fn, "q_t", x.device)
    scale = _quant_out(scale, (R // 128, C), torch.float32, "scale", x.device)
    if R and q_t.stride(1) != 1:
        raise ValueError("q_t must be row-major")
    q8 = q_t.view(torch.uint8)
    _check(load().bsmm_quant_fp8_columns(
        x2.data_ptr(), x2.stride(0), code, q8.data_ptr(), q8.stride(0),
        scale.data_ptr(), scale.stride(0), scale.stride(1), R, C, _stream(stream)))
    return q_t, scale


def bsmm_quant_fp8_blockwise_columns(x, *, q=None, scale=None, q_t=None, scale_t=None,
                                     stream=None):
    """Both fp8 quantisations of a layer input x [R, C] (bf16 or fp32; R and C
    multiples of 128) from one read of x: the 1 x 128 row blocks of
    bsmm_quant_fp8_blockwise (the forward GEMM's A) and the groups of 128
    rows down the columns of bsmm_quant_fp8_columns (the weight gradient's
    operand).  Bit-identical to the two separate calls.

    Returns (q float8_e4m3fn [R, C], scale fp32 [R, C/128], q_t
    float8_e4m3fn [C, R], scale_t fp32 [R/128, C]).  Unless given, ``scale``
    is allocated column-major (strides (1, R)): the kernel writes one
    128-column block of every row per tile, which is then one contiguous
    run; bsmm_fp8_blockwise takes scale_a with any strides.
    """
    torch = _torch()
    x2, code = _quant_input(x)
    if x.dim() != 2:
        raise ValueError("x must be 2-D [R, C]")
    R, C = x2.shape
    q = _quant_out(q, (R, C), torch.float8_e4m3fn, "q", x.device)
    if scale is None:
        scale = torch.empty((C // 128, R), dtype=torch.float32, device=x.device).t()
    scale = _quant_out(scale, (R, C // 128), torch.float32, "scale", x.device)
    q_t = _quant_out(q_t, (C, R), torch.float8_e4m3fn, "q_t", x.device)
    scale_t = _quant_out(scale_t, (R // 128, C), torch.float32, "scale_t", x.device)
    for t, n in ((q, "q"), (q_t, "q_t")):
        if t.numel() and t.stride(1) != 1:
            raise ValueError(f"{n} must be row-major")
    qv, qtv = q.view(torch.uint8), q_t.view(torch.uint8)
    _check(load().bsmm_quant_fp8_blockwise_columns(
        x2.data_ptr(), x2.stride(0), code, qv.data_ptr(), qv.stride(0),
        scale.data_ptr(), scale.stride(0), scale.stride(1), qtv.data_ptr(), qtv.stride(0),
        scale_t.data_ptr(), scale_t.stride(0), scale_t.stride(1), R, C, _stream(stream)))
    return q, scale, q_t, scale_t


def bsmm_quant_fp8_weight(w, *, plain=True, transposed=True, q=None, q_t=None, scale=None,
                          stream=None):
    """fp8 E4M3 quantisation of a weight w [R, C] (bf16 or fp32; R and C
    multiples of 128) in 128 x 128 blocks, one fp32 scale each.

    Returns (q [R, C] or None, q_t [C, R] or None, scale fp32 [R/128, C/128]):
    the codes as they are (the forward GEMM's B = ``q.t()`` with scale_b
    ``scale.t()``) and transposed (the input gradient's B = ``q_t.t()`` with
    scale_b ``scale``).
    """
    torch = _torch()
    if not (plain or transposed):
        raise ValueError("ask for the plain or the transposed codes (or both)")
    w2, code = _quant_input(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [R, C]")
    R, C = w2.shape
    q = _quant_out(q, (R, C), torch.float8_e4m3fn, "q", w.device) if plain else None
    q_t = _quant_out(q_t, (C, R), torch.float8_e4m3fn, "q_t", w.device) if transposed else None
    scale = _quant_out(scale, (R // 128, C // 128), torch.float32, "scale", w.device)
    for t, n in ((q, "q"), (q_t, "q_t")):
        if t is not None and t.numel() and t.stride(1) != 1:
            raise ValueError(f"{n} must be row-major")
    qv = q.view(torch.uint8) if q is not None else None
    qtv = q_t.view(torch.uint8) if q_t is not None else None
    _check(load().bsmm_quant_fp8_weight(
        w2.data_ptr(), w2.stride(0), code,
        qv.data_ptr() if qv is not None else None, qv.stride(0) if qv is not None else 0,
        qtv.data_ptr() if qtv is not None else None, qtv.stride(0) if qtv is not None else 0,
        scale.data_ptr(), scale.stride(0), scale.stride(1), R, C, _stream(stream)))
    return q, q_t, scale


def bsmm_quant_fp8_mx(x, *, block=128, q=None, scale=None, stream=None):
    """fp8 E4M3 quantisation with an e8m0 scale per 1 x ``block`` block
    (128, or 32 for bsmm_fp8_mx32_mm) along the last dimension of x [..., K]
    (bf16 or fp32), e.g. the BMM's x [M, G, K] or [G, M, K].

    Returns (q float8_e4m3fn [..., K], scale uint8 e8m0 bytes
    [..., K/block]): the x and x_scale of bsmm_fp8_mx_bmm, or (block 32) an
    operand and its scales for bsmm_fp8_mx32_mm.
    """
    torch = _torch()
    if block not in (32, 128):
        raise ValueError("block must be 32 or 128")
    x2, code = _quant_input(x)
    K = x.shape[-1]
    lead = tuple(x.shape[:-1])
    q = _quant_out(q, lead + (K,), torch.float8_e4m3fn, "q", x.device)
    scale = _quant_out(scale, lead + (K // block,), torch.uint8, "scale", x.device)
    if not q.is_contiguous() or not scale.is_contiguous():
        raise ValueError("q and scale must be contiguous")
    q8 = q.view(torch.uint8).view(-1, K) if K else q.view(torch.uint8)
    M = x2.shape[0]
    fn = load().bsmm_quant_fp8_mx if block == 128 else load().bsmm_quant_fp8_mx32
    _check(fn(x2.data_ptr(), x2.stride(0), code, q8.data_ptr(), K,
              scale.data_ptr(), K // block, 1, M, K, _stream(stream)))
    return q, scale


def bsmm_workspace_bytes(op, G, M, N, K, out_dtype):
    return load().bsmm_workspace_bytes(op, G, M, N, K, _dtype_code(out_dtype))


def bsmm_query_plan(op, G, M, N, K, out_dtype, workspace_bytes=2**62):
    info = PlanInfo()
    _check(load().bsmm_query_plan(op, G, M, N, K, _dtype_code(out_dtype),
                                  workspace_bytes, ctypes.byref(info)))
    return {"variant": info.variant.decode(), "tile_m": info.tile_m,
            "tile_n": info.tile_n, "split_k": info.split_k, "m_split": info.m_split,
            "workspace": info.workspace, "source": info.source,
            "tail_variant": info.tail_variant.decode(), "tail_split_k": info.tail_split_k}


def bsmm_set_override(variant=None, split_k=0):
    _WS_NEED.clear()              # the plans, and so their workspace, change
    _check(load().bsmm_set_override(variant.encode() if variant else None, split_k))


def bsmm_set_override_tail(m_split=0, tail_variant=None, tail_split=1):
    """Force an M-split (bulk rows [0, m_split), a tail launch of
    `tail_variant` with `tail_split` K slices) for the following calls;
    m_split 0 removes it (tests and tuning)."""
    _WS_NEED.clear()
    _check(load().bsmm_set_override_tail(int(m_split),
                                         tail_variant.encode() if tail_variant else None,
                                         int(tail_split)))


def bsmm_set_streamk_grid(workgroups=0):
    """Grid of the stream-K kernels for the following calls (0: as many
    workgroups as the device holds at once; tests and tuning)."""
    _WS_NEED.clear()
    _check(load().bsmm_set_streamk_grid(int(workgroups)))


def bsmm_mfma_probe(kind, workgroups, iters, out, stream=None):
    """Matrix-core throughput probe (kind 0: fp8 16x16x128, 1: int8
    16x16x64, 2: int8 32x32x32, 3: fp8 32x32x64); out: fp32 device tensor of
    workgroups * 256 elements.
    Returns the number of flops (ops) the launch performs."""
    if out.numel() < workgroups * 256:
        raise ValueError("out holds fewer than workgroups * 256 floats")
    _check(load().bsmm_mfma_probe(int(kind), int(workgroups), int(iters), out.data_ptr(),
                                  _stream(stream)))
    per = {0: 65536, 1: 32768, 2: 65536, 3: 131072}[kind]
    return float(workgroups) * 4 * iters * 8 * per


def bsmm_timing_enable(enable=True):
    """Time the main launch of every following call with HIP events."""
    _check(load().bsmm_timing_enable(1 if enable else 0))


def bsmm_timing_read():
    """(mean ms, launches, variant) of the launches timed since enabling."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    name = ctypes.create_string_buffer(64)
    _check(load().bsmm_timing_read(ctypes.byref(ms), ctypes.byref(n), name, 64))
    return ms.value, n.value, name.value.decode()


def bsmm_variant_names():
    return load().bsmm_variant_names().decode().split(",")


def bsmm_version():
    return load().bsmm_version()
