"""Helpers for the GPU parity tests: move synthetic inputs to the device, call
the library through its binding, bring results back as numpy, and compare
with the oracle."""

import sys

import numpy as np
import torch

import block_scaled_precision_gemm_amd as bsmm
from oracle import scaled_mm as S
from oracle.formats import bf16_bits_to_f64

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host_out(t):
    """GPU output -> numpy in the oracle's representation (uint16 bf16 bits,
    float32, int32)."""
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(out_np):
    if out_np.dtype == np.uint16:
        return bf16_bits_to_f64(out_np)
    return out_np.astype(np.float64)


class Forced:
    """Force a kernel variant / split for the calls inside the block."""

    def __init__(self, variant=None, split=0):
        self.v, self.s = variant, split

    def __enter__(self):
        bsmm.bsmm_set_override(self.v, self.s)

    def __exit__(self, *exc):
        bsmm.bsmm_set_override(None, 0)


# ----------------------------------------------------------- int8 rowwise --

def run_int8(p, out_dtype, out=None):
    a = dev(p["a"])
    b = dev(p["b_nk"]).t()
    sa = dev(p["scale_a"]).reshape(-1, 1)
    sb = dev(p["scale_b"]).reshape(1, -1)
    return bsmm.bsmm_int8_rowwise(a, b, sa, sb, out_dtype=out_dtype, out=out)


def oracle_int8(p, out_dtype, rows=None):
    return S.int8_rowwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], out_dtype,
                          rows=rows)


def check_int8(p, out_dtype, y, rows=None):
    ref = oracle_int8(p, out_dtype, rows)
    got = host_out(y)
    if rows is not None:
        got = got[rows]
    rep = S.compare(got, ref, exact=True)
    assert rep["ok"], rep


# ---------------------------------------------------------- fp8 blockwise --

def run_blockwise(p, out_dtype, out=None):
    a = dev(p["a"])
    b = dev(p["b_nk"]).t()
    return bsmm.bsmm_fp8_blockwise(a, b, dev(p["scale_a"]), dev(p["scale_b"]),
                                   out_dtype=out_dtype, out=out)


def check_blockwise(p, out_dtype, y, rows=None, cols=None):
    ref = S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], out_dtype,
                          rows=rows, cols=cols)
    got = as_f64(host_out(y))
    if rows is not None:
        got = got[rows]
    if cols is not None:
        got = got[:, cols]
    rep = S.compare(got, ref)
    assert rep["ok"], rep
    return rep


# ------------------------------------------------------------------- mx --

def run_mx(p, out_dtype, out=None):
    return bsmm.bsmm_fp8_mx_bmm(dev(p["x"]), dev(p["w"]), dev(p["x_scale"]),
                                dev(p["w_scale"]), layout=p["layout"],
                                out_dtype=out_dtype, out=out)


def check_mx(p, out_dtype, y, rows=None, groups=None):
    ref = S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], p["layout"], out_dtype,
                       rows=rows, groups=groups)
    got = as_f64(host_out(y))
    if p["layout"] == "m_major":
        if rows is not None:
            got = got[rows]
        if groups is not None:
            got = got[:, groups]
    else:
        if groups is not None:
            got = got[groups]
        if rows is not None:
            got = got[:, rows]
    rep = S.compare(got, ref)
    assert rep["ok"], rep
    return rep


# ------------------------------------------------ fp32 accumulation bound --

def gamma_fp32(KB, adds=8):
    """Bound on |Y32 - C| / Bd for the fp8 kernels' binary32 result Y32 over
    KB blocks of 128 K (Bd = sum_k |a_deq| |b_deq|).

    Per block, the matrix instruction's partial.  Measured on gfx950 (see
    test_gpu_mfma_numerics.py): the instruction adds each group of 16
    products (in its own K order) with additions that drop the bits of the
    smaller operand below 2**-13 of the larger operand's binade (a term
    beside 448 keeps only whole multiples of 2**-5), and combines the group
    sums without that loss.  A group's 15 additions then lose less than
    15 * 2**-13 of the group's magnitude sum, and a block less than 2**-9 of
    its share of Bd.  Then per block: the binary32 scale product (2**-24,
    blockwise) and one rounded multiply-add or accumulation into a running
    sum that never exceeds Bd (2**-24).  ``adds`` more roundings cover the
    split-K / stream-K partial sums.  Valid while every scale product and
    partial stays in the binary32 normal range."""
    return 2.0**-9 + (KB + adds + 2) * 2.0**-24


def check_within(y_np, res, KB, adds=8):
    """The tight rule on an oracle Result (fp32 or bf16 bits)."""
    rep = S.compare_within(y_np, res, gamma_fp32(KB, adds))
    assert rep["ok"], rep
    return rep
