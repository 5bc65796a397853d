"""The allocation-free entry point bsmm_fp8_blockwise_scratch against the
workspace entry point bsmm_fp8_blockwise (GPU): two calls in a row, the
second smaller, each bit-identical to the workspace entry's result (the same
plan runs, with the static scratch as its workspace) and within the fp8 bar
of the oracle.  Both plans use the scratch: the first packs scale_a and runs
a split-K tail launch, the second splits K."""

import numpy as np
import pytest
import torch

import block_scaled_precision_gemm_amd as bsmm
from oracle import scaled_mm as S
from synth import fp8_blockwise_inputs
from tests.gpu_util import DEV, as_f64, dev, host_out, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_scratch_entry_matches_the_workspace_entry(out_dtype):
    for M, N, K, seed, rows in ((16534, 1024, 2048, 801, np.r_[0:8, 16380:16390, 16526:16534]),
                                (300, 384, 1024, 802, None)):
        need = bsmm.bsmm_workspace_bytes(bsmm.OP_FP8_BLOCKWISE, 1, M, N, K, out_dtype)
        assert 0 < need <= 64 << 20
        p = fp8_blockwise_inputs(M, N, K, seed)
        a, b = dev(p["a"]), dev(p["b_nk"]).t()
        sa, sb = dev(p["scale_a"]), dev(p["scale_b"])
        tdt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
        out = torch.full((M, N), 3.0, dtype=tdt, device=DEV)
        say(f"scratch entry {M}x{N}x{K} {out_dtype} (needs {need} bytes)")
        bsmm.bsmm_fp8_blockwise_scratch(a, b, sa, sb, out_dtype=out_dtype, out=out)
        ref = bsmm.bsmm_fp8_blockwise(a, b, sa, sb, out_dtype=out_dtype)
        got, want = host_out(out), host_out(ref)
        assert np.array_equal(got.view(np.uint16 if out_dtype == "bf16" else np.uint32),
                              want.view(np.uint16 if out_dtype == "bf16" else np.uint32))
        res = S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], out_dtype,
                              rows=rows)
        rep = S.compare(as_f64(got if rows is None else got[rows]), res)
        assert rep["ok"], rep
