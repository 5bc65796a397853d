"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (the dispatcher's own plan, with workspace).  The GPU computes
the whole output; the oracle computes sampled rows (all columns) one by one:
the first and last rows, the rows of a ragged tail, and random rows.

Workloads (``synth.CONFIGS``): int8 tiny 64x256x128; int8 dynamic-quant linear
8192x4096x4096; fp8 blockwise 16640x8192x5120; fp8 mx BMM m-major G=8 N=1024
K=4096 at M = 1, 128, 8192; fp8 mx BMM batch-first G=2 M=9000 N=2048 K=7168
with student-t values.
"""

import numpy as np
import pytest

from oracle import scaled_mm as S
from synth import CONFIGS, config_inputs
from tests.gpu_util import (check_blockwise, check_int8, check_mx, check_within, host_out,
                            run_blockwise, run_int8, run_mx, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _lib(gpu_lib):
    yield


def sample_rows(M, seed, n_random=24, tail_from=None, per_tile=256):
    """The first and last rows, one random row in every 256-row tile (so
    every tile row of every launch is sampled), rows spread over a ragged
    tail, and random rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(M, 4))) | set(range(max(0, M - 4), M))
    if tail_from is not None:
        rows |= set(range(tail_from, M, max(1, (M - tail_from) // 8)))
    for t0 in range(0, M, per_tile):
        rows.add(int(t0 + rng.integers(0, min(per_tile, M - t0))))
    rows |= set(rng.integers(0, M, n_random).tolist())
    return np.array(sorted(rows))


def test_c1_int8_tiny():
    p = config_inputs("c1")
    say("c1 int8 tiny (full oracle)")
    check_int8(p, "f32", run_int8(p, "f32"))
    check_int8(p, "i32", run_int8(p, "i32"))


def test_c2_int8_dynamic_quant():
    c = CONFIGS["c2"]
    p = config_inputs("c2")
    say("c2 int8 8192x4096x4096 bf16 + i32")
    rows = sample_rows(c["M"], 2)
    check_int8(p, "bf16", run_int8(p, "bf16"), rows=rows)
    check_int8(p, "i32", run_int8(p, "i32"), rows=rows)


def test_c3_fp8_blockwise():
    c = CONFIGS["c3"]
    p = config_inputs("c3")
    say("c3 fp8 blockwise 16640x8192x5120 bf16")
    y = run_blockwise(p, "bf16")
    rows = sample_rows(c["M"], 3, n_random=20, tail_from=16384)
    rep = check_blockwise(p, "bf16", y, rows=rows)
    res = S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], "bf16", rows=rows)
    say("c3", rep, check_within(host_out(y)[rows], res, c["K"] // 128))


@pytest.mark.parametrize("name", ["c4_m1", "c4_m128", "c4_m8192"])
def test_c4_mx_m_major(name):
    c = CONFIGS[name]
    p = config_inputs(name)
    say(f"{name} mx m-major G=8 M={c['M']} N=1024 K=4096 bf16")
    y = run_mx(p, "bf16")
    rows = None if c["M"] <= 128 else sample_rows(c["M"], 4)
    rep = check_mx(p, "bf16", y, rows=rows)
    res = S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], "m_major", "bf16", rows=rows)
    got = host_out(y) if rows is None else host_out(y)[rows]
    say(name, rep, check_within(got, res, c["K"] // 128))


def test_c5_mx_batch_first_tail():
    c = CONFIGS["c5"]
    p = config_inputs("c5")
    say("c5 mx batch-first G=2 M=9000 N=2048 K=7168 fp32 (t-distributed)")
    y = run_mx(p, "f32")
    rows = sample_rows(c["M"], 5, n_random=16, tail_from=8192)
    rep = check_mx(p, "f32", y, rows=rows)
    res = S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], "batch_first", "f32",
                       rows=rows)
    say("c5", rep, check_within(host_out(y)[:, rows], res, c["K"] // 128))
