#!/usr/bin/env python3
"""Benchmark of the block-scaled matmul on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3]

A step is one call of the scaled matmul (validation, dispatch and every
kernel of the plan) on one batch of synthetic input that is already resident
in HBM.  About half a second of untimed calls lets the GPU clock settle, then
W untimed warm-up steps, then exactly K timed steps bracketed by device
synchronisation; HIP events on the stream the kernels are launched on time
every step.  Rank 0 prints one JSON line.

Default workload: the fp8 E4M3 blockwise GEMM M=16640, N=5120, K=8192 with
1x128 activation and 128x128 weight fp32 scales and bf16 output (the large
blockwise GEMM whose throughput is the headline target).  Other workloads:
--config c1 | c2 | c4_m1 | c4_m128 | c4_m8192 | c5.

The JSON line also carries
  roofline      achieved / peak for the dominant kernel (MFMA-bound shapes
                against the dense fp8 / int8 peak, HBM-bound shapes against
                8 TB/s), and the HBM traffic measured by rocprofv3 counters
                when a counter summary for the current kernel source exists
                under profiles/;
  cpu_baseline  the CPU oracle (numpy, fp64) timed on this host on a bounded
                sample of the same workload (a subset of output rows).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"fp8": 5.0e15, "int8": 5.0e15}    # MI355X dense MFMA, ops/s
HBM_PEAK = 8.0e12                          # bytes/s
KERNEL_SOURCES = ["block_scaled_precision_gemm_amd/csrc/bsmm_kernels.hip"]


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def describe(name, c):
    if c["op"] == "int8":
        return (f"int8 rowwise scaled GEMM M={c['M']} N={c['N']} K={c['K']}, "
                f"{c['kind']} inputs, {c['out']} out")
    if c["op"] == "fp8_blockwise":
        return (f"fp8 e4m3 blockwise GEMM M={c['M']} N={c['N']} K={c['K']}, 1x128 / "
                f"128x128 fp32 scales, {c['out']} out")
    return (f"fp8 e4m3 mxscale BMM {c['layout']} G={c['G']} M={c['M']} N={c['N']} "
            f"K={c['K']}, e8m0 per-128-K scales, {c['dist']} values, {c['out']} out")


def alg_bytes(c):
    """Algorithmic HBM bytes per step: operands, scales read once, output
    written once."""
    G = c.get("G", 1)
    M, N, K = c["M"], c["N"], c["K"]
    ob = 2 if c["out"] == "bf16" else 4
    if c["op"] == "int8":
        sc = 4 * (M + N)
    elif c["op"] == "fp8_blockwise":
        sc = 4 * (M * (K // 128) + (K // 128) * (N // 128))
    else:
        sc = G * (M * (K // 128) + (N // 128) * (K // 128))
    return G * (M * K + N * K) + sc + G * M * N * ob


def make_call(name, c, p, torch, bsmm):
    dev = "cuda:0"

    def d(x):
        return torch.from_numpy(x).to(dev)

    if c["op"] == "int8":
        a, b = d(p["a"]), d(p["b_nk"]).t()
        sa, sb = d(p["scale_a"]).reshape(-1, 1), d(p["scale_b"]).reshape(1, -1)
        out = torch.empty((c["M"], c["N"]), dtype=torch.bfloat16 if c["out"] == "bf16"
                          else torch.float32, device=dev)
        return lambda: bsmm.bsmm_int8_rowwise(a, b, sa, sb, out_dtype=c["out"], out=out)
    if c["op"] == "fp8_blockwise":
        a, b = d(p["a"]), d(p["b_nk"]).t()
        sa, sb = d(p["scale_a"]), d(p["scale_b"])
        out = torch.empty((c["M"], c["N"]), dtype=torch.bfloat16 if c["out"] == "bf16"
                          else torch.float32, device=dev)
        return lambda: bsmm.bsmm_fp8_blockwise(a, b, sa, sb, out_dtype=c["out"], out=out)
    x, w, xs, ws = d(p["x"]), d(p["w"]), d(p["x_scale"]), d(p["w_scale"])
    shape = (c["M"], c["G"], c["N"]) if c["layout"] == "m_major" else (c["G"], c["M"], c["N"])
    out = torch.empty(shape, dtype=torch.bfloat16 if c["out"] == "bf16" else torch.float32,
                      device=dev)
    return lambda: bsmm.bsmm_fp8_mx_bmm(x, w, xs, ws, layout=c["layout"],
                                        out_dtype=c["out"], out=out)


def cpu_baseline(name, c, p, budget_s=15.0):
    """Time the oracle on a bounded row sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import scaled_mm as S
    G = c.get("G", 1)
    M, N, K = c["M"], c["N"], c["K"]

    def run(rows):
        r = np.arange(rows)
        t0 = time.perf_counter()
        if c["op"] == "int8":
            S.int8_rowwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], c["out"], rows=r)
        elif c["op"] == "fp8_blockwise":
            S.fp8_blockwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], c["out"], rows=r)
        else:
            S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], c["layout"], c["out"],
                         rows=r)
        return time.perf_counter() - t0

    rows = min(M, 16)
    t = run(rows)
    # grow the sample toward the time budget
    while rows < M and t < budget_s / 3:
        rows = min(M, int(rows * max(2.0, min(8.0, budget_s / 2 / max(t, 1e-3)))))
        t = run(rows)
    flops = 2.0 * G * rows * N * K
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": flops / t / 1e12, "unit": "TFLOP/s" if c["op"] != "int8" else "TOP/s",
            "cores": int(max(threads) if threads else 1), "kind": "oracle",
            "sample": f"{rows} of {M} output rows (all {G}x{N} columns), full K={K}; "
                      f"{t:.2f} s; numpy/OpenBLAS fp64 incl. the error-bound GEMM",
            "seconds": t}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed calls before the warm-up steps")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the scaled matmul "
              "shards along M, N or G with no exchange, so per-GPU work is the one-GPU "
              "number", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_scaled_precision_gemm_amd as bsmm
    from synth import CONFIGS, config_inputs

    name = args.config
    c = CONFIGS[name]
    bsmm.load()
    t0 = time.time()
    p = config_inputs(name)
    print(f"[bench] inputs {name} generated in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    call = make_call(name, c, p, torch, bsmm)
    G = c.get("G", 1)
    M, N, K = c["M"], c["N"], c["K"]
    flops = 2.0 * G * M * N * K
    kind = "int8" if c["op"] == "int8" else "fp8"

    # Settle: the GPU raises its clock over the first few hundred ms under
    # load, so the call runs for about half a second before the W warm-up
    # steps (untimed, like them) and the timed steps see the steady state.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s, e in ev:
        s.record(stream)
        call()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    durs = sorted(s.elapsed_time(e) for s, e in ev)       # ms per step
    mean_ms = sum(durs) / len(durs)
    med_ms = durs[len(durs) // 2]
    ms_per_step = wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12

    plan = bsmm.bsmm_query_plan({"int8": 0, "fp8_blockwise": 1, "mx": 2}[c["op"]], G, M, N, K,
                                c["out"])
    abytes = alg_bytes(c)
    intensity = flops / abytes
    hbm_bound = intensity < PEAK[kind] / HBM_PEAK
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": abytes / (mean_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / (mean_ms * 1e-3) / 1e12,
                "peak": PEAK[kind] / 1e12, "unit": "TFLOP/s" if kind == "fp8" else "TOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if os.path.exists(tf):
        t = json.load(open(tf))
        if t.get("kernel_hash") == kernel_hash():
            roof["traffic"] = t["hbm_bytes_per_launch"]
    roof["alg_bytes"] = abytes
    roof["kernel_ms_mean"] = mean_ms
    roof["kernel_ms_median"] = med_ms
    roof["plan"] = plan["variant"] + (f" split{plan['split_k']}" if plan["split_k"] > 1 else "")

    line = {
        "metric": "TFLOP/s and % of MI355X peak fp8/int8 MFMA, block-scaled GEMM/BMM",
        "value": round(value, 2),
        "unit": "TFLOP/s" if kind == "fp8" else "TOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8_e4m3" if kind == "fp8" else "int8",
        "data": "synthetic",
        "config": {"workload": describe(name, c), "name": name, "G": G, "M": M, "N": N,
                   "K": K, "out": c["out"], "seed": c["seed"]},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(name, c, p, args.cpu_budget)
        line["cpu_baseline"] = {k: v for k, v in cb.items() if k != "seconds"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
