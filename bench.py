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
--config c1 | c2 | c4_m1 | c4_m128 | c4_m8192 | c5 | c3r (the fp8 scaled_mm with
rowwise scales and a bias on the blockwise workload's shape) | c3x (the same
shape with 32-element MX scales) | c3d, c3w (that layer's backward pass: the
input gradient, a blockwise GEMM 16640x8192x5120, and the weight gradient, a
groupwise GEMM 5120x8192 over 16640 tokens), and the dynamic
quantisers of their bf16 activations --config q_int8 | q_fp8 | q_mx | q_mx_t | q_mx32,
and of the backward pass q_cols_x | q_cols_dy | q_w | q_rows_cols_x (one quantiser call per step,
GB/s against 8 TB/s).

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
KERNEL_SOURCES = ["block_scaled_precision_gemm_amd/csrc/bsmm_kernels.hip",
                  "block_scaled_precision_gemm_amd/csrc/bsmm_pack.hip"]
QUANT_SOURCES = ["block_scaled_precision_gemm_amd/csrc/bsmm_quant.hip"]

# Dynamic-quantisation workloads: the bf16 activations of the matmul
# workloads (kind, shape, distribution, seed).
QUANT_CONFIGS = {
    "q_int8": ("int8", (8192, 4096), "normal", 2),        # X of the int8 8192x4096x4096 GEMM
    "q_fp8": ("fp8", (16640, 8192), "normal", 3),         # A of the fp8 16640x5120x8192 GEMM
    "q_mx": ("mx", (8192, 8, 4096), "normal", 43),        # x of the mx BMM, M=8192, G=8
    "q_mx_t": ("mx", (2, 9000, 7168), "t", 5),            # x of the mx BMM, G=2, M=9000
    "q_mx32": ("mx32", (16640, 8192), "normal", 3),       # A of the MX-32 16640x5120x8192 GEMM
    # the backward pass of the 16640-token layer: X and dY in groups of 128
    # tokens down their columns (codes transposed), W in 128 x 128 blocks
    # (plain and transposed codes)
    "q_cols_x": ("columns", (16640, 8192), "normal", 31),
    "q_cols_dy": ("columns", (16640, 5120), "normal", 32),
    "q_w": ("weight", (5120, 8192), "normal", 33),
    # X once for both: the forward's 1 x 128 row blocks and the column groups
    "q_rows_cols_x": ("rows_cols", (16640, 8192), "normal", 31),
}


OP_CODES = {"int8": 0, "fp8_blockwise": 1, "mx": 2, "fp8_scaled_mm": 3, "fp8_mx32": 4,
            "fp8_groupwise": 5}


def kernel_hash(sources=None):
    h = hashlib.sha256()
    for f in sources or KERNEL_SOURCES:
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
    if c["op"] == "fp8_mx32":
        return (f"fp8 e4m3 MX GEMM M={c['M']} N={c['N']} K={c['K']}, e8m0 scales per 32-long "
                f"K block of every row and column, {c['out']} out")
    if c["op"] == "fp8_groupwise":
        return (f"fp8 e4m3 groupwise GEMM M={c['M']} N={c['N']} K={c['K']}, fp32 scales per "
                f"128-long K block of every row and column, {c['out']} out")
    if c["op"] == "fp8_scaled_mm":
        return (f"fp8 e4m3 scaled_mm M={c['M']} N={c['N']} K={c['K']}, {c['scaling']} fp32 "
                f"scales, {c['bias']} bias, {c['out']} out")
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
    elif c["op"] == "fp8_scaled_mm":
        sc = 4 * (M + N) + 2 * N          # row and column scales, bf16 bias
    elif c["op"] == "fp8_mx32":
        sc = (M + N) * (K // 32)
    elif c["op"] == "fp8_groupwise":
        sc = 4 * (M + N) * (K // 128)
    elif c["op"] == "fp8_blockwise":
        sc = 4 * (M * (K // 128) + (K // 128) * (N // 128))
    else:
        sc = G * (M * (K // 128) + (N // 128) * (K // 128))
    return G * (M * K + N * K) + sc + G * M * N * ob


def launch_bytes(c, rows):
    """Algorithmic HBM bytes of one launch over `rows` of the M rows: its rows
    of A and of scale_a, all of B and scale_b, its rows of the output."""
    G = c.get("G", 1)
    N, K = c["N"], c["K"]
    ob = 2 if c["out"] == "bf16" else 4
    if c["op"] == "int8":
        sa, sb = 4 * rows, 4 * N
    elif c["op"] == "fp8_scaled_mm":
        sa, sb = 4 * rows, 4 * N + 2 * N
    elif c["op"] == "fp8_mx32":
        sa, sb = rows * (K // 32), N * (K // 32)
    elif c["op"] == "fp8_groupwise":
        sa, sb = 4 * rows * (K // 128), 4 * N * (K // 128)
    elif c["op"] == "fp8_blockwise":
        sa, sb = 4 * rows * (K // 128), 4 * (K // 128) * (N // 128)
    else:
        sa, sb = G * rows * (K // 128), G * (N // 128) * (K // 128)
    return G * (rows * K + N * K) + sa + sb + G * rows * N * ob


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
    if c["op"] == "fp8_mx32":
        a, b = d(p["a"]), d(p["b_nk"]).t()
        sa, sb = d(p["a_scale"]), d(p["b_scale"])
        out = torch.empty((c["M"], c["N"]), dtype=torch.bfloat16 if c["out"] == "bf16"
                          else torch.float32, device=dev)
        return lambda: bsmm.bsmm_fp8_mx32_mm(a, b, sa, sb, out_dtype=c["out"], out=out)
    if c["op"] == "fp8_groupwise":
        a, b = d(p["a"]), d(p["b_nk"]).t()
        sa, sb = d(p["scale_a"]), d(p["scale_b"])
        out = torch.empty((c["M"], c["N"]), dtype=torch.bfloat16 if c["out"] == "bf16"
                          else torch.float32, device=dev)
        return lambda: bsmm.bsmm_fp8_groupwise(a, b, sa, sb, out_dtype=c["out"], out=out)
    if c["op"] == "fp8_scaled_mm":
        a, b = d(p["a"]), d(p["b_nk"]).t()
        sa, sb = d(p["scale_a"]), d(p["scale_b"])
        bias = None if p["bias"] is None else d(p["bias"]).to(
            torch.bfloat16 if c["bias"] == "bf16" else torch.float32)
        out = torch.empty((c["M"], c["N"]), dtype=torch.bfloat16 if c["out"] == "bf16"
                          else torch.float32, device=dev)
        return lambda: bsmm.bsmm_fp8_scaled_mm(a, b, sa, sb, bias=bias, out_dtype=c["out"],
                                               out=out)
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
        elif c["op"] == "fp8_mx32":
            S.fp8_mx32_mm(p["a"], p["b_nk"].T, p["a_scale"], p["b_scale"], c["out"], rows=r)
        elif c["op"] == "fp8_groupwise":
            S.fp8_groupwise(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], c["out"], rows=r)
        elif c["op"] == "fp8_scaled_mm":
            S.fp8_scaled_mm(p["a"], p["b_nk"].T, p["scale_a"], p["scale_b"], bias=p["bias"],
                            out_dtype=c["out"], rows=r)
        else:
            S.fp8_mx_bmm(p["x"], p["w"], p["x_scale"], p["w_scale"], c["layout"], c["out"],
                         rows=r)
        return time.perf_counter() - t0

    rows = min(M, 16)
    t = run(rows)
    # grow the sample toward the time budget (the last sample takes roughly
    # 0.6 to 1 times the budget)
    while rows < M and t < budget_s * 0.6:
        rows = min(M, int(rows * max(1.5, min(8.0, budget_s * 0.8 / max(t, 1e-3)))))
        t = run(rows)
    flops = 2.0 * G * rows * N * K
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": flops / t / 1e12, "unit": "TFLOP/s" if c["op"] != "int8" else "TOP/s",
            "cores": int(max(threads) if threads else 1), "kind": "oracle",
            "sample": f"{rows} of {M} output rows (all {G}x{N} columns), full K={K}; "
                      f"{t:.2f} s; numpy/OpenBLAS fp64 incl. the error-bound GEMM",
            "seconds": t}


# ---------------------------------------------------------------------------
# Profile helpers: the summaries under profiles/ are made with these modes.
#   python bench.py --copy-kernel            (counter calibration workload)
#   python bench.py --summarize DIR          (rocprofv3 --kernel-trace --stats)
#   python bench.py --traffic F W CF CW      (FETCH_SIZE / WRITE_SIZE runs of
#                                             the bench and of --copy-kernel)
# ---------------------------------------------------------------------------
COPY_BYTES = 256 << 20


def copy_kernel():
    """A plain device copy of COPY_BYTES, three times: the reference workload
    that scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}))


def _csvs(d, suffix):
    import glob
    return sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))


def _main_kernel(name):
    return any(k in name for k in ("tile_kernel", "tile4_kernel", "sk_kernel", "skinny_kernel",
                                   "narrow_kernel", "quant_"))


def launches_per_call(name):
    """Main-kernel launches of one call of a workload: two for an M-split
    plan (the bulk launch first, then the tail), else one."""
    if name in QUANT_CONFIGS:
        return 1
    import block_scaled_precision_gemm_amd as bsmm
    from synth import CONFIGS
    c = CONFIGS[name]
    plan = bsmm.bsmm_query_plan(OP_CODES[c["op"]], c.get("G", 1), c["M"], c["N"], c["K"],
                                c["out"])
    return 2 if plan["m_split"] else 1


def summarize(d, name=None):
    """Kernel statistics of a rocprofv3 run plus the main kernel's dispatches
    grouped by grid size and, for an M-split plan of workload `name`, by
    launch (the bulk and the tail launch run the same kernel, often with the
    same persistent grid)."""
    import csv
    per_call = launches_per_call(name) if name else 1
    out = []
    for f in _csvs(d, "kernel_stats.csv"):
        rows = list(csv.DictReader(open(f)))
        out.append("kernel statistics (rocprofv3 --stats)")
        out.append(f"{'calls':>6} {'avg us':>10} {'min us':>10} {'max us':>10} {'total %':>8}  kernel")
        for r in rows:
            out.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                       f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                       f"{float(r['Percentage']):8.2f}  {r['Name'][:110]}")
    for f in _csvs(d, "kernel_trace.csv"):
        rows = [r for r in csv.DictReader(open(f)) if _main_kernel(r["Kernel_Name"])]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        groups = {}
        for i, r in enumerate(rows):
            grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
            launch = ("bulk" if i % per_call == 0 else "tail") if per_call > 1 else "-"
            key = (r["Kernel_Name"][:110], grid, launch)
            groups.setdefault(key, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        out.append("")
        out.append("main-kernel dispatches by grid size and launch (rocprofv3 --kernel-trace)")
        out.append(f"{'grid':>9} {'launch':>6} {'calls':>6} {'avg us':>10} {'min us':>10} "
                   f"{'max us':>10}  kernel")
        for (k, grid, launch), v in sorted(groups.items(), key=lambda kv: (-kv[0][1], kv[0][2])):
            out.append(f"{grid:9d} {launch:>6} {len(v):6d} {sum(v) / len(v):10.2f} "
                       f"{min(v):10.2f} {max(v):10.2f}  {k}")
    print("\n".join(out))


def _counter(d, counter, pick):
    """Per-dispatch values of one counter (summed over its instances) for the
    dispatches `pick` selects; returns (values, grid)."""
    import csv
    per = {}
    for f in _csvs(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter or not pick(r):
                continue
            key = (f, r["Dispatch_Id"])
            grid = int(r.get("Grid_Size") or 0)
            v, _ = per.get(key, (0.0, grid))
            per[key] = (v + float(r["Counter_Value"]), grid)
    return per


def traffic(name, fdir, wdir, cfdir, cwdir):
    """HBM bytes per launch of the main kernel from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the counter reads for the plain
    copy of COPY_BYTES."""
    per_call = launches_per_call(name)

    def largest_main(per):
        # the bulk launch: the first main-kernel dispatch of every call
        keys = sorted(per, key=lambda k: (k[0], int(k[1])))
        picked = [per[k] for i, k in enumerate(keys) if i % per_call == 0]
        return [v for v, _ in picked], picked[0][1]
    copy = lambda r: "copy" in r["Kernel_Name"].lower()
    cf = [v for v, _ in _counter(cfdir, "FETCH_SIZE", copy).values()]
    cw = [v for v, _ in _counter(cwdir, "WRITE_SIZE", copy).values()]
    f_scale = COPY_BYTES / (sum(cf) / len(cf) * 1024)
    w_scale = COPY_BYTES / (sum(cw) / len(cw) * 1024)
    main = lambda r: _main_kernel(r["Kernel_Name"])
    fv, grid = largest_main(_counter(fdir, "FETCH_SIZE", main))
    wv, _ = largest_main(_counter(wdir, "WRITE_SIZE", main))
    fetch = sum(fv) / len(fv) * 1024 * f_scale
    write = sum(wv) / len(wv) * 1024 * w_scale
    res = {"config": name,
           "kernel_hash": kernel_hash(QUANT_SOURCES if name in QUANT_CONFIGS else None),
           "grid": grid,
           "dispatches": len(fv), "fetch_bytes_per_launch": fetch,
           "write_bytes_per_launch": write, "hbm_bytes_per_launch": fetch + write,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "copy_fetch_kib": sum(cf) / len(cf), "copy_write_kib": sum(cw) / len(cw)}
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res))


def counters(name, dirs):
    """Per-launch averages of every counter collected (rocprofv3 --pmc, one
    pass per directory) for the dominant kernel's main launch of workload
    `name` -- the bulk launch of an M-split plan -- and derived figures:
    clock, matrix-core busy fraction, instruction-wait fraction, L2 hit rate
    and L2 read latency.  Durations come from the same runs' kernel traces
    when they were collected (--kernel-trace)."""
    import csv
    per_call = launches_per_call(name)
    vals = {}
    durs = []
    for d in dirs:
        per = {}
        for f in _csvs(d, "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                if not _main_kernel(r["Kernel_Name"]):
                    continue
                key = (f, int(r["Dispatch_Id"]))
                per.setdefault(key, {}).setdefault(r["Counter_Name"], 0.0)
                per[key][r["Counter_Name"]] += float(r["Counter_Value"])
        keys = sorted(per)
        for i, k in enumerate(keys):
            if i % per_call:
                continue                       # tail launches
            for c, v in per[k].items():
                vals.setdefault(c, []).append(v)
        for f in _csvs(d, "kernel_trace.csv"):
            rows = sorted((r for r in csv.DictReader(open(f)) if _main_kernel(r["Kernel_Name"])),
                          key=lambda r: int(r["Dispatch_Id"]))
            durs += [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
                     for i, r in enumerate(rows) if i % per_call == 0]
    avg = {c: sum(v) / len(v) for c, v in vals.items()}
    out = [f"counters per main launch ({name}; {min(len(v) for v in vals.values())} or more "
           "launches per counter)"]
    for c in sorted(avg):
        out.append(f"  {c:36s} {avg[c]:18.6g}")
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count if \
        torch.cuda.is_available() else 256
    xcds = 8
    der = []
    gui = avg.get("GRBM_GUI_ACTIVE")
    if gui and durs:
        dur = sum(durs) / len(durs)
        der.append(f"  launch duration (kernel trace, counter runs)  {dur * 1e6:10.2f} us")
        der.append(f"  clock  GRBM_GUI_ACTIVE / {xcds} XCDs / duration   "
                   f"{gui / xcds / dur / 1e9:10.3f} GHz")
    if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / xcds * cus * 4)
        der.append(f"  matrix cores busy  SQ_VALU_MFMA_BUSY_CYCLES / (GUI_ACTIVE/{xcds} x "
                   f"{cus} CUs x 4 SIMDs)  {busy:8.3f}")
    for mops in ("SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_I8"):
        if mops in avg:
            der.append(f"  matrix ops  {mops} x 512  {avg[mops] * 512:14.4g}")
    if "SQ_WAIT_INST_ANY" in avg and "SQ_WAVE_CYCLES" in avg:
        der.append(f"  waves waiting to issue  SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES  "
                   f"{avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:8.3f}")
    if "SQ_WAIT_ANY" in avg and "SQ_WAVE_CYCLES" in avg:
        der.append(f"  waves waiting (any)  SQ_WAIT_ANY / SQ_WAVE_CYCLES  "
                   f"{avg['SQ_WAIT_ANY'] / avg['SQ_WAVE_CYCLES']:8.3f}")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
        der.append(f"  VALU issued beside a busy matrix core  COEXEC / MFMA_BUSY  "
                   f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:8.3f}")
    if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
        h, m = avg["TCC_HIT_sum"], avg["TCC_MISS_sum"]
        der.append(f"  L2 hit rate  TCC_HIT / (HIT + MISS)  {h / (h + m):8.3f}")
    if "TCP_TCC_READ_REQ_LATENCY_sum" in avg and "TCP_TCC_READ_REQ_sum" in avg:
        der.append(f"  L2 read latency  TCP_TCC_READ_REQ_LATENCY / READ_REQ  "
                   f"{avg['TCP_TCC_READ_REQ_LATENCY_sum'] / avg['TCP_TCC_READ_REQ_sum']:8.1f} "
                   "cycles")
    if "TCC_EA0_RDREQ_LEVEL_sum" in avg and "TCC_EA0_RDREQ_sum" in avg:
        der.append(f"  L2-to-fabric reads in flight per request  EA0_RDREQ_LEVEL / EA0_RDREQ  "
                   f"{avg['TCC_EA0_RDREQ_LEVEL_sum'] / avg['TCC_EA0_RDREQ_sum']:8.1f} cycles")
    if "TCC_EA0_RDREQ_DRAM_sum" in avg and "TCC_EA0_RDREQ_sum" in avg:
        der.append(f"  L2 read misses sent to DRAM  EA0_RDREQ_DRAM / EA0_RDREQ  "
                   f"{avg['TCC_EA0_RDREQ_DRAM_sum'] / avg['TCC_EA0_RDREQ_sum']:8.3f}")
    if der:
        out.append("derived")
        out += der
    print("\n".join(out))


def quant_bytes(kind, rows, K):
    """Algorithmic HBM bytes of one quantiser call: bf16 input read once,
    1-byte codes and the scales written once."""
    if kind == "int8":
        scale = rows * 4
    elif kind == "mx32":
        scale = rows * (K // 32)
    elif kind == "columns":
        scale = (rows // 128) * K * 4
    elif kind == "weight":               # plain and transposed codes
        return rows * K * 2 + 2 * rows * K + (rows // 128) * (K // 128) * 4
    elif kind == "rows_cols":            # both layouts, row-block and column-group scales
        return rows * K * 2 + 2 * rows * K + rows * (K // 128) * 4 + (rows // 128) * K * 4
    else:
        scale = rows * (K // 128) * (4 if kind == "fp8" else 1)
    return rows * K * 2 + rows * K + scale


def quant_cpu_baseline(kind, x_rows, budget_s):
    """The oracle's quantiser on a growing sample of rows (about budget_s)."""
    from oracle import quant as Q
    fn = {"int8": Q.quant_int8_rowwise, "fp8": Q.quant_fp8_blockwise,
          "mx": Q.quant_fp8_mx, "mx32": lambda x: Q.quant_fp8_mx(x, block=32),
          "columns": Q.quant_fp8_columns, "weight": Q.quant_fp8_weight_blocks,
          "rows_cols": lambda x: (Q.quant_fp8_blockwise(x), Q.quant_fp8_columns(x))}[kind]
    R, K = x_rows.shape
    step = 128 if kind in ("columns", "weight", "rows_cols") else 1    # whole groups of 128 rows
    rows, t = min(R, max(64, step)), 0.0
    while True:
        t0 = time.perf_counter()
        fn(x_rows[:rows])
        t = time.perf_counter() - t0
        if rows >= R or t >= budget_s * 0.6:
            break
        rows = min(R, int(rows * max(1.5, min(8.0, budget_s * 0.8 / max(t, 1e-3)))))
        rows = max(step, rows // step * step)
    return {"value": quant_bytes(kind, rows, K) / t / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{rows} of {R} rows of K={K} (bf16 values widened to fp32); "
                      f"{t:.2f} s; numpy fp64, one thread"}


def bench_quant(args):
    import numpy as np
    import torch

    import block_scaled_precision_gemm_amd as bsmm
    from synth import activations

    name = args.config
    kind, shape, dist, seed = QUANT_CONFIGS[name]
    bsmm.load()
    t0 = time.time()
    x32 = activations(shape, seed=seed, dist=dist)
    xb = torch.from_numpy(x32).to(torch.bfloat16)
    K = shape[-1]
    R = int(np.prod(shape[:-1]))
    nbytes = quant_bytes(kind, R, K)
    # enough copies that successive calls never find their data in the 256 MB
    # last-level cache
    copies = max(2, -(-(1 << 30) // nbytes))
    xs = [xb.cuda() for _ in range(copies)]
    fn = {"int8": bsmm.bsmm_quant_int8_rowwise, "fp8": bsmm.bsmm_quant_fp8_blockwise,
          "mx": bsmm.bsmm_quant_fp8_mx,
          "mx32": lambda x, **kw: bsmm.bsmm_quant_fp8_mx(x, block=32, **kw),
          "columns": bsmm.bsmm_quant_fp8_columns, "weight": bsmm.bsmm_quant_fp8_weight,
          "rows_cols": bsmm.bsmm_quant_fp8_blockwise_columns}[kind]
    outs = [fn(x) for x in xs]
    torch.cuda.synchronize()
    print(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s, {copies} copies",
          file=sys.stderr, flush=True)
    if kind == "columns":
        calls = [(lambda x=x, o=o: fn(x, q_t=o[0], scale=o[1])) for x, o in zip(xs, outs)]
    elif kind == "weight":
        calls = [(lambda x=x, o=o: fn(x, q=o[0], q_t=o[1], scale=o[2]))
                 for x, o in zip(xs, outs)]
    elif kind == "rows_cols":
        calls = [(lambda x=x, o=o: fn(x, q=o[0], scale=o[1], q_t=o[2], scale_t=o[3]))
                 for x, o in zip(xs, outs)]
    else:
        calls = [(lambda x=x, o=o: fn(x, q=o[0], scale=o[1])) for x, o in zip(xs, outs)]
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(8):
            calls[i % copies]()
            i += 1
        torch.cuda.synchronize()
    for j in range(args.warmup):
        calls[j % copies]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()      # the stream the quantiser launches on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_wall = time.perf_counter()
    for j, (s, e) in enumerate(ev):
        s.record(stream)
        calls[j % copies]()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    kern_ms = sum(s.elapsed_time(e) for s, e in ev) / len(ev)
    ms_per_step = wall * 1e3 / args.steps
    roof = {"bound": "hbm", "achieved": nbytes / (kern_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if os.path.exists(tf):
        t = json.load(open(tf))
        if t.get("kernel_hash") == kernel_hash(QUANT_SOURCES):
            roof["traffic"] = t["hbm_bytes_per_launch"]
    roof["kernel"] = {"int8": "quant_int8_rows", "fp8": "quant_fp8_blocks<fp32 scale>",
                      "mx": "quant_fp8_blocks<e8m0 scale>",
                      "mx32": "quant_fp8_blocks<e8m0 scale, 32-element blocks>",
                      "columns": "quant_fp8_tiles<groups of 128 rows down the columns>",
                      "weight": "quant_fp8_tiles<128 x 128 blocks, plain and transposed>",
                      "rows_cols": "quant_fp8_tiles<1 x 128 row blocks and column groups>"}[kind]
    roof["kernel_ms_mean"] = kern_ms
    roof["kernel_alg_bytes"] = nbytes
    line = {
        "metric": "GB/s of dynamic quantisation (algorithmic HBM bytes) and % of 8 TB/s",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{kind} quantisation of bf16 "
                               f"{'weights' if kind == 'weight' else 'activations'} {list(shape)}",
                   "name": name, "rows": R, "K": K, "seed": seed, "dist": dist,
                   "copies": copies},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = quant_cpu_baseline(kind, xb.float().numpy().reshape(R, K),
                                                  args.cpu_budget)
    print(json.dumps(line), flush=True)


def mfma_peak(args):
    """The matrix cores' sustained rate on this device: the probe kernel
    (register operands only) on 2 workgroups of 4 waves per CU, timed with
    HIP events on its stream after the clock settles; fp8 and both int8
    instructions."""
    import torch

    import block_scaled_precision_gemm_amd as bsmm
    bsmm.load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs = 2 * cus
    out = torch.empty(wgs * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for kind, label in ((0, "fp8"), (1, "int8"), (2, "int8_32x32x32"), (3, "fp8_32x32x64")):
        iters = 20000
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < args.settle:
            bsmm.bsmm_mfma_probe(kind, wgs, iters, out)
            torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for s0, e0 in ev:
            s0.record(stream)
            flops = bsmm.bsmm_mfma_probe(kind, wgs, iters, out)
            e0.record(stream)
        torch.cuda.synchronize()
        ms = sorted(s0.elapsed_time(e0) for s0, e0 in ev)
        med = ms[len(ms) // 2]
        pk = PEAK["fp8" if kind in (0, 3) else "int8"]
        res[label] = {"achieved": flops / (med * 1e-3) / 1e12, "peak": pk / 1e12,
                      "unit": "TFLOP/s" if kind in (0, 3) else "TOP/s",
                      "frac_of_spec": flops / (med * 1e-3) / pk,
                      "launch_ms_median": med, "launch_ms_min": ms[0], "launches": len(ms),
                      "workgroups": wgs, "instructions_per_wave": iters * 8}
    print(json.dumps({"metric": "matrix-core probe rate (register operands, no memory "
                                "traffic) against the MI355X dense spec",
                      "cus": cus, "results": res}), flush=True)


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
    ap.add_argument("--copy-kernel", action="store_true")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="time the matrix-core probe kernel (fp8 and the int8 instructions)")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                   "COPY_WRITE_DIR"))
    ap.add_argument("--counters", nargs="+", metavar="PMC_DIR",
                    help="summarise rocprofv3 --pmc runs of --config's main launch")
    args = ap.parse_args()
    if args.summarize:
        return summarize(args.summarize, args.config)
    if args.traffic:
        return traffic(args.config, *args.traffic)
    if args.counters:
        return counters(args.config, args.counters)
    if args.copy_kernel:
        return copy_kernel()
    if args.mfma_peak:
        return mfma_peak(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the scaled matmul "
              "shards along M, N or G with no exchange, so per-GPU work is the one-GPU "
              "number", file=sys.stderr)
        sys.exit(2)

    if args.config in QUANT_CONFIGS:
        return bench_quant(args)

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
    G = c.get("G", 1)
    M, N, K = c["M"], c["N"], c["K"]
    flops = 2.0 * G * M * N * K
    kind = "int8" if c["op"] == "int8" else "fp8"
    intensity = flops / alg_bytes(c)
    hbm_bound = intensity < PEAK[kind] / HBM_PEAK
    # HBM-bound shapes are timed cold: enough independent copies of the
    # inputs and output (>= 1 GiB together, far more than the 256 MB
    # last-level cache) that no call finds its operands cached by the ones
    # before it; the hot figure (one copy, operands cached) is reported too.
    copies = min(64, max(9, -(-(1 << 30) // alg_bytes(c)))) if hbm_bound else 1
    calls = [make_call(name, c, p, torch, bsmm) for _ in range(copies)]
    torch.cuda.synchronize()
    print(f"[bench] {copies} input copies on the device", file=sys.stderr, flush=True)

    def timed(fns, steps):
        """(wall ms per step, event ms per step, main-launch ms) over `steps`
        calls rotating through `fns`, HIP events on the launch stream."""
        stream = torch.cuda.current_stream()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        bsmm.bsmm_timing_enable(True)       # events around each step's main launch
        t_wall = time.perf_counter()
        for j, (s, e) in enumerate(ev):
            s.record(stream)
            fns[j % len(fns)]()
            e.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_wall
        kern = bsmm.bsmm_timing_read()
        bsmm.bsmm_timing_enable(False)
        return wall * 1e3 / steps, sum(s.elapsed_time(e) for s, e in ev) / steps, kern

    # Settle: the GPU raises its clock over the first few hundred ms under
    # load, so the call runs for about half a second before the W warm-up
    # steps (untimed, like them) and the timed steps see the steady state.
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(8):
            calls[i % copies]()
            i += 1
        torch.cuda.synchronize()
    for j in range(args.warmup):
        calls[j % copies]()
    torch.cuda.synchronize()
    ms_per_step, step_ms_mean, (kern_ms, kern_n, kern_variant) = timed(calls, args.steps)
    value = flops / (ms_per_step * 1e-3) / 1e12
    hot = None
    host_loop_us = None
    if hbm_bound:
        hot = timed(calls[:1], args.steps)
        # decode-sized calls: the per-call cost of a plain host loop (no
        # events, no synchronisation between calls), cold
        n_loop = 2000
        torch.cuda.synchronize()
        t_loop = time.perf_counter()
        for j in range(n_loop):
            calls[j % copies]()
        torch.cuda.synchronize()
        host_loop_us = (time.perf_counter() - t_loop) * 1e6 / n_loop

    op = OP_CODES[c["op"]]
    plan = bsmm.bsmm_query_plan(op, G, M, N, K, c["out"])
    # dominant kernel: the main launch of the plan (all rows, or the bulk rows
    # of an M-split plan); its algorithmic work is its share of the rows
    rows = plan["m_split"] or M
    kflops = flops * rows / M
    kbytes = launch_bytes(c, rows)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": kbytes / (kern_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": kflops / (kern_ms * 1e-3) / 1e12,
                "peak": PEAK[kind] / 1e12, "unit": "TFLOP/s" if kind == "fp8" else "TOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    tf = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if os.path.exists(tf):
        t = json.load(open(tf))
        if t.get("kernel_hash") == kernel_hash():
            roof["traffic"] = t["hbm_bytes_per_launch"]
    roof["kernel"] = kern_variant
    roof["kernel_ms_mean"] = kern_ms
    roof["kernel_launches"] = kern_n
    roof["kernel_rows"] = rows
    roof["kernel_alg_flops"] = kflops
    roof["kernel_alg_bytes"] = kbytes
    roof["step_ms_mean"] = step_ms_mean
    if hbm_bound:
        roof["timing"] = (f"cold: {copies} rotating input copies, "
                          f"{copies * alg_bytes(c) / 2**20:.0f} MiB in all")
        roof["hot_kernel_ms_mean"] = hot[2][0]
        roof["hot_achieved"] = kbytes / (hot[2][0] * 1e-3) / 1e9
        roof["hot_ms_per_step"] = hot[0]
        roof["host_loop_us_per_call"] = host_loop_us
    roof["plan"] = (plan["variant"] + (f" split{plan['split_k']}" if plan["split_k"] > 1 else "")
                    + (f" + rows {plan['m_split']}..{M}: {plan['tail_variant']}"
                       f" split{plan['tail_split_k']}" if plan["m_split"] else ""))

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
