"""Measure kernel plans per problem shape on the GPU and write the
shape-keyed dispatch table (csrc/bsmm_tuned_table.inc).

For every shape the dispatcher's own plan and every (variant, split-K)
candidate are timed on device-resident random operands; a shape gets a table
entry when its best candidate beats the dispatcher's plan by more than the
margin.  Entries for shapes not measured in this run are kept.  Rebuild the
library afterwards (``python -m block_scaled_precision_gemm_amd.build``).

    python -m block_scaled_precision_gemm_amd.tune \\
        --shape mx,bf16,8,128,1024,4096,m_major --shape fp8_blockwise,bf16,1,16640,5120,8192
"""

from __future__ import annotations

import argparse
import os
import re

import torch

from . import (BF16, E4M3, F32, I32, OP_FP8_BLOCKWISE, OP_FP8_MX32_MM, OP_FP8_MX_BMM,
               OP_FP8_SCALED_MM, OP_INT8_ROWWISE, OP_FP8_GROUPWISE, bsmm_fp8_blockwise,
               bsmm_fp8_groupwise, bsmm_fp8_mx32_mm,
               bsmm_fp8_mx_bmm, bsmm_fp8_scaled_mm, bsmm_int8_rowwise, bsmm_query_plan,
               bsmm_set_override, bsmm_variant_names, load)

TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "bsmm_tuned_table.inc")
OPS = {"int8": OP_INT8_ROWWISE, "fp8_blockwise": OP_FP8_BLOCKWISE, "mx": OP_FP8_MX_BMM,
       "scaled_mm": OP_FP8_SCALED_MM, "mx32": OP_FP8_MX32_MM, "groupwise": OP_FP8_GROUPWISE}
DTYPES = {"i32": I32, "f32": F32, "bf16": BF16, "e4m3": E4M3}
SPLITS = (1, 2, 3, 4, 6, 8, 12)


def parse_shape(s):
    f = s.split(",")
    op, out = f[0], f[1]
    G, M, N, K = (int(x) for x in f[2:6])
    layout = f[6] if len(f) > 6 else "m_major"
    if op not in OPS or out not in DTYPES:
        raise SystemExit(f"bad shape {s!r}: op in {list(OPS)}, out in {list(DTYPES)}")
    return dict(op=op, out=out, G=G, M=M, N=N, K=K, layout=layout)


def make_call(sh, dev="cuda:0"):
    """Random operands of the shape (timing only: codes are random bytes with
    the E4M3 NaN patterns masked out, scales random)."""
    G, M, N, K, out = sh["G"], sh["M"], sh["N"], sh["K"], sh["out"]
    g = torch.Generator(device=dev).manual_seed(0)
    odt = {"i32": torch.int32, "f32": torch.float32, "bf16": torch.bfloat16,
           "e4m3": torch.float8_e4m3fn}[out]
    if sh["op"] == "int8":
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        b = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
        sa = torch.rand((M, 1), device=dev, generator=g)
        sb = torch.rand((1, N), device=dev, generator=g)
        o = torch.empty((M, N), dtype=odt, device=dev)
        return lambda: bsmm_int8_rowwise(a, b.t(), sa, sb, out_dtype=out, out=o)
    codes = lambda *s: torch.randint(0, 256, s, dtype=torch.uint8, device=dev, generator=g) & 0x77
    if sh["op"] == "scaled_mm":
        a, b = codes(M, K), codes(N, K)
        sa = torch.rand((M, 1), device=dev, generator=g)
        sb = torch.rand((1, N), device=dev, generator=g)
        bias = torch.rand((N,), device=dev, generator=g).to(torch.bfloat16)
        o = torch.empty((M, N), dtype=odt, device=dev)
        return lambda: bsmm_fp8_scaled_mm(a, b.t(), sa, sb, bias=bias, out_dtype=out, out=o)
    e8 = lambda *s: torch.randint(120, 135, s, dtype=torch.uint8, device=dev, generator=g)
    if sh["op"] == "mx32":
        a, b = codes(M, K), codes(N, K)
        o = torch.empty((M, N), dtype=odt, device=dev)
        sa, sb = e8(M, K // 32), e8(N, K // 32)
        return lambda: bsmm_fp8_mx32_mm(a, b.t(), sa, sb, out_dtype=out, out=o)
    if sh["op"] == "groupwise":
        a, b = codes(M, K), codes(N, K)
        sa = torch.rand((M, K // 128), device=dev, generator=g)
        sb = torch.rand((K // 128, N), device=dev, generator=g)
        o = torch.empty((M, N), dtype=odt, device=dev)
        return lambda: bsmm_fp8_groupwise(a, b.t(), sa, sb, out_dtype=out, out=o)
    if sh["op"] == "fp8_blockwise":
        a, b = codes(M, K), codes(N, K)
        sa = torch.rand((M, K // 128), device=dev, generator=g)
        sb = torch.rand((K // 128, N // 128), device=dev, generator=g)
        o = torch.empty((M, N), dtype=odt, device=dev)
        return lambda: bsmm_fp8_blockwise(a, b.t(), sa, sb, out_dtype=out, out=o)
    if sh["layout"] == "m_major":
        x, xs = codes(M, G, K), e8(M, G, K // 128)
        o = torch.empty((M, G, N), dtype=odt, device=dev)
    else:
        x, xs = codes(G, M, K), e8(G, M, K // 128)
        o = torch.empty((G, M, N), dtype=odt, device=dev)
    w, ws = codes(G, N, K), e8(G, N // 128, K // 128)
    return lambda: bsmm_fp8_mx_bmm(x, w, xs, ws, layout=sh["layout"], out_dtype=out, out=o)


def time_call(call, reps=3, n=20):
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            call()
        e.record()
        torch.cuda.synchronize()
        best = min(best, s.elapsed_time(e) / n)
    return best


def candidates(sh):
    """Distinct (variant, split) plans the override produces for the shape
    (groupwise: packed-scale variants only, the kernels it has)."""
    op, dt = OPS[sh["op"]], sh["out"]
    seen = {}
    try:
        for v in bsmm_variant_names():
            if sh["op"] == "groupwise" and not v.endswith("p"):
                continue
            for sp in SPLITS:
                bsmm_set_override(v, sp)
                p = bsmm_query_plan(op, sh["G"], sh["M"], sh["N"], sh["K"], dt)
                seen.setdefault((p["variant"], p["split_k"]), (v, sp))
    finally:
        bsmm_set_override(None, 0)
    return list(seen)


def read_table(path=None):
    path = path or TABLE
    rows = {}
    if os.path.exists(path):
        for line in open(path):
            body = line.split("//")[0].strip()
            m = re.match(r"\{(.*)\},?$", body)
            if m:
                f = [x.strip() for x in m.group(1).split(",")]
                rows[tuple(int(x) for x in f[:6])] = body.rstrip(",")
    return rows


def write_table(rows, path=None):
    with open(path or TABLE, "w") as fh:
        fh.write("// op, out_dtype, G, M, N, K, variant, split, m_split, tail_variant, tail_split\n")
        fh.write("// measured on MI355X by block_scaled_precision_gemm_amd.tune\n")
        for key in sorted(rows):
            fh.write(rows[key] + ",\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--shape", action="append", required=True,
                    help="op,out,G,M,N,K[,layout]  "
                         "(op: int8 | fp8_blockwise | mx | scaled_mm | mx32 | groupwise)")
    ap.add_argument("--margin", type=float, default=0.03,
                    help="required gain over the dispatcher's own plan")
    ap.add_argument("--dry-run", action="store_true", help="print, do not write the table")
    ap.add_argument("--out", default=None, help="table file to write (default: the package's)")
    args = ap.parse_args(argv)
    load()
    rows = read_table(args.out if args.out and os.path.exists(args.out) else None)
    for s in args.shape:
        sh = parse_shape(s)
        call = make_call(sh)
        key = (OPS[sh["op"]], DTYPES[sh["out"]], sh["G"], sh["M"], sh["N"], sh["K"])
        bsmm_set_override(None, 0)              # the library's current dispatch
        base = time_call(call)
        best = (base, None)
        for v, sp in candidates(sh):
            bsmm_set_override(v, sp)
            try:
                t = time_call(call)
            finally:
                bsmm_set_override(None, 0)
            print(f"{s}: {v} split {sp}: {t * 1e3:.2f} us", flush=True)
            if t < best[0]:
                best = (t, (v, sp))
        print(f"{s}: dispatcher {base * 1e3:.2f} us, best {best[0] * 1e3:.2f} us {best[1]}", flush=True)
        if best[1] and best[0] < base * (1.0 - args.margin):
            v, sp = best[1]
            rows[key] = "{%d, %d, %d, %d, %d, %d, \"%s\", %d, 0, \"\", 1}" % (key + (v, sp))
    if args.dry_run:
        for k in sorted(rows):
            print(rows[k])
    else:
        write_table(rows, args.out)
        print(f"wrote {args.out or TABLE} ({len(rows)} entries)")


if __name__ == "__main__":
    main()
