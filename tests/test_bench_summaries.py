"""bench.py's reading of rocprofv3 output (host logic, no GPU): the
dispatches of every main-kernel family are grouped and timed; the helper
kernels that run beside them (scale packing, the split-K reduction, copies)
are not taken for the main launch."""

import csv

import bench

MAIN = [
    "void bsmm::(anonymous namespace)::tile_kernel<1, 2, 4, 2, 5, true>(bsmm::KArgs)",
    "void bsmm::(anonymous namespace)::tile4_kernel<2, 2, true>(bsmm::KArgs)",
    "void bsmm::(anonymous namespace)::sk_kernel<0, 2, 4, 2, 5, false>(bsmm::KArgs, bsmm::SkArgs)",
    "void bsmm::(anonymous namespace)::skinny_kernel<2, 2, 2>(bsmm::KArgs)",
    "void bsmm::(anonymous namespace)::quant_fp8_tiles<unsigned short, 128, false, true>(...)",
]
HELPERS = [
    "void bsmm::(anonymous namespace)::splitk_reduce<2, 2>(bsmm::KArgs)",
    "void bsmm::(anonymous namespace)::pack_kernel<2>(bsmm::Problem, void*, long)",
    "__amd_rocclr_copyBuffer",
]


def test_main_kernel_families():
    for k in MAIN:
        assert bench._main_kernel(k), k
    for k in HELPERS:
        assert not bench._main_kernel(k), k


def _write(path, fields, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_summarize_groups_the_skinny_launches(tmp_path, capsys):
    """Three calls of a decode-sized plan (pack, skinny kernel, reduction
    interleaved): only the three skinny dispatches form the main group, with
    their mean, minimum and maximum durations."""
    skinny, reduce_, pack = MAIN[3], HELPERS[0], HELPERS[1]
    trace, t, did = [], 1_000_000, 0
    for dur in (8000, 9000, 10000):
        for name, d, grid in ((pack, 2000, 4096), (skinny, dur, 2048), (reduce_, 3000, 65536)):
            did += 1
            trace.append(dict(Dispatch_Id=did, Kernel_Name=name, Grid_Size=grid,
                              Start_Timestamp=t, End_Timestamp=t + d))
            t += d + 500
    d = tmp_path / "run" / "host"
    d.mkdir(parents=True)
    _write(d / "1_kernel_trace.csv", list(trace[0]), trace)
    stats = [dict(Name=n, Calls=3, AverageNs=a, MinNs=a, MaxNs=a, Percentage=p)
             for n, a, p in ((skinny, 9000, 64.3), (reduce_, 3000, 21.4), (pack, 2000, 14.3))]
    _write(d / "1_kernel_stats.csv", list(stats[0]), stats)
    bench.summarize(str(tmp_path))
    out = capsys.readouterr().out
    section = out.split("main-kernel dispatches")[1]
    lines = [ln.split() for ln in section.splitlines() if "skinny_kernel" in ln]
    assert len(lines) == 1, section
    grid, launch, calls, avg, lo, hi = lines[0][:6]
    assert (grid, launch, calls) == ("2048", "-", "3")
    assert (float(avg), float(lo), float(hi)) == (9.0, 8.0, 10.0)
    assert "splitk_reduce" not in section and "pack_kernel" not in section
