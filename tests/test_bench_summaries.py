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


def _counters(d, rows):
    d.mkdir(parents=True)
    _write(d / "1_counter_collection.csv",
           ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"], rows)


def test_traffic_scales_the_counters_by_the_copy_calibration(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch, summed over the counter's
    instances) of the main kernel, averaged over its dispatches and scaled
    by the copy kernel's bytes over what the counter read for the copy; a
    helper kernel's dispatches do not count."""
    import json
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_hash", lambda sources=None: "0" * 16)
    (tmp_path / "profiles").mkdir()
    copy_kib = bench.COPY_BYTES / 1024
    cp = "__amd_rocclr_copyBuffer"
    # the copy reads as half its size (scale 2) and writes as a quarter (scale 4)
    _counters(tmp_path / "cf", [dict(Dispatch_Id=1, Kernel_Name=cp, Grid_Size=1, Counter_Name="FETCH_SIZE",
                                     Counter_Value=copy_kib / 4)] * 2)
    _counters(tmp_path / "cw", [dict(Dispatch_Id=1, Kernel_Name=cp, Grid_Size=1, Counter_Name="WRITE_SIZE",
                                     Counter_Value=copy_kib / 4)])
    q = "void bsmm::(anonymous namespace)::quant_fp8_blocks<unsigned short, 128, 0>(...)"
    fetch = [dict(Dispatch_Id=i + 1, Kernel_Name=q, Grid_Size=4096, Counter_Name="FETCH_SIZE",
                  Counter_Value=v) for i, v in enumerate((1000, 1100, 1200))]
    fetch.append(dict(Dispatch_Id=9, Kernel_Name=HELPERS[0], Grid_Size=64, Counter_Name="FETCH_SIZE",
                      Counter_Value=99999))
    _counters(tmp_path / "f", fetch)
    # dispatch 1 in two counter instances (200 + 300), dispatch 2 in one (500)
    _counters(tmp_path / "w", [dict(Dispatch_Id=i, Kernel_Name=q, Grid_Size=4096,
                                    Counter_Name="WRITE_SIZE", Counter_Value=v)
                               for i, v in ((1, 200), (1, 300), (2, 500))])
    bench.traffic("q_fp8", *(str(tmp_path / n) for n in ("f", "w", "cf", "cw")))
    res = json.load(open(tmp_path / "profiles" / "traffic_q_fp8.json"))
    assert res["fetch_scale"] == 2.0 and res["write_scale"] == 4.0
    assert res["dispatches"] == 3 and res["grid"] == 4096
    assert res["fetch_bytes_per_launch"] == 1100 * 1024 * 2.0
    assert res["write_bytes_per_launch"] == 500 * 1024 * 4.0
    assert res["hbm_bytes_per_launch"] == res["fetch_bytes_per_launch"] + res["write_bytes_per_launch"]
