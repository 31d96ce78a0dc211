"""Host logic of bench.py (no GPU): kernel-name shortening, cutting a rocprofv3 trace into the
bench's phases and launch positions, the traffic arithmetic, and the algorithmic byte counts of
the stage entry points."""

import csv
import os

import pytest

import bench
import moe_inputs


def _trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size_X", "Start_Timestamp",
                                          "End_Timestamp"])
        w.writeheader()
        for i, (name, grid, ns) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size_X": grid, "Start_Timestamp": 1000 * i,
                        "End_Timestamp": 1000 * i + ns})


def _counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, grid, cname, val) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": cname,
                        "Counter_Value": val})


MARK = "void (anonymous namespace)::bench_mark_kernel(unsigned int*, unsigned int)"
FILL = "void (anonymous namespace)::fill_kernel(unsigned int __vector(4)*, long, unsigned int)"
G1 = "void moe::(anonymous namespace)::gemm_bf16_kernel<256, 2, true, false, 1>(unsigned short const*, int)"
G2 = "void moe::(anonymous namespace)::gemm_bf16_kernel<256, 2, false, false, 4>(unsigned short const*, int)"
COPY = "void (anonymous namespace)::stream_copy_kernel(unsigned int __vector(4) const*, long)"


def test_short_kernel_name():
    assert bench.short_kernel_name(G1) == "gemm_bf16_kernel<256, 2, true, false, 1>"
    assert bench.short_kernel_name(MARK) == "bench_mark_kernel"
    assert bench.short_kernel_name('"moe::(anonymous namespace)::combine_kernel<1, 1, 8>(void const*)"') == \
        "combine_kernel<1, 1, 8>"


def test_segments_and_positions(tmp_path):
    # two warm-up steps, one cold step (flush first), a foreign kernel before any marker
    rows = [("at::native::foo(int)", 256, 5),
            (MARK, 64, 1), (G1, 1024, 100), (G2, 1024, 50), (G1, 1024, 30), (G2, 1024, 20),
            (MARK, 64, 1), (G1, 1024, 110), (G2, 1024, 60), (G1, 1024, 40), (G2, 1024, 10),
            (FILL, 4096, 900), (MARK, 3 * 64, 1), (G1, 1024, 200), (G2, 1024, 80), (G1, 1024, 35), (G2, 1024, 25)]
    _trace(tmp_path / "x_kernel_trace.csv", rows)
    segs = bench.all_segments([str(tmp_path)])
    assert [p for p, _ in segs] == [1, 1, 3]
    stats, n = bench.position_stats(segs, 1)
    assert n == 2
    assert [r["ns"] for r in stats["gemm_bf16_kernel<256, 2, true, false, 1> #0"]] == [100, 110]
    assert [r["ns"] for r in stats["gemm_bf16_kernel<256, 2, true, false, 1> #1"]] == [30, 40]
    cold, n = bench.position_stats(segs, 3)
    assert n == 1 and [r["ns"] for r in cold["gemm_bf16_kernel<256, 2, false, false, 4> #0"]] == [80]
    assert not any(lab.startswith("fill_kernel") for _, s in segs for lab, _ in s)
    text = bench.summarize_trace([str(tmp_path)])
    assert "phase 3" in text and "| gemm_bf16_kernel<256, 2, true, false, 1> #0 | 1 | 0.20 |" in text


def test_traffic_report(tmp_path, capsys):
    dirs = {}
    for name, counter, kib, cal_kib in (("f", "FETCH_SIZE", 3000.0, 524288.0), ("w", "WRITE_SIZE", 200.0, 1048576.0)):
        d = tmp_path / name
        d.mkdir()
        _counters(d / "r_counter_collection.csv",
                  [(MARK, 3 * 64, counter, 0), (G1, 1024, counter, kib), (G2, 1024, counter, 7.0),
                   (MARK, 3 * 64, counter, 0), (G1, 1024, counter, kib + 2), (G2, 1024, counter, 7.0)])
        c = tmp_path / ("c" + name)
        c.mkdir()
        _counters(c / "r_counter_collection.csv", [(MARK, 11 * 64, counter, 0), (COPY, 4096, counter, cal_kib)])
        dirs[name] = (str(d), str(c))

    class A:
        traffic_report = (dirs["f"][0], dirs["w"][0], dirs["f"][1], dirs["w"][1])
        traffic_phase = 3
        traffic_label = "gemm_bf16_kernel<256, 2, true, false, 1> #0"
        traffic_alg_bytes = 1000

    bench.traffic_report(A)
    kv = dict(line.split(" = ") for line in capsys.readouterr().out.strip().splitlines())
    # fetch 3001 KiB scaled by 2 (the copy's 1 GiB read shows as 0.5 GiB), write 201 KiB by 1
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["read_bytes_per_launch"]) == pytest.approx(3001 * 1024 * 2)
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx(3001 * 1024 * 2 + 201 * 1024)


def test_stage_call_bytes():
    cfg = moe_inputs.CONFIGS["deepseek_v3"]
    b = bench.algorithmic_stage_calls(cfg)
    T, H, k, E = cfg.T, cfg.H, cfg.k, cfg.E
    R = T * k
    assert b["permute_bf16"] == T * H * 2 + R * H * 2 + R * 12 + (2 * E + 1) * 4
    assert b["permute_e4m3"] == T * H * 2 + R * H + R * (H // 128) * 4 + R * 12 + (2 * E + 1) * 4
    assert b["combine"] == R * H * 2 + R * 8 + T * H * 2


def test_committed_traffic_files_parse():
    for path in (bench.traffic_file("gemm1_swiglu", "mixtral_8x7b"),
                 bench.traffic_file("wgrad_w1_backward", "mixtral_8x7b")):
        if os.path.exists(path):
            kv = bench.read_kv(path)
            assert float(kv["traffic_bytes_per_launch"]) > 0
