"""Host checks of the profile summarisers (counter files are synthetic here)."""
import csv
import json

from nvfp4_w4a4_quantized_amd import kernel_stats, mfma_counters, stall_counters, traffic

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]
FC1 = "void nvfp4::gemm_w4a4_kernel<4, 2, 8, 2>(nvfp4::GemmArgs)"
FC2 = "void nvfp4::gemm_w4a4_kernel<4, 2, 4, 1>(nvfp4::GemmArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, bitwise_not>(int)"


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (did, name, grid, counter, value, t0, t1) in enumerate(rows):
            w.writerow({c: 0 for c in COLS} | {
                "Correlation_Id": i, "Dispatch_Id": did, "Kernel_Name": name,
                "Grid_Size": grid, "Counter_Name": counter, "Counter_Value": value,
                "Start_Timestamp": t0, "End_Timestamp": t1})


def test_mfma_counters_groups_by_launch_and_drops_warmup(tmp_path):
    p = tmp_path / "m.csv"
    rows = []
    # FC1: a slow warm-up dispatch, then two at 400 us with 450 GFLOP of MOPS
    for did, ns, util in ((1, 900_000, 10.0), (3, 400_000, 50.0), (5, 400_000, 60.0)):
        rows.append((did, FC1, 1000, "MfmaUtil", util, 0, ns))
        rows.append((did, FC1, 1000, "SQ_INSTS_VALU_MFMA_MOPS_F16", 450e9 / 512, 0, ns))
    # the same kernel at two grid sizes (two dense GEMMs) stays apart
    for did, grid in ((7, 2000), (8, 3000), (9, 2000), (10, 3000)):
        rows.append((did, FC2, grid, "MfmaUtil", 40.0, 0, 100_000))
        rows.append((did, FC2, grid, "SQ_INSTS_VALU_MFMA_MOPS_F16", 100e9 / 512, 0, 100_000))
    _write(p, rows)
    per = mfma_counters.per_dispatch(str(p))
    assert [len(v) for v in per.values()] == [3, 2, 2]
    text = mfma_counters.table(str(p), {"4, 2, 8, 2>": 412.3, "/3000": 90.0})
    lines = [l for l in text.splitlines() if l.startswith("| `")]
    assert len(lines) == 3
    fc1 = lines[0].split("|")
    # warm-up dropped: 400 us, 55% mean utilisation, 450 GFLOP -> 1125 TFLOP/s
    assert fc1[3].strip() == "2" and fc1[4].strip() == "400.0" and fc1[5].strip() == "55.0%"
    assert fc1[6].strip() == "450.0" and fc1[7].strip() == "412.3" and fc1[8].strip() == "1125"
    assert lines[1].split("|")[7].strip() == "-" and lines[2].split("|")[7].strip() == "90.0"


def test_stall_counters_joins_passes_and_drops_warmup(tmp_path):
    p1, p2 = tmp_path / "p1.csv", tmp_path / "p2.csv"
    ns = 100_000
    clock = 2.0                                   # GHz
    cycles = clock * ns                           # shader-engine cycles per dispatch
    first = {"SQ_BUSY_CYCLES": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1.0, "SQ_WAVE_CYCLES": 1.0,
             "SQ_WAIT_ANY": 1.0, "SQ_WAIT_INST_ANY": 0.0, "SQ_ACTIVE_INST_ANY": 0.0}
    pass1 = {"SQ_BUSY_CYCLES": stall_counters.SHADER_ENGINES * cycles,
             "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * stall_counters.SIMDS * cycles,
             "SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 300.0, "SQ_WAIT_INST_ANY": 200.0,
             "SQ_ACTIVE_INST_ANY": 500.0}
    idx = 0.1 * stall_counters.CUS * cycles
    pass2 = {"SQ_INSTS_VALU": 4000.0, "SQ_INSTS_MFMA": 1000.0, "SQ_INSTS_LDS": 500.0,
             "SQ_VALU_MFMA_COEXEC_CYCLES": 0.25 * 4 * 4000.0, "SQ_LDS_IDX_ACTIVE": idx,
             "SQ_LDS_BANK_CONFLICT": 0.2 * idx}
    # dispatch 1 is the warm-up (dropped); a non-GEMM kernel is ignored
    rows1 = [(1, FC1, 1000, c, v, 0, 5 * ns) for c, v in first.items()]
    rows1 += [(2, COPY, 64, "SQ_WAVE_CYCLES", 7.0, 0, 10)]
    rows1 += [(3, FC1, 1000, c, v, 0, ns) for c, v in pass1.items()]
    rows2 = [(1, FC1, 1000, c, 1.0, 0, 5 * ns) for c in pass2]
    rows2 += [(3, FC1, 1000, c, v, 0, ns) for c, v in pass2.items()]
    _write(p1, rows1)
    _write(p2, rows2)
    lines = [l for l in stall_counters.table([str(p1), str(p2)]).splitlines() if l.startswith("| `")]
    assert len(lines) == 1
    cells = [c.strip() for c in lines[0].split("|")[1:-1]]
    assert cells == ["`gemm_w4a4_kernel<4, 2, 8, 2>`", "1000", "100.0", "2.00", "50%", "30%", "20%",
                     "50%", "4.0", "0.50", "25%", "10%", "20%"]


def test_kernel_stats_last_dispatches_per_grid(tmp_path):
    p = tmp_path / "kt.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # FC1: two slow warm-up dispatches, then three at 100, 110, 120 us
        for i, d in enumerate((900, 800, 100, 110, 120)):
            w.writerow({"Kernel_Name": FC1, "Grid_Size_X": 1000, "Start_Timestamp": 10_000_000 * i,
                        "End_Timestamp": 10_000_000 * i + d * 1000})
        # the same kernel at another grid size stays apart
        w.writerow({"Kernel_Name": FC1, "Grid_Size_X": 2000, "Start_Timestamp": 5, "End_Timestamp": 5005})
    lines = [l for l in kernel_stats.last_table(str(p), 3).splitlines() if l.startswith("| `")]
    assert len(lines) == 2
    cells = [c.strip() for c in lines[0].split("|")[1:-1]]
    assert cells == ["`gemm_w4a4_kernel<4, 2, 8, 2>`", "1000", "5", "3", "110.0", "100.0", "120.0"]
    w = kernel_stats.window(str(p), "4, 2, 8, 2>", 1000, 1, 2)
    assert "dispatches 1-2 of 5" in w and "average 450.0 us" in w


def test_traffic_scales_by_copy_calibration(tmp_path):
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    mib = 64
    known = mib << 20
    # the copy reads half its bytes by FETCH_SIZE (KiB) and all of them by WRITE_SIZE
    _write(f, [(1, COPY, 1, "FETCH_SIZE", known / 2 / 1024, 0, 1),
               (2, FC1, 1, "FETCH_SIZE", 100_000.0, 0, 1),
               (3, FC1, 1, "FETCH_SIZE", 300_000.0, 0, 1)])
    _write(w, [(1, COPY, 1, "WRITE_SIZE", known / 1024, 0, 1),
               (2, FC1, 1, "WRITE_SIZE", 50_000.0, 0, 1),
               (3, FC1, 1, "WRITE_SIZE", 50_000.0, 0, 1)])
    out = tmp_path / "t.json"
    traffic.main(["traffic", str(f), str(w), str(mib), str(out)])
    rec = json.load(open(out))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fc1_hbm_bytes_per_launch"] == 2.0 * 200_000 * 1024 + 50_000 * 1024
    assert rec["gemm_source_sha256"] == traffic.gemm_source_hash()


def test_bench_refuses_more_than_one_gpu():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_stats_span_of_back_to_back_launches(tmp_path):
    p = tmp_path / "kt.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        # three steps: hist at t0, entries ending 20 + i us later; an unrelated
        # kernel in between does not end a span
        for i in range(3):
            t0 = 1_000_000 * i
            w.writerow({"Kernel_Name": "void nvfp4::route_hist_quant_kernel<8, 2>(x)", "Grid_Size_X": 1,
                        "Start_Timestamp": t0, "End_Timestamp": t0 + 10_000})
            w.writerow({"Kernel_Name": "nvfp4::other_kernel(x)", "Grid_Size_X": 1,
                        "Start_Timestamp": t0 + 10_500, "End_Timestamp": t0 + 11_000})
            w.writerow({"Kernel_Name": "nvfp4::route_scan_entries_kernel(x)", "Grid_Size_X": 1,
                        "Start_Timestamp": t0 + 12_000, "End_Timestamp": t0 + 20_000 + 1000 * i})
    s = kernel_stats.span(str(p), "route_hist_quant", "route_scan_entries", 2)
    assert "last 2 of 3 spans" in s and "median 22.0 us" in s and "min 21.0" in s


def test_traffic_kernel_table_scales_per_dispatch(tmp_path):
    mib = 8
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    names = ["Kernel_Name", "Grid_Size_X", "Dispatch_Id", "Counter_Name", "Counter_Value"]
    for path, counter, copy_kib in ((f, "FETCH_SIZE", mib * 512), (w, "WRITE_SIZE", mib * 1024)):
        with open(path, "w", newline="") as fo:
            wr = csv.DictWriter(fo, fieldnames=names)
            wr.writeheader()
            wr.writerow({"Kernel_Name": "bitwise_not_kernel", "Grid_Size_X": 1, "Dispatch_Id": 1,
                         "Counter_Name": counter, "Counter_Value": copy_kib})
            # first dispatch (warm-up) 999 KiB, then 100 and 300 KiB, the
            # second split over two counter instances
            for d, v in ((2, [999]), (3, [100]), (4, [150, 150])):
                for x in v:
                    wr.writerow({"Kernel_Name": "void nvfp4::route_hist_quant_kernel<8, 2>(a)",
                                 "Grid_Size_X": 64, "Dispatch_Id": d, "Counter_Name": counter,
                                 "Counter_Value": x})
    t = traffic.kernel_table("route", str(f), str(w), mib)
    row = [l for l in t.splitlines() if l.startswith("| `route")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    # fetch counts scale by 2 (the copy's 8 MiB read shows as 4 MiB), writes by 1
    assert cells == ["`route_hist_quant_kernel<8, 2>`", "64", "%.2f" % (200 * 1024 * 2 / 1e6),
                     "%.2f" % (200 * 1024 / 1e6)]
