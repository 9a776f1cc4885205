"""Host-side checks of the rocprofv3 summaries (tensor_gemm_reduction_amd.profiling)
on small synthetic CSV files in rocprofv3's column layout: one launch per
step, the fold scheduler's two launches per step, counter scaling against the
copy calibration, and the matrix-core / clock summary."""
import csv
import json

from tensor_gemm_reduction_amd import profiling as P

TRACE_COLS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Queue_Id"]
COUNTER_COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, cols, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def trace(tmp_path, launches):
    """launches: (name, start_ns, duration_ns) in any order."""
    d = tmp_path / "trace"
    d.mkdir()
    write_csv(d / "run_kernel_trace.csv", TRACE_COLS,
              [{"Kernel_Name": n, "Start_Timestamp": t0, "End_Timestamp": t0 + dt, "Queue_Id": 0}
               for n, t0, dt in launches])
    return str(d)


def test_last_dispatches_one_kernel(tmp_path):
    gemm, red = "tpf::tile_kernel<A, 0, 0>", "tpf::reduce_rows_kernel"
    launches = []
    for i in range(6):   # settle steps at 900 ns, timed steps at 500 ns
        launches.append((gemm, 10_000 * i, 900 if i < 3 else 500))
        launches.append((red, 10_000 * i + 5_000, 70))
    name, avg_us, n = P.last_dispatches(trace(tmp_path, launches), "tile_kernel", 3)
    assert name == gemm and n == 3
    assert abs(avg_us - 0.5) < 1e-12          # reduce_rows does not match the substring


def test_last_dispatches_sums_the_fold_pair(tmp_path):
    first, fold = "tpf::tile_kernel<A, 0, 0>", "tpf::tile_kernel<A, 0, 2>"
    launches = []
    for i in range(5):
        launches.append((first, 10_000 * i, 3000))
        launches.append((fold, 10_000 * i + 4000, 1000 + 100 * i))
    label, avg_us, n = P.last_dispatches(trace(tmp_path, launches), "tile_kernel", 2)
    assert n == 2 and label.startswith("2 kernels per step")
    # last two steps: 3000 + 1300 and 3000 + 1400 ns
    assert abs(avg_us - (3.0 + 1.35)) < 1e-12


def counters(tmp_path, name, rows):
    d = tmp_path / name
    d.mkdir()
    write_csv(d / "run_counter_collection.csv", COUNTER_COLS, rows)
    return str(d)


def test_traffic_scales_by_the_copy_calibration(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    nbytes = 1 << 30
    # the copy's counters report half of the bytes read and all of the bytes written
    cf = counters(tmp_path, "cf", [{"Dispatch_Id": 1, "Kernel_Name": copy, "Counter_Name": "FETCH_SIZE",
                                    "Counter_Value": nbytes / 2 / 1024, "Start_Timestamp": 0, "End_Timestamp": 1}])
    cw = counters(tmp_path, "cw", [{"Dispatch_Id": 1, "Kernel_Name": copy, "Counter_Name": "WRITE_SIZE",
                                    "Counter_Value": nbytes / 1024, "Start_Timestamp": 0, "End_Timestamp": 1}])
    k0, k2 = "tpf::tile_kernel<A, 0, 0>", "tpf::tile_kernel<A, 0, 2>"
    fetch = [{"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": v,
              "Start_Timestamp": 0, "End_Timestamp": 1}
             for i, (k, v) in enumerate([(k0, 1000.0), (k2, 300.0), (k0, 1000.0), (k2, 300.0)])]
    write = [{"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": v,
              "Start_Timestamp": 0, "End_Timestamp": 1}
             for i, (k, v) in enumerate([(k0, 600.0), (k2, 20.0), (k0, 600.0), (k2, 20.0)])]
    f = counters(tmp_path, "f", fetch)
    w = counters(tmp_path, "w", write)
    out = tmp_path / "traffic.json"
    P.traffic("wl", "auto", "tile_kernel", f, w, cf, cw, nbytes, str(out))
    rec = json.loads(out.read_text())
    assert abs(rec["fetch_scale"] - 2.0) < 1e-12 and abs(rec["write_scale"] - 1.0) < 1e-12
    # per step: both kernels of the pair, summed
    assert rec["hbm_read_bytes"] == (1000.0 + 300.0) * 1024 * 2
    assert rec["hbm_write_bytes"] == (600.0 + 20.0) * 1024
    assert rec["source_hash"] == P.source_hash()


def test_mfma_summary(tmp_path):
    k = "tpf::tile_kernel<A,0,0>"                      # no spaces: the row is split on whitespace below
    dur_ns = 500_000                                   # 0.5 ms
    clk = 2.0e9
    active_per_xcd = clk * dur_ns * 1e-9               # 1e6 cycles
    simds = 256 * 4
    busy = 0.5 * active_per_xcd * simds                # half of the SIMD cycles
    flops = 1.0e15 * dur_ns * 1e-9                     # 1 PFLOP/s
    vals = {"GRBM_GUI_ACTIVE": active_per_xcd * 8, "SQ_VALU_MFMA_BUSY_CYCLES": busy,
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": flops / 512, "SQ_LDS_BANK_CONFLICT": 0.0}
    rows = [{"Dispatch_Id": 7, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v,
             "Start_Timestamp": 1000, "End_Timestamp": 1000 + dur_ns} for c, v in vals.items()]
    d = counters(tmp_path, "m", rows)
    out = tmp_path / "m.txt"
    P.mfma(d, "tile_kernel", str(out), command="test")
    line = out.read_text().strip().splitlines()[-1].split()
    # dispatch, kernel, dur_us, clk_GHz, busy, TFLOP/s, peak@clk, frac@clk, frac@2.4, conflicts
    assert line[0] == "7"
    assert abs(float(line[2]) - 500.0) < 0.05
    assert abs(float(line[3]) - 2.0) < 5e-4
    assert line[4] == "50.0%"
    assert abs(float(line[5]) - 1000) < 0.5
    peak = simds * 1024 * clk / 1e12                   # 2097 TFLOP/s at 2.0 GHz
    assert abs(float(line[6]) - peak) < 0.5
    assert abs(float(line[7]) - 1000 / peak) < 5e-4


def test_overlap_of_gemm_and_reduction(tmp_path):
    g, r = "tpf::tile_kernel<A, 0, 0>", "tpf::reduce_rows_kernel"
    # an earlier step, then the step summarised: GEMMs 0-100, 90-200, 200-300 ns,
    # reductions 95-120 (inside the GEMMs), 290-330 (10 ns inside) and 340-350 (alone)
    launches = [(g, 0, 50), (r, 60, 10)]
    base = 1000
    launches += [(g, base, 100), (g, base + 90, 110), (g, base + 200, 100),
                 (r, base + 95, 25), (r, base + 290, 40), (r, base + 340, 10)]
    out = tmp_path / "o.txt"
    res = P.overlap(trace(tmp_path, launches), 6, str(out), "test")
    assert abs(res["step_us"] - 0.350) < 1e-12
    assert abs(res["gemm_busy_us"] - 0.300) < 1e-12
    assert abs(res["reduce_busy_us"] - 0.075) < 1e-12
    assert abs(res["both_us"] - 0.035) < 1e-12        # 25 + 10 ns
    assert len(out.read_text().splitlines()) == 4 + 6 + 2


def test_kernel_kind_names_fold_launches():
    cfg = "tpf::TileCfg<256, 256, 2, 4, 2, 64, 0, 0, 0, 2>"
    assert P.kernel_kind(f"void tpf::tile_kernel<{cfg}, 0, 0>(tpf::TileArgs)") == "gemm"
    assert P.kernel_kind(f"void tpf::tile_kernel<{cfg}, 0, 1>(tpf::TileArgs)") == "gemm"      # tile scheduler
    for red in (2, 3, 4, 5):
        assert P.kernel_kind(f"void tpf::tile_kernel<{cfg}, 0, {red}>(tpf::TileArgs)") == "fold"
    assert P.kernel_kind("tpf::reduce_rows_kernel(void const*, long, int)") == "reduce"
    assert P.kernel_kind("void tpf::fused_kernel<A, 0>(tpf::FusedArgs)") == "gemm"


def test_overlap_with_fold_launches_as_the_reduction(tmp_path):
    """The chunked fold schedule: plain GEMM launches of chunk c+1 beside
    the fold-epilogue launch of chunk c."""
    g, f = "tpf::tile_kernel<A, 0, 0>(x)", "tpf::tile_kernel<A, 0, 2>(x)"
    launches = [(g, 0, 100), (f, 100, 50), (g, 110, 100), (f, 210, 50)]
    res = P.overlap(trace(tmp_path, launches), 4, str(tmp_path / "o.txt"), "test")
    assert res["reduction_carrier"] == "fold"
    assert abs(res["reduce_busy_us"] - 0.100) < 1e-12
    assert abs(res["both_us"] - 0.040) < 1e-12         # fold 100-150 beside GEMM 110-210
