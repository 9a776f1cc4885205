"""Turn rocprofv3 CSV output into the small summaries kept under profiles/.

  python -m tensor_gemm_reduction_amd.profiling stats  <kernel_stats.csv> <out.txt> <bench.json|-> <command...>
      Kernel durations (calls, average, min, max) of the library's kernels,
      next to the HIP-event average the same bench run printed.

  python -m tensor_gemm_reduction_amd.profiling traffic <workload> <sched> <kernel-substring>
          <fetch.csv> <write.csv> <copy_fetch.csv> <copy_write.csv> <copy_bytes> <out.json>
      HBM bytes per dispatch of one kernel from the FETCH_SIZE and WRITE_SIZE
      counters (KiB per dispatch), each scaled by the ratio between the true
      bytes of a plain device copy of known size and what the same counter
      reports for it.  The record carries a hash of the kernel sources; the
      benchmark only reports it while the sources still match.

  python -m tensor_gemm_reduction_amd.profiling mfma <counter dir> <kernel-substring> <out.txt> <command...>
      Matrix-core busy fraction, the clock the GPU ran at and TFLOP/s per
      dispatch, from one --pmc pass over MFMA_COUNTERS.

  python -m tensor_gemm_reduction_amd.profiling overlap <trace dir> <dispatches per step> <out.txt> <command...>
      The last step's dispatches of the library's kernels (queue, start and
      end relative to the step), and how long GEMM and reduction kernels ran
      at the same time: the two-stream scheduler's overlap, from a
      --kernel-trace run.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")


def _code_only(text: str) -> str:
    """C/C++ source without comments and whitespace: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def source_hash() -> str:
    """sha256 over the code of libtpfuse's sources (what the counters
    describe); comments and whitespace do not change it."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                h.update(name.encode())
                h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _rows(path_or_dir: str, suffix: str):
    paths = [path_or_dir] if os.path.isfile(path_or_dir) else \
        glob.glob(os.path.join(path_or_dir, "**", "*" + suffix), recursive=True)
    for p in paths:
        with open(p) as f:
            yield from csv.DictReader(f)


def last_dispatches(trace_path: str, name_sub: str, k: int):
    """Average duration (us) of the last k dispatches of each kernel whose name
    contains name_sub, summed over those kernels: one launch per step gives
    that launch's average; the fold scheduler's two launches per step (the
    partial GEMMs, then the last shard with the fold epilogue) give the
    average of the pair."""
    by_name = {}
    for r in _rows(trace_path, "kernel_trace.csv"):
        if name_sub in r["Kernel_Name"]:
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            by_name.setdefault(r["Kernel_Name"], []).append((t0, t1 - t0))
    if not by_name:
        return None
    total, n = 0.0, 0
    for name in by_name:
        last = sorted(by_name[name])[-k:]
        total += sum(d for _, d in last) / len(last) / 1e3
        n = len(last)
    names = sorted(by_name, key=lambda m: -sum(d for _, d in by_name[m]))
    label = names[0] if len(names) == 1 else f"{len(names)} kernels per step ({', '.join(m[:40] for m in names)})"
    return label, total, n


def _union(intervals):
    """Merge [start, end) intervals; returns the sorted disjoint list."""
    out = []
    for a, b in sorted(intervals):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _covered(u):
    return sum(b - a for a, b in u)


def _intersect(u, v):
    """Length of the intersection of two disjoint sorted interval lists."""
    i = j = 0
    total = 0
    while i < len(u) and j < len(v):
        lo, hi = max(u[i][0], v[j][0]), min(u[i][1], v[j][1])
        if hi > lo:
            total += hi - lo
        if u[i][1] < v[j][1]:
            i += 1
        else:
            j += 1
    return total


def kernel_kind(name: str) -> str:
    """'reduce' for the reduction kernel, 'fold' for the shard-GEMM tiles
    whose epilogue folds the reduction (tile_kernel's last template argument
    2..5), 'gemm' for the other GEMM tiles."""
    if "reduce" in name:
        return "reduce"
    if "tile_kernel" in name:
        head = name.split("(")[0].rstrip(">").rstrip()
        last = head.rsplit(",", 1)[-1].strip()
        if last.isdigit() and int(last) >= 2:
            return "fold"
    return "gemm"


def overlap(trace_path: str, per_step: int, out_path: str, command: str) -> dict:
    """Summarise the last `per_step` dispatches of the library's kernels: how
    long the reduction ran beside GEMM work.  The reduction is either the
    reduction kernel or the fold-epilogue launches (which also compute the
    last shard's GEMM tiles)."""
    rows = [r for r in _rows(trace_path, "kernel_trace.csv") if "tpf::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    step = rows[-per_step:]
    t0 = min(int(r["Start_Timestamp"]) for r in step)
    t1 = max(int(r["End_Timestamp"]) for r in step)
    kinds = {kernel_kind(r["Kernel_Name"]) for r in step}
    red_kind = "reduce" if "reduce" in kinds else "fold"
    kind = lambda r: kernel_kind(r["Kernel_Name"])  # noqa: E731
    spans = {"gemm": [], "reduce": [], "fold": []}
    lines = [f"# rocprofv3 kernel trace: the last step's {per_step} dispatches (microseconds from the step's first start)",
             f"# command: {command}", "",
             f"{'#':>3s} {'kind':6s} {'queue':>5s} {'start_us':>9s} {'end_us':>9s} {'dur_us':>8s}"]
    for i, r in enumerate(step):
        a, b = int(r["Start_Timestamp"]) - t0, int(r["End_Timestamp"]) - t0
        spans[kind(r)].append((a, b))
        lines.append(f"{i:3d} {kind(r):6s} {r.get('Queue_Id', '?'):>5s} {a / 1e3:9.2f} {b / 1e3:9.2f} {(b - a) / 1e3:8.2f}")
    g, red = _union(spans["gemm"]), _union(spans[red_kind])
    res = {"step_us": (t1 - t0) / 1e3, "gemm_busy_us": _covered(g) / 1e3, "reduce_busy_us": _covered(red) / 1e3,
           "both_us": _intersect(g, red) / 1e3, "reduction_carrier": red_kind}
    res["reduce_hidden_frac"] = res["both_us"] / res["reduce_busy_us"] if res["reduce_busy_us"] else 0.0
    what = "a reduction kernel" if red_kind == "reduce" else "a fold-epilogue launch (last shard's tiles + reduction)"
    lines += ["", f"step {res['step_us']:.2f} us; a plain GEMM kernel running {res['gemm_busy_us']:.2f} us; "
                  f"{what} running {res['reduce_busy_us']:.2f} us, of which {res['both_us']:.2f} us "
                  f"({100 * res['reduce_hidden_frac']:.0f} %) beside a plain GEMM kernel"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return res


def counter_per_dispatch(path: str, counter: str, kernel_sub: str) -> float:
    """Per-dispatch average of `counter` for each kernel whose name contains
    kernel_sub, summed over those kernels (see last_dispatches)."""
    by_name = {}
    for r in _rows(path, "counter_collection.csv"):
        if r.get("Counter_Name") == counter and kernel_sub in r.get("Kernel_Name", ""):
            by_name.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not by_name:
        raise SystemExit(f"no {counter} samples for kernels matching {kernel_sub!r} in {path}")
    return sum(sum(v) / len(v) for v in by_name.values())


def stats(csv_path: str, out_path: str, command: str, bench_json: str = "", name_filter=("tpf::", "copyBuffer"),
          width: int = 90) -> None:
    lines = [f"# rocprofv3 kernel statistics (durations in microseconds)", f"# command: {command}", ""]
    lines.append(f"{'kernel':{width}s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
    for r in _rows(csv_path, "kernel_stats.csv"):
        name = r["Name"]
        if not any(f in name for f in name_filter):
            continue
        lines.append(f"{name[:width]:{width}s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")
    if bench_json and os.path.exists(bench_json) and "yardstick" in open(bench_json).read():
        with open(bench_json) as f:
            rec = json.loads(f.read().strip().splitlines()[-1])
        lines += ["", f"# bench.py --yardstick (same run): " + json.dumps(rec)]
    elif bench_json and os.path.exists(bench_json):
        # The same command's own JSON line: its HIP-event average of the
        # dominant kernel must agree with the rocprofv3 average above.
        with open(bench_json) as f:
            rec = json.loads(f.read().strip().splitlines()[-1])
        r = rec["roofline"]
        k = int(r.get("timed_launches") or 0)
        last = last_dispatches(csv_path, r["kernel"].split()[0], k) if k else None
        if last:
            name, avg_us, n = last
            lines += ["", f"# rocprofv3, the last {n} dispatches of {name[:150]}",
                      f"#   (the bench's timed launches; earlier ones are its settle and warmup steps): "
                      f"average {avg_us:.2f} us"]
        lines += ["", f"# bench.py (same run): dominant kernel = {r['kernel']}",
                  f"#   HIP-event average over {r.get('timed_launches')} timed launches: "
                  f"{1e3 * r['avg_kernel_ms']:.2f} us; roofline {r['achieved']} {r['unit']} of {r['peak']} "
                  f"(frac {r['frac']}); value {rec['value']} {rec['unit']}"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def traffic(workload, sched, kernel_sub, fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes, out_path,
            command=""):
    copy_bytes = int(copy_bytes)
    cf = counter_per_dispatch(cfetch_csv, "FETCH_SIZE", "copyBuffer")
    cw = counter_per_dispatch(cwrite_csv, "WRITE_SIZE", "copyBuffer")
    fetch_scale = copy_bytes / (cf * 1024.0)
    write_scale = copy_bytes / (cw * 1024.0)
    f = counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel_sub)
    w = counter_per_dispatch(write_csv, "WRITE_SIZE", kernel_sub)
    rec = {
        "workload": workload,
        "sched": sched,
        "kernel": kernel_sub,
        "source_hash": source_hash(),
        "fetch_kib_per_dispatch": f,
        "write_kib_per_dispatch": w,
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": cf,
        "copy_write_kib": cw,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "hbm_read_bytes": f * 1024.0 * fetch_scale,
        "hbm_write_bytes": w * 1024.0 * write_scale,
        "hbm_bytes": f * 1024.0 * fetch_scale + w * 1024.0 * write_scale,
        "command": command,
    }
    with open(out_path, "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps(rec, indent=1))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT "
                 "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_WAVE_CYCLES GRBM_GUI_ACTIVE GRBM_COUNT")


def mfma(counter_dir: str, kernel_sub: str, out_path: str, command: str = "", xcds: int = 8, cus: int = 256,
         simds_per_cu: int = 4, flop_per_clk_simd: int = 1024) -> None:
    """Matrix-core utilisation of each dispatch of the kernels matching
    kernel_sub, from one rocprofv3 --pmc pass over MFMA_COUNTERS:
      clock      = GRBM_GUI_ACTIVE per XCD / dispatch duration (the clock the
                   GPU actually ran at, against 2.4 GHz for the published peak)
      MFMA busy  = SQ_VALU_MFMA_BUSY_CYCLES / (active cycles x SIMDs)
      TFLOP/s    = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / duration
      peak@clock = SIMDs x 1024 bf16 flop/clk x clock."""
    by = {}
    for r in _rows(counter_dir, "counter_collection.csv"):
        if kernel_sub not in r.get("Kernel_Name", ""):
            continue
        d = by.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                             "dur": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    if not by:
        raise SystemExit(f"no dispatches of {kernel_sub!r} in {counter_dir}")
    simds = cus * simds_per_cu
    lines = ["# rocprofv3 hardware counters: matrix-core utilisation per dispatch",
             f"# command: {command}", f"# counters: {MFMA_COUNTERS}", "",
             f"{'dispatch':>8s} {'kernel':40s} {'dur_us':>8s} {'clk_GHz':>8s} {'mfma_busy':>9s} "
             f"{'TFLOP/s':>8s} {'peak@clk':>8s} {'frac@clk':>8s} {'frac@2.4':>8s} {'lds_conf':>8s}"]
    for k in sorted(by, key=int):
        d = by[k]
        dur = d["dur"] * 1e-9
        active = d["GRBM_GUI_ACTIVE"] / xcds
        clk = active / dur
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * simds)
        tf = d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / dur / 1e12
        peak = simds * flop_per_clk_simd * clk / 1e12
        lines.append(f"{k:>8s} {d['name'][:40]:40s} {dur * 1e6:8.1f} {clk / 1e9:8.3f} {100 * busy:8.1f}% "
                     f"{tf:8.0f} {peak:8.0f} {tf / peak:8.3f} {tf / (simds * flop_per_clk_simd * 2.4e9 / 1e12):8.3f} "
                     f"{int(d['SQ_LDS_BANK_CONFLICT']):8d}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_traffic(workload: str, profiles_dir: str):
    """HBM bytes per dispatch recorded for `workload`, or None if absent or stale."""
    path = os.path.join(profiles_dir, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec


if __name__ == "__main__":
    cmd = sys.argv[1]
    if cmd == "stats":
        # stats <csv> <out.txt> <bench_json or -> <command...>
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[5:]), "" if sys.argv[4] == "-" else sys.argv[4])
    elif cmd == "traffic":
        traffic(*sys.argv[2:11], command=" ".join(sys.argv[11:]))
    elif cmd == "yardstick":
        # yardstick <csv dir> <out.txt> <bench_json> <command...>: the vendor GEMM kernels, full names
        stats(sys.argv[2], sys.argv[3], " ".join(sys.argv[5:]), sys.argv[4], name_filter=("Cijk",), width=400)
    elif cmd == "overlap":
        # overlap <trace dir> <dispatches per step> <out.txt> <command...>
        overlap(sys.argv[2], int(sys.argv[3]), sys.argv[4], command=" ".join(sys.argv[5:]))
    elif cmd == "mfma":
        # mfma <counter dir> <kernel-substring> <out.txt> <command...>
        mfma(sys.argv[2], sys.argv[3], sys.argv[4], command=" ".join(sys.argv[5:]))
    else:
        raise SystemExit(__doc__)
