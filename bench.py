#!/usr/bin/env python3
"""Benchmark of the fused tensor-parallel MatMul + reduction on one MI355X.

One step = one fused call of the whole path (all shard GEMMs, the chunk-ready
scheduling and the fixed-order reduction) over one batch of synthetic,
HBM-resident inputs.  Default workload: the Llama-style MLP down projection
(row-parallel, p=4 shards X_k [4096,4096] . W_k [4096,4096], 8 M-chunks,
AllReduce layout, bf16 out).

Before the W warmup steps, untimed steps run for at least --settle-ms
(default 300 ms): the clocks take that long under sustained load to reach
their steady state, and the K timed steps are meant to see it.

Prints ONE JSON line.  `value` is whole-step TFLOP/s of the library call
(algorithmic 2*M*N*K_total over the wall time per step; the default
scheduler is AUTO, which at this workload runs the fold scheduler: the GEMMs
of shards 0..p-2 into fp32 partials, then the last shard's GEMM whose epilogue
sums them; `config.sched_ran` names what ran); `roofline` prices the step's
dominant kernel (for the fold scheduler, its pair of launches) against
the bf16 dense MFMA peak, its average duration measured by HIP events that
the library records around that launch on the stream it is launched on;
`modes` gives the GEMM-only, reduce-only, unfused, two-stream, persistent
and tile-scheduler times and the exposed reduction time (step minus
GEMM-only); `cpu_baseline` times the CPU oracle on a bounded sample of rows
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
ROTATION_BYTES = 512 << 20    # inputs streamed per rotation of the input sets: twice the last-level cache


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20, or 100 for workloads under 0.1 TFLOP per step)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp_down")
    ap.add_argument("--chunks", type=int, default=0, help="0 = the workload's default")
    ap.add_argument("--sched", default="auto",
                    help="auto (= unfused on one GPU), unfused, persistent, two_stream, tile, gemm_only")
    ap.add_argument("--message", default="fp32", choices=["fp32", "bf16"],
                    help="precision of the shard partials (the 2-byte message variant: bf16)")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated to defeat the 256 MB last-level cache (default: enough that one "
                         "rotation streams at least 512 MiB, 2 to 8 sets)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps run for at least this long before the warmup steps: the GPU's clocks "
                         "take ~0.1-0.2 s of sustained load to reach their steady state")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the timed steps in one HIP graph and report its replay time per step")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--modes", default="gemm_only,reduce_only,unfused,two_stream,persistent,tile,fold,auto")
    ap.add_argument("--yardstick", action="store_true",
                    help="only time the vendor GEMM (torch.matmul -> hipBLASLt) on the workload's shard GEMMs, "
                         "with the weights as given ([K][N]) and K-contiguous, for comparison")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the p simulated ranks all live on one MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import torch
    from tensor_gemm_reduction_amd import inputs, tpfuse as tp

    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters
        # give the scale between those counters and real HBM bytes.
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "note": "plain device copy for counter calibration"}), flush=True)
        return

    if args.steps is None:       # short steps need more repetitions for a steady figure
        args.steps = 100 if inputs.WORKLOADS[args.workload].flops() < 1e11 else 20

    if args.yardstick:
        yardstick(args, inputs.WORKLOADS[args.workload])
        return

    tp.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    wl = inputs.WORKLOADS[args.workload]
    n = args.chunks or wl.default_chunks
    dev = "cuda"
    handle = tp.Handle(0)

    # --- inputs (generated on the GPU with seeded generators, kept resident) ---
    sets = [inputs.make_inputs(wl, seed=0, device=dev)]
    if args.sets <= 0:
        set_bytes = sum(t.numel() * t.element_size() for t in list(sets[0].X) + list(sets[0].W))
        args.sets = min(8, max(2, -(-ROTATION_BYTES // set_bytes)))
    for s in range(1, args.sets):
        sets.append(inputs.make_inputs(wl, seed=s, device=dev))
    M, N, K, p = wl.M, wl.N, wl.K, wl.p
    flops = wl.flops()
    kflops = flops / 2 if wl.op == "mlp_sp" else flops    # the timed launch of the MLP block is FC2
    msg = args.message

    if wl.op in ("allreduce", "reducescatter"):
        op_id = tp.OP_MATMUL_ALLREDUCE if wl.op == "allreduce" else tp.OP_MATMUL_REDUCESCATTER
        ws = torch.empty(tp.workspace_size(op_id, p, M, N, K, n, message=msg), dtype=torch.uint8, device=dev)
        if wl.op == "allreduce":
            Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        else:
            Y = [torch.empty((M // p, N), dtype=torch.bfloat16, device=dev) for _ in range(p)]

        def call(i, sched):
            inp = sets[i % len(sets)]
            if wl.op == "allreduce":
                tp.matmul_allreduce(inp.X, inp.W, n_chunks=n, sched=sched, Y=Y, ws=ws, handle=handle, message=msg)
            else:
                tp.matmul_reducescatter(inp.X, inp.W, n_chunks=n, sched=sched, Y=Y, ws=ws, handle=handle,
                                        message=msg)
        ws_bytes = ws.numel()
    elif wl.op == "dx":
        ws = torch.empty(tp.workspace_size(tp.OP_MATMUL_DX, p, M, K, N, n, message=msg), dtype=torch.uint8,
                         device=dev)
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)

        def call(i, sched):
            inp = sets[i % len(sets)]
            tp.matmul_dx(inp.X, inp.W, tp.ALLREDUCE, n_chunks=n, sched=sched, dX=dX, ws=ws, handle=handle,
                         message=msg)
        ws_bytes = ws.numel()
    elif wl.op == "mlp_sp":
        # AllGather -> FC1 + GeLU -> FC2 -> ReduceScatter; N = hidden, K = ffn shard
        ws = torch.empty(tp.workspace_size(tp.OP_MLP_SP, p, M, N, K, n, message=msg), dtype=torch.uint8,
                         device=dev)
        XG = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        Hs = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(p)]
        Ys = [torch.empty((M // p, N), dtype=torch.bfloat16, device=dev) for _ in range(p)]

        def call(i, sched):
            inp = sets[i % len(sets)]
            tp.mlp_sp(inp.X, inp.W[:p], inp.W[p:], n_chunks=n, sched=sched, X_gathered=XG, H=Hs, Y=Ys, ws=ws,
                      handle=handle, message=msg)
        ws_bytes = ws.numel()
    elif wl.op == "rowpar_dx":
        # dX_k [M, K] = dY W_k^T, bf16 out (the gradient handed to the layer below)
        dXs = [torch.empty((M, K), dtype=torch.bfloat16, device=dev) for _ in range(p)]

        def call(i, sched):
            inp = sets[i % len(sets)]
            tp.rowpar_dx(inp.X[0], inp.W, dX=dXs, handle=handle)
        ws_bytes = 0
        args.modes = "none"      # no reduction: there are no schedules to compare
    elif wl.op.startswith("wgrad"):
        # dW_k [K, N] = A_k^T B_k over M rows, fp32 out (the optimizer's input)
        dWs = [torch.empty((K, N), dtype=torch.float32, device=dev) for _ in range(p)]
        operands = [inputs.weight_grad_operands(inp) for inp in sets]

        def call(i, sched):
            A, B = operands[i % len(operands)]
            tp.weight_grad(A, B, dW=dWs, handle=handle)
        ws_bytes = 0
        args.modes = "none"      # no reduction: there are no schedules to compare
    else:  # allgather
        XG = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def call(i, sched):
            inp = sets[i % len(sets)]
            tp.allgather_matmul(inp.X, inp.W[0], n_chunks=n, sched=sched, X_gathered=XG, Y=Y, handle=handle)
        ws_bytes = 0

    stream = torch.cuda.current_stream()

    def time_slice(sched, steps, warmup):
        """Per-step event times (ms) and wall seconds of `steps` steps of one mode.
        No synchronisation between the warmup and the timed steps: the GPU is
        still busy with the warmup while the host enqueues them, so the
        events do not see host launch latency."""
        for i in range(warmup):
            call(i, sched)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            evs[i][0].record(stream)
            call(i, sched)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs], time.perf_counter() - t0

    def time_modes(mode_list, steps):
        """Median step time of each mode, measured round-robin (four steps of
        every mode per round) so that clock and temperature drift over the
        run affects all modes alike instead of favouring the first ones."""
        per = {m: [] for m in mode_list}
        wall = {m: 0.0 for m in mode_list}
        chunk = 4
        for r in range(max(2, (steps + chunk - 1) // chunk)):
            for m in mode_list:
                t, w = time_slice(m, chunk, 1 if r else 2)
                per[m] += t
                wall[m] += w
        out = {}
        for m in mode_list:
            v = sorted(per[m])
            out[m] = {"ms_median": v[len(v) // 2], "ms_min": v[0], "ms_mean": sum(v) / len(v),
                      "wall_ms_per_step": 1e3 * wall[m] / len(v)}
        return out

    # --- settle (untimed, time-bounded), then the warmup steps ---
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        call(settle_steps, args.sched)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()      # measure GPU progress, not how fast the host can enqueue
    torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3

    # --- the timed region: exactly `steps` fused steps ---
    for i in range(args.warmup):
        call(i, args.sched)
    torch.cuda.synchronize()
    handle.set_kernel_timing(True)   # events around each step's dominant kernel launch
    # One event pair around all K steps: a timed event costs the stream a few
    # microseconds, so none is recorded between the steps beyond the pair the
    # library records around each dominant launch.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        call(i, args.sched)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = handle.sync_status()
    if st != tp.OK:
        raise RuntimeError(f"fused path reported status {st}")
    launch_ms = handle.kernel_times(args.steps)
    handle.set_kernel_timing(False)
    # the scheduler the library ran for args.sched (AUTO resolved): it names
    # the timed kernels and sets their algorithmic bytes
    ran = handle.last_sched() or args.sched
    kbytes = kernel_bytes(wl, 2 if args.message == "bf16" else 4, ran)
    step_event_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = 1e3 * wall / args.steps
    kern_ms = launch_ms if launch_ms else [step_event_ms]   # two_stream records no single dominant launch
    avg_kernel_ms = sum(kern_ms) / len(kern_ms)
    value = flops / (ms_per_step * 1e-3) / 1e12
    # The dominant kernel is priced against MFMA or HBM, whichever bounds it:
    # its algorithmic flops per byte against the ridge point peak_flops / peak_bw.
    hbm_bound = kflops / kbytes < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        achieved, peak, unit = kbytes / (avg_kernel_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = kflops / (avg_kernel_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"

    # --- the same steps captured in one HIP graph (launch overhead removed) ---
    graph = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(0, args.sched)          # warm the side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(args.steps):
                call(i, args.sched)
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        g0.record(stream)
        for _ in range(reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        st = handle.sync_status()
        if st != tp.OK:
            raise RuntimeError(f"graph replay reported status {st}")
        gms = g0.elapsed_time(g1) / (reps * args.steps)
        graph = {"ms_per_step": round(gms, 4), "value": round(flops / (gms * 1e-3) / 1e12, 3),
                 "steps_per_graph": args.steps, "replays": reps}
        del g

    # --- the other modes (measurement context) ---
    mode_list = [x for x in args.modes.split(",") if x and x != "none"]
    modes = time_modes(mode_list, max(6, args.steps // 2)) if mode_list else {}
    extra = {}
    if "gemm_only" in modes and args.sched in modes:
        t_f = modes[args.sched]["ms_median"]
        t_g = modes["gemm_only"]["ms_median"]
        exposed = t_f - t_g
        extra = {"exposed_reduce_ms": exposed, "exposed_over_fused": exposed / t_f}
        if "reduce_only" in modes:
            extra["exposed_over_reduce_only"] = exposed / modes["reduce_only"]["ms_median"]
        if "unfused" in modes:
            extra["fused_over_unfused"] = t_f / modes["unfused"]["ms_median"]
        # the pages' two-engine model with measured whole-op times split per chunk
        t_c = t_g / n
        t_m = modes.get("reduce_only", {"ms_median": 0.0})["ms_median"] / n
        extra["model_pipeline_ms"] = t_c + (n - 1) * max(t_c, t_m) + t_m
        extra["model_serial_ms"] = n * (t_c + t_m)

    # --- HBM bytes per launch from the committed counter summary (if current) ---
    from tensor_gemm_reduction_amd import profiling
    rec = profiling.load_traffic(wl.name, os.path.join(ROOT, "profiles"))
    traffic = round(rec["hbm_bytes"]) if rec and rec.get("sched") == args.sched else None

    # --- CPU oracle baseline on a bounded sample of rows ---
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, sets[0], args.cpu_seconds)

    out = {
        "metric": "TFLOP/s & % bf16 MFMA peak, fused MatMul+reduce; exposed reduce ms vs unfused",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "op": wl.op, "p": p, "M": M, "N": N, "K_shard": K,
                   "n_chunks": n, "sched": args.sched, "sched_ran": ran, "out": "bf16", "message": args.message,
                   "input_sets": args.sets,
                   "workspace_bytes": ws_bytes, "note": wl.note},
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic,
                     "algorithmic_bytes": kbytes, "algorithmic_flops": kflops,
                     "kernel": kernel_name(ran, wl.op),
                     "avg_kernel_ms": round(avg_kernel_ms, 4),
                     "timed_launches": len(launch_ms) if launch_ms else args.steps,
                     "avg_step_event_ms": round(step_event_ms, 4)},
        "cpu_baseline": cpu,
        "graph": graph,
        "modes": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in modes.items()},
        **{k: round(v, 4) for k, v in extra.items()},
    }
    print(json.dumps(out), flush=True)


def yardstick(args, wl):
    """The vendor library on the same shard GEMMs (run, not read): p products
    X_k [M, K] @ W_k per step, bf16 in and out, with W_k as the library's
    callers store it ([K][N], the "NN" case) and K-contiguous (a transposed
    copy, the "NT" case).  Context for the roofline, not part of the path."""
    import torch
    if wl.op not in ("allreduce", "reducescatter"):
        raise SystemExit("--yardstick covers the row-parallel workloads (allreduce, reducescatter)")
    torch.manual_seed(0)
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    X = [torch.randn(M, K, device="cuda").to(torch.bfloat16) for _ in range(p)]
    W = [(torch.randn(K, N, device="cuda") * 0.02).to(torch.bfloat16) for _ in range(p)]
    Wt = [w.t().contiguous().t() for w in W]     # same values, K-contiguous storage
    out = {"yardstick": "torch.matmul (hipBLASLt)", "workload": wl.name, "p": p, "M": M, "N": N, "K": K}
    flops = 2.0 * p * M * N * K
    for name, ws in (("nn", W), ("nt", Wt)):
        def step():
            for k in range(p):
                X[k] @ ws[k]
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle_ms / 1e3:
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        out[f"{name}_ms_per_step"] = round(ms, 4)
        out[f"{name}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    print(json.dumps(out), flush=True)


def kernel_bytes(wl, part_bytes=4, sched="unfused"):
    """Algorithmic HBM bytes of one launch of the shard-GEMM kernel: every
    operand read once and every output written once (the partials of the
    reducing ops, `part_bytes` per element; the bf16 output of AllGather).
    For the fold scheduler's pair of launches: the operands once, the
    partials of p - 1 shards written and read back once, the bf16 result
    written once."""
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    if sched == "fold" and wl.op in ("allreduce", "reducescatter", "mlp_sp"):
        return p * (2.0 * M * K + 2.0 * K * N) + 2.0 * (p - 1) * part_bytes * M * N + 2.0 * M * N
    if sched == "fold" and wl.op == "dx":    # dY_k [M, N], W_k [K, N], dX [M, K]
        return p * (2.0 * M * N + 2.0 * K * N) + 2.0 * (p - 1) * part_bytes * M * K + 2.0 * M * K
    if wl.op == "allgather":
        return 2.0 * M * K + 2.0 * K * N + 2.0 * M * N
    if wl.op == "rowpar_dx":        # dY [M, N] (one, shared), W_k [K, N], dX_k [M, K] bf16
        return 2.0 * M * N + p * (2.0 * K * N + 2.0 * M * K)
    if wl.op.startswith("wgrad"):   # A_k [M, K], B_k [M, N], dW_k [K, N] fp32
        return p * (2.0 * M * K + 2.0 * M * N + 4.0 * K * N)
    if wl.op == "mlp_sp":           # FC2 launch: H_k [M, K], W2_k [K, N], partials [M, N]
        return p * (2.0 * M * K + 2.0 * K * N + part_bytes * M * N)
    if wl.op == "dx":      # dY_k [M, N], W_k [K, N], partials [M, K]
        return p * (2.0 * M * N + 2.0 * K * N + part_bytes * M * K)
    return p * (2.0 * M * K + 2.0 * K * N + part_bytes * M * N)


def kernel_name(sched, op=""):
    """The kernel (or, for the fold scheduler, the pair of launches) that
    dominates one step of the scheduler the library ran: what `roofline`
    prices."""
    if op.startswith("wgrad"):
        return "tile_kernel A_KM (weight-gradient GEMM tiles, transposed A)"
    if op == "rowpar_dx":
        return "tile_kernel NK (row-parallel input-gradient tiles, transposed weights, one dY for every shard)"
    if op == "mlp_sp":
        if sched == "fold":
            return ("tile_kernel pair (FC2: shards 0..p-2 into partials, then shard p-1 with the fold epilogue; "
                    "FC1 with GeLU runs before it)")
        return "tile_kernel RED=0 (FC2 shard GEMM tiles; FC1 with GeLU runs before it)"
    if sched == "persistent":
        return "fused_kernel (persistent: shard GEMM tiles + chunk reductions)"
    if sched == "fold":
        return "tile_kernel pair (shards 0..p-2 into partials, then shard p-1 with the fold epilogue)"
    if sched == "tile":
        return "tile_kernel RED=1 (shard GEMM tiles + last-arriver tile sums)"
    if sched == "two_stream":
        return "whole step (per-chunk GEMM and reduction kernels on three streams)"
    return "tile_kernel RED=0 (shard GEMM tiles)"


def cpu_baseline(wl, inp, seconds):
    """Time the CPU oracle on a bounded sample of output rows of the same inputs."""
    import numpy as np
    from oracle import tpf_oracle as O
    from tensor_gemm_reduction_amd import inputs

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    Xb = [inputs.bf16_to_bits(x) for x in inp.X]
    Wb = [inputs.bf16_to_bits(w) for w in inp.W]
    # output rows the sample is drawn from (a weight gradient's rows are K)
    M = wl.K if wl.op.startswith("wgrad") else wl.M

    def run(rows):
        r = np.arange(rows)
        t0 = time.perf_counter()
        if wl.op in ("allreduce", "reducescatter"):
            O.matmul_allreduce(Xb, Wb, rows=r)
        elif wl.op == "dx":
            O.matmul_dx(Xb, Wb, rows=r)
        elif wl.op == "rowpar_dx":
            O.rowpar_dx(Xb[0][:rows], Wb)
        elif wl.op.startswith("wgrad"):
            A, B = (Xb * wl.p, Wb) if wl.op == "wgrad_col" else (Xb, Wb * wl.p)
            O.weight_grad([a[:, :rows] for a in A], B)
        elif wl.op == "mlp_sp":
            x = O.allgather(Xb)[:rows]
            hid = [O.round_to_bf16_bits(O.gelu(x @ O.bf16_bits_to_f64(w))) for w in Wb[:wl.p]]
            O.matmul_allreduce(hid, Wb[wl.p:])
        else:
            xg = O.allgather(Xb)[:rows]
            _ = xg @ O.bf16_bits_to_f64(Wb[0])
        return time.perf_counter() - t0

    rows = min(M, 8)
    dt = run(rows)
    while dt < seconds / 4 and rows < M:
        rows = min(M, rows * 4)
        dt = run(rows)
    reps, total = 1, dt
    while rows == M and total < seconds:      # the whole workload is quick: repeat it for a steady figure
        total += run(rows)
        reps += 1
    per_row_flops = wl.flops() / M
    tflops = per_row_flops * rows * reps / total / 1e12
    return {"value": round(tflops, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {M} output rows of the same inputs (float64 numpy oracle, "
                      f"including bf16->f64 conversion), {reps} run(s), {total:.2f} s on {cpu_model()}"}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the CPU baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "an unknown CPU"


if __name__ == "__main__":
    main()
