#!/usr/bin/env python3
"""Benchmark of the fused tensor-parallel MatMul + reduction on one MI355X.

One step = one call of the whole path (every shard GEMM and the fixed-order
cross-shard reduction into the collective's output layout) over one batch of
synthetic, HBM-resident inputs.  The headline workload is the Llama-style
MLP down projection (row-parallel, p = 4 shards X_k [4096,4096] .
W_k [4096,4096], AllReduce layout, bf16 out) with the default scheduler
(AUTO: for this shape the last shard's GEMM epilogue folds the reduction;
`config.sched_ran` names what ran and `config.n_chunks_effective` how many
chunks it actually used).

Before the W warmup steps, untimed steps run for at least --settle-ms
(default 300 ms): the clocks take that long under sustained load to reach
their steady state, and the K timed steps are meant to see it.

Prints ONE JSON line.  `value` is whole-step TFLOP/s of the headline
(algorithmic 2*M*N*K_total over the wall time per step).  `roofline` prices
the step's dominant kernel(s) against the bf16 dense MFMA peak (or HBM for
decode shapes), timed by HIP events the library records around that launch
on the stream it is launched on.  `parity` compares the output of the timed
call with the float64 oracle on every row.  `modes` gives the GEMM-only,
reduce-only, unfused and chunked-scheduler times and the exposed reduction
(step minus GEMM-only).  `configs` repeats the measurement (a shorter one)
for every other configured workload: the worked example, the
sequence-parallel ReduceScatter, AllGather->MatMul, the column-parallel dX
(AllReduce and ReduceScatter layouts) and the decode shapes with their chunk
sweep.  `cpu_baseline` times the plain C oracle on a bounded sample of the
headline's rows on the host cores.
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
TARGET_MFMA_FRAC = 0.60       # goals stated for this path: large-M configs
TARGET_HBM_FRAC = 0.70        # decode-shaped config
TARGET_EXPOSED = 0.10         # exposed reduction / step

# The other configured workloads measured into `configs` after the headline:
# (record name, workload, semantic for dX, mode list).  Decode shapes also
# sweep the chunked schedulers over 1, 2 and 4 chunks.
CONFIGS = [
    ("worked", "worked", None),
    ("sp_rs", "sp_rs", None),
    ("ag_fwd", "ag_fwd", None),
    ("dx_bwd_ar", "dx_bwd", "allreduce"),
    ("dx_bwd_rs", "dx_bwd", "reducescatter"),
    ("decode16", "decode16", None),
    ("decode64", "decode64", None),
]


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 20, or 100 for workloads under 0.1 TFLOP per step)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mlp_down")
    ap.add_argument("--chunks", type=int, default=0, help="0 = the workload's default")
    ap.add_argument("--sched", default="auto",
                    help="auto, fold, stationary, unfused, persistent, two_stream, tile, gemm_only")
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
    ap.add_argument("--no-parity", action="store_true", help="skip the comparison with the oracle")
    ap.add_argument("--no-configs", action="store_true", help="measure the headline workload only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--modes", default="gemm_only,reduce_only,unfused,two_stream,persistent,tile,fold,auto")
    ap.add_argument("--yardstick", action="store_true",
                    help="only time the vendor GEMM (torch.matmul -> hipBLASLt) on the workload's shard GEMMs, "
                         "with the weights as given ([K][N]) and K-contiguous, for comparison")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (reference for HBM byte counters)")
    return ap.parse_args(argv)


# ---------------------------------------------------------------------------
# Algorithmic counts
# ---------------------------------------------------------------------------

def compulsory_bytes(wl) -> float:
    """Bytes the whole step must move at least: every input read once and
    every final output written once, bf16 (the shard partials, the
    "messages", are overhead and not credited)."""
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    if wl.op in ("allreduce", "reducescatter"):      # X_k [M, K], W_k [K, N], Y [M, N]
        return p * (2.0 * M * K + 2.0 * K * N) + 2.0 * M * N
    if wl.op == "allgather":                          # slices [M/p, K], W [K, N], Y [M, N]
        return 2.0 * M * K + 2.0 * K * N + 2.0 * M * N
    if wl.op == "dx":                                 # dY_k [M, N], W_k [K, N], dX [M, K]
        return p * (2.0 * M * N + 2.0 * K * N) + 2.0 * M * K
    if wl.op == "mlp_sp":                             # slices [M/p, N], W1_k [N, K], W2_k [K, N], Y [M, N]
        return 2.0 * M * N + p * 4.0 * N * K + 2.0 * M * N
    if wl.op == "rowpar_dx":                          # dY [M, N], W_k [K, N], dX_k [M, K]
        return 2.0 * M * N + p * (2.0 * K * N + 2.0 * M * K)
    if wl.op.startswith("wgrad"):                     # A_k [M, K], B_k [M, N], dW_k [K, N] fp32
        return p * (2.0 * M * K + 2.0 * M * N + 4.0 * K * N)
    raise ValueError(wl.op)


def kernel_bytes(wl, part_bytes=4, sched="unfused"):
    """HBM bytes of one launch of the timed kernel(s), every tensor that
    launch touches counted once: the shard-GEMM kernel reads the operands and
    writes the partials (`part_bytes` per element) of the reducing ops; the
    fold scheduler's pair of launches also reads back the partials of p - 1
    shards and writes the bf16 result; the single-launch (stationary) path
    touches exactly the compulsory bytes."""
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    if sched == "stationary":
        return compulsory_bytes(wl)
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


def kernel_name(sched, op="", M=0):
    """The kernel (or, for the fold scheduler, the pair of launches) that
    dominates one step of the scheduler the library ran: what `roofline`
    prices (the single-launch path picks its tile kernel by the row count M)."""
    if op.startswith("wgrad"):
        return "tile_kernel A_KM (weight-gradient GEMM tiles, transposed A)"
    if op == "rowpar_dx":
        return "tile_kernel NK (row-parallel input-gradient tiles, transposed weights, one dY for every shard)"
    if op == "mlp_sp":
        if sched == "fold":
            return ("tile_kernel pair (FC2: shards 0..p-2 into partials, then shard p-1 with the fold epilogue; "
                    "FC1 with GeLU runs before it)")
        if sched == "stationary":
            return ("stationary_large_kernel (FC2: every shard of a 128x256 output tile in one workgroup; "
                    "FC1 runs before it)" if M > 64 else
                    "stationary_kernel (FC2: every shard of an output tile in one workgroup; FC1 runs before it)")
        return "tile_kernel RED=0 (FC2 shard GEMM tiles; FC1 with GeLU runs before it)"
    if sched == "stationary" and M > 64:
        return ("stationary_large_kernel (one launch: each workgroup runs every shard's K loop for its 128x256 "
                "output tile and keeps the running sum in registers)")
    if sched == "stationary":
        return "stationary_kernel (one launch: each workgroup computes every shard's partial of its output tile and folds them on chip)"
    if sched == "persistent":
        return "fused_kernel (persistent: shard GEMM tiles + chunk reductions)"
    if sched == "fold":
        return "tile_kernel pair (shards 0..p-2 into partials, then shard p-1 with the fold epilogue)"
    if sched == "tile":
        return "tile_kernel RED=1 (shard GEMM tiles + last-arriver tile sums)"
    if sched == "two_stream":
        return "whole step (per-chunk GEMM and reduction kernels on three streams)"
    if op == "allgather":
        return "tile_kernel RED=0 (GEMM tiles over the gathered input; the gather copy runs before it)"
    return "tile_kernel RED=0 (shard GEMM tiles)"


def chunks_effective(sched: str, n: int) -> int:
    """Chunks the scheduler that ran actually pipelines: the chunked
    schedulers use the requested count; the others do not chunk (the tile
    scheduler's readiness is per output tile, reported as 0)."""
    if sched in ("persistent", "two_stream"):
        return n
    if sched == "tile":
        return 0
    return 1


# ---------------------------------------------------------------------------
# One workload: calls, timing, parity
# ---------------------------------------------------------------------------

class Runner:
    """The library calls of one workload on preallocated outputs."""

    def __init__(self, wl, sets, n, msg, handle, semantic="allreduce"):
        import torch
        from tensor_gemm_reduction_amd import tpfuse as tp
        self.wl, self.sets, self.n, self.msg, self.h = wl, sets, n, msg, handle
        self.sem = tp.ALLREDUCE if semantic == "allreduce" else tp.REDUCESCATTER
        self.tp, self.torch = tp, torch
        p, M, N, K = wl.p, wl.M, wl.N, wl.K
        dev = "cuda"
        self.ws = None
        if wl.op in ("allreduce", "reducescatter", "dx", "mlp_sp"):
            op_id = {"allreduce": tp.OP_MATMUL_ALLREDUCE, "reducescatter": tp.OP_MATMUL_REDUCESCATTER,
                     "dx": tp.OP_MATMUL_DX, "mlp_sp": tp.OP_MLP_SP}[wl.op]
            dims = (M, K, N) if wl.op == "dx" else (M, N, K)
            self.ws = torch.empty(tp.workspace_size(op_id, p, *dims, n, message=msg), dtype=torch.uint8, device=dev)
        self.outs = {dt: self._alloc(dt) for dt in (torch.bfloat16,)}
        self.ws_bytes = 0 if self.ws is None else self.ws.numel()

    def _alloc(self, dt):
        torch, wl = self.torch, self.wl
        p, M, N, K = wl.p, wl.M, wl.N, wl.K
        e = lambda *s, d=dt: torch.empty(s, dtype=d, device="cuda")  # noqa: E731
        if wl.op == "allreduce":
            return e(M, N)
        if wl.op == "reducescatter":
            return [e(M // p, N) for _ in range(p)]
        if wl.op == "dx":
            return e(M, K) if self.sem == self.tp.ALLREDUCE else [e(M // p, K) for _ in range(p)]
        if wl.op == "mlp_sp":
            return (e(M, N, d=torch.bfloat16), [e(M, K, d=torch.bfloat16) for _ in range(p)],
                    [e(M // p, N) for _ in range(p)])
        if wl.op == "rowpar_dx":
            return [e(M, K) for _ in range(p)]
        if wl.op.startswith("wgrad"):
            return [e(K, N) for _ in range(p)]
        return (e(M, K, d=torch.bfloat16), e(M, N))      # allgather: X_gathered, Y

    def call(self, i, sched, n=None, out_dtype=None):
        tp, wl = self.tp, self.wl
        n = self.n if n is None else n
        inp = self.sets[i % len(self.sets)]
        o = self.outs[out_dtype or self.torch.bfloat16]
        kw = dict(handle=self.h)
        if wl.op == "allreduce":
            tp.matmul_allreduce(inp.X, inp.W, n_chunks=n, sched=sched, Y=o, ws=self.ws, message=self.msg, **kw)
        elif wl.op == "reducescatter":
            tp.matmul_reducescatter(inp.X, inp.W, n_chunks=n, sched=sched, Y=o, ws=self.ws, message=self.msg, **kw)
        elif wl.op == "dx":
            tp.matmul_dx(inp.X, inp.W, self.sem, n_chunks=n, sched=sched, dX=o, ws=self.ws, message=self.msg, **kw)
        elif wl.op == "mlp_sp":
            tp.mlp_sp(inp.X, inp.W[:wl.p], inp.W[wl.p:], n_chunks=n, sched=sched, X_gathered=o[0], H=o[1], Y=o[2],
                      ws=self.ws, message=self.msg, **kw)
        elif wl.op == "rowpar_dx":
            tp.rowpar_dx(inp.X[0], inp.W, dX=o, **kw)
        elif wl.op.startswith("wgrad"):
            from tensor_gemm_reduction_amd import inputs
            A, B = inputs.weight_grad_operands(inp)
            tp.weight_grad(A, B, dW=o, **kw)
        else:
            tp.allgather_matmul(inp.X, inp.W[0], n_chunks=n, sched=sched, X_gathered=o[0], Y=o[1], **kw)

    def output(self, sched, out_dtype):
        """The final output of one call on input set 0, as one tensor."""
        torch = self.torch
        if out_dtype not in self.outs:
            self.outs[out_dtype] = self._alloc(out_dtype)
        self.call(0, sched, out_dtype=out_dtype)
        torch.cuda.synchronize()
        o = self.outs[out_dtype]
        wl = self.wl
        if wl.op == "allgather":
            return o[1]
        if wl.op == "mlp_sp":
            return torch.cat(o[2], 0)
        if isinstance(o, list):
            return torch.cat(o, 0) if wl.op in ("reducescatter", "dx") else torch.stack(o, 0)
        return o


def oracle_output(wl, inp):
    """The float64 oracle's full output for input set `inp` (shape as
    Runner.output returns it)."""
    import numpy as np
    from oracle import tpf_oracle as O
    from tensor_gemm_reduction_amd import inputs
    b = lambda ts: [inputs.bf16_to_bits(t) for t in ts]  # noqa: E731
    if wl.op in ("allreduce", "reducescatter"):
        return O.matmul_allreduce(b(inp.X), b(inp.W))
    if wl.op == "dx":
        return O.matmul_dx(b(inp.X), b(inp.W))
    if wl.op == "allgather":
        return O.allgather(b(inp.X)) @ O.bf16_bits_to_f64(b(inp.W)[0])
    if wl.op == "mlp_sp":
        return np.concatenate(O.mlp_sp(b(inp.X), b(inp.W[:wl.p]), b(inp.W[wl.p:])), 0)
    if wl.op == "rowpar_dx":
        return np.stack(O.rowpar_dx(b(inp.X)[0], b(inp.W)), 0)
    A, B = inputs.weight_grad_operands(inp)
    return np.stack(O.weight_grad(b(A), b(B)), 0)


def parity(runner, sched):
    """Errors of the call's bf16 and fp32 outputs against the float64 oracle
    on every output element: max|d|/rms for fp32; for bf16 the literal
    max|d|/rms and the rounding-aware max(|d| - ulp/2)/rms, plus whether the
    bf16 output is the RNE rounding of the fp32 output bit for bit."""
    import numpy as np
    import torch
    from oracle import tpf_oracle as O
    wl = runner.wl
    y16 = runner.output(sched, torch.bfloat16)
    y32 = runner.output(sched, torch.float32)
    ref = oracle_output(wl, runner.sets[0]).reshape(tuple(y16.shape))
    rms = float(np.sqrt(np.mean(np.square(ref))))
    g32 = y32.double().cpu().numpy()
    g16 = y16.float().double().cpu().numpy()
    d16 = np.abs(g16 - ref)
    _, e = np.frexp(ref)
    half_ulp = np.ldexp(1.0, np.maximum(e - 9, -134))
    rne = O.round_to_bf16_bits(g32)
    have = y16.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    out = {"elements": int(ref.size), "oracle": "float64 (numpy, every element)",
           "f32_max_abs_over_rms": float(np.abs(g32 - ref).max() / rms),
           "bf16_max_abs_over_rms_literal": float(d16.max() / rms),
           "bf16_max_over_rms_ulp_aware": float((d16 - half_ulp).max() / rms),
           "bf16_is_rne_of_f32": bool(np.array_equal(rne, have))}
    out["pass"] = bool(out["f32_max_abs_over_rms"] <= 1e-4 and out["bf16_max_over_rms_ulp_aware"] <= 1e-2
                       and out["bf16_is_rne_of_f32"])
    return out


def make_sets(wl, args_sets, dev="cuda"):
    from tensor_gemm_reduction_amd import inputs
    sets = [inputs.make_inputs(wl, seed=0, device=dev)]
    nsets = args_sets
    if nsets <= 0:
        set_bytes = sum(t.numel() * t.element_size() for t in list(sets[0].X) + list(sets[0].W))
        nsets = min(8, max(2, -(-ROTATION_BYTES // set_bytes)))
    for s in range(1, nsets):
        sets.append(inputs.make_inputs(wl, seed=s, device=dev))
    return sets


def measure(runner, sched, steps, warmup, settle_ms, mode_specs, graph=False):
    """Time `steps` calls of `sched` after a settle and `warmup` calls; the
    library's HIP events time each call's dominant launch.  Then time each
    (label, sched, n) of `mode_specs` round-robin.  Returns a dict."""
    import torch
    tp = runner.tp
    handle = runner.h
    stream = torch.cuda.current_stream()
    call = runner.call

    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < settle_ms:
        call(settle_steps, sched)
        settle_steps += 1
        if settle_steps % 8 == 0:
            torch.cuda.synchronize()      # measure GPU progress, not how fast the host can enqueue
    torch.cuda.synchronize()
    settle_ms_done = (time.perf_counter() - t_settle) * 1e3

    for i in range(warmup):
        call(i, sched)
    torch.cuda.synchronize()
    handle.set_kernel_timing(True)   # events around each step's dominant kernel launch
    # One event pair around all K steps: a timed event costs the stream a few
    # microseconds, so none is recorded between the steps beyond the pair the
    # library records around each dominant launch.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        call(i, sched)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = handle.sync_status()
    if st != tp.OK:
        raise RuntimeError(f"{runner.wl.name}: the path reported status {st}")
    launch_ms = handle.kernel_times(steps)
    handle.set_kernel_timing(False)
    ran = handle.last_sched() or sched
    res = {"sched_ran": ran, "ms_per_step": 1e3 * wall / steps, "step_event_ms": ev0.elapsed_time(ev1) / steps,
           "launch_ms": launch_ms, "settle": {"ms": round(settle_ms_done, 1), "steps": settle_steps}}

    if graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(0, sched)          # warm the side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(steps):
                call(i, sched)
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        g0.record(stream)
        for _ in range(reps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        if handle.sync_status() != tp.OK:
            raise RuntimeError("graph replay reported a timeout")
        res["graph_ms_per_step"] = g0.elapsed_time(g1) / (reps * steps)
        del g

    def time_slice(s, n, k, w):
        for i in range(w):
            call(i, s, n)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
        for i in range(k):
            evs[i][0].record(stream)
            call(i, s, n)
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    # Round-robin, four steps of every mode per round, so that clock and
    # temperature drift over the run affects all modes alike.
    per = {lab: [] for lab, _, _ in mode_specs}
    mode_steps = max(8, steps // 2)
    for r in range(max(2, (mode_steps + 3) // 4)):
        for lab, s, n in mode_specs:
            per[lab] += time_slice(s, n, 4, 1 if r else 2)
    modes = {}
    for lab, _, _ in mode_specs:
        v = sorted(per[lab])
        modes[lab] = {"ms_median": v[len(v) // 2], "ms_min": v[0]}
    if handle.sync_status() != tp.OK:
        raise RuntimeError(f"{runner.wl.name}: a mode reported a timeout")
    res["modes"] = modes
    return res


def summarize(wl, res, sched_req, n, msg_bytes, timed_label):
    """Throughput, roofline and exposed-reduction figures of one measurement."""
    flops = wl.flops()
    kflops = flops / 2 if wl.op == "mlp_sp" else flops    # the timed launch of the MLP block is FC2
    ran = res["sched_ran"]
    comp = compulsory_bytes(wl)
    lbytes = kernel_bytes(wl, msg_bytes, ran)
    launch_ms = res["launch_ms"]
    kern = launch_ms if launch_ms else [res["step_event_ms"]]     # two_stream records no single launch
    avg_kernel_ms = sum(kern) / len(kern)
    hbm_bound = flops / comp < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        # the dominant kernel's share of the compulsory bytes: for the
        # single-launch path all of them; otherwise the launch's own bytes
        kb = comp if ran == "stationary" else lbytes
        achieved, peak, unit = kb / (avg_kernel_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = kflops / (avg_kernel_ms * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    step_ms = res["ms_per_step"]
    rec = {
        "ms_per_step": round(step_ms, 4),
        "tflops": round(flops / (step_ms * 1e-3) / 1e12, 3),
        "step_gbs_compulsory": round(comp / (step_ms * 1e-3) / 1e9, 1),
        "sched_ran": ran, "n_chunks": n, "n_chunks_effective": chunks_effective(ran, n),
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": unit, "frac": round(achieved / peak, 4),
                     "algorithmic_bytes": comp, "launch_bytes": lbytes, "algorithmic_flops": kflops,
                     "kernel": kernel_name(ran, wl.op, wl.M), "avg_kernel_ms": round(avg_kernel_ms, 4),
                     "timed_launches": len(launch_ms) if launch_ms else 0,
                     "avg_step_event_ms": round(res["step_event_ms"], 4)},
    }
    if hbm_bound:
        rec["step_frac_hbm_compulsory"] = round(comp / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    modes = res["modes"]
    if "gemm_only" in modes and timed_label in modes:
        t_f = modes[timed_label]["ms_median"]
        t_g = modes["gemm_only"]["ms_median"]
        exposed = t_f - t_g
        rec["exposed_reduce_ms"] = round(exposed, 4)
        rec["exposed_over_fused"] = round(exposed / t_f, 4)
        if "reduce_only" in modes:
            rec["exposed_over_reduce_only"] = round(exposed / modes["reduce_only"]["ms_median"], 4)
        if "unfused" in modes:
            rec["fused_over_unfused"] = round(t_f / modes["unfused"]["ms_median"], 4)
        # the pages' two-engine model with measured whole-op times split per chunk
        t_c = t_g / n
        t_m = modes.get("reduce_only", {"ms_median": 0.0})["ms_median"] / n
        rec["model_pipeline_ms"] = round(t_c + (n - 1) * max(t_c, t_m) + t_m, 4)
        rec["model_serial_ms"] = round(n * (t_c + t_m), 4)
    chunked = {k: v["ms_median"] for k, v in modes.items() if k.startswith(("two_stream", "persistent"))}
    if chunked and "unfused" in modes:
        best = min(chunked, key=chunked.get)
        rec["chunked_best"] = {"mode": best, "ms": round(chunked[best], 4),
                               "over_unfused": round(chunked[best] / modes["unfused"]["ms_median"], 4)}
    goal = TARGET_HBM_FRAC if hbm_bound else TARGET_MFMA_FRAC
    rec["targets"] = {"roofline_frac_goal": goal, "roofline_frac_met": rec["roofline"]["frac"] >= goal,
                      "exposed_goal": TARGET_EXPOSED,
                      "exposed_met": rec.get("exposed_over_fused", 0.0) < TARGET_EXPOSED}
    rec["modes"] = {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in modes.items()}
    return rec


def chunk_sweep(wl, n):
    """The chunked two-stream scheduler at 2, 4 and 8 chunks beside the
    default count, for the large-M reducing workloads: where chunking pays."""
    if wl.M <= 64 or wl.op not in ("allreduce", "reducescatter", "dx"):
        return []
    return [(f"two_stream_n{m}", "two_stream", m) for m in (2, 4, 8) if m != n and m <= wl.M]


def default_modes(wl, n, requested, sched):
    """(label, scheduler, chunks) triples timed beside the headline."""
    specs = [(m, m, n) for m in requested if m]
    if sched not in [m for m, _, _ in specs]:
        specs.append((sched, sched, n))
    if "two_stream" in requested:
        specs += chunk_sweep(wl, n)
    return specs


def config_modes(wl, n):
    """Modes timed for a `configs` record: the timed scheduler (auto), its
    phases and the unfused baseline; decode shapes add the chunked
    schedulers at 1, 2 and 4 chunks, where chunking stops paying."""
    specs = [("auto", "auto", n), ("gemm_only", "gemm_only", n), ("reduce_only", "reduce_only", n),
             ("unfused", "unfused", n)]
    if wl.op != "allgather":
        specs.append(("fold", "fold", n))
        specs.append(("stationary", "stationary", n))
    if wl.M <= 64:
        for m in (1, 2, 4):
            specs.append((f"persistent_n{m}", "persistent", m))
            specs.append((f"two_stream_n{m}", "two_stream", m))
    else:
        specs.append(("persistent", "persistent", n))
        specs.append(("two_stream", "two_stream", n))
        specs += chunk_sweep(wl, n)
    return specs


def main(argv=None):
    args = parse(argv)
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
        nb = args.copy_calibration * (1 << 20)
        src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nb, "note": "plain device copy for counter calibration"}), flush=True)
        return

    wl = inputs.WORKLOADS[args.workload]
    if args.steps is None:       # short steps need more repetitions for a steady figure
        args.steps = 100 if wl.flops() < 1e11 else 20
    if args.yardstick:
        yardstick(args, wl)
        return

    tp.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    handle = tp.Handle(0)
    n = args.chunks or wl.default_chunks
    msg_bytes = 2 if args.message == "bf16" else 4

    sets = make_sets(wl, args.sets)
    runner = Runner(wl, sets, n, args.message, handle)
    specs = default_modes(wl, n, [m for m in args.modes.split(",") if m and m != "none"], args.sched)
    if wl.op in ("rowpar_dx",) or wl.op.startswith("wgrad"):
        specs = []       # no reduction: there are no schedules to compare
    res = measure(runner, args.sched, args.steps, args.warmup, args.settle_ms, specs, graph=args.graph)
    head = summarize(wl, res, args.sched, n, msg_bytes, args.sched)
    par = None if args.no_parity else parity(runner, args.sched)

    # HBM bytes per launch from the committed counter summary (only while
    # the kernel sources are the ones the counters were taken on)
    from tensor_gemm_reduction_amd import profiling
    rec = profiling.load_traffic(wl.name, os.path.join(ROOT, "profiles"))
    traffic = round(rec["hbm_bytes"]) if rec and rec.get("sched") == head["sched_ran"] else None
    head["roofline"]["traffic"] = traffic

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, sets[0], args.cpu_seconds, runner)
    nsets, ws_bytes = len(sets), runner.ws_bytes
    del runner, sets
    torch.cuda.empty_cache()

    configs = {}
    if not args.no_configs and args.workload == "mlp_down":
        for name, wname, sem in CONFIGS:
            cwl = inputs.WORKLOADS[wname]
            cn = cwl.default_chunks
            csets = make_sets(cwl, 0)
            cr = Runner(cwl, csets, cn, args.message, handle, semantic=sem or "allreduce")
            csteps = 100 if cwl.flops() < 1e11 else 20
            cres = measure(cr, "auto", csteps, 3, 150.0, config_modes(cwl, cn))
            crec = summarize(cwl, cres, "auto", cn, msg_bytes, "auto")
            crec.update({"workload": cwl.name, "op": cwl.op, "p": cwl.p, "M": cwl.M, "N": cwl.N, "K_shard": cwl.K,
                         "semantic": sem, "input_sets": len(csets), "note": cwl.note})
            if not args.no_parity:
                crec["parity"] = parity(cr, "auto")
            configs[name] = crec
            del cr, csets
            torch.cuda.empty_cache()
            print(f"# config {name}: {crec['ms_per_step']} ms/step, {crec['tflops']} TFLOP/s, "
                  f"frac {crec['roofline']['frac']}", file=sys.stderr, flush=True)

    out = {
        "metric": "TFLOP/s & % bf16 MFMA peak, fused MatMul+reduce; exposed reduce ms vs unfused",
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "settle": res["settle"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "op": wl.op, "p": wl.p, "M": wl.M, "N": wl.N, "K_shard": wl.K,
                   "n_chunks": n, "n_chunks_effective": head["n_chunks_effective"], "sched": args.sched,
                   "sched_ran": head["sched_ran"], "out": "bf16", "message": args.message,
                   "input_sets": nsets, "workspace_bytes": ws_bytes, "note": wl.note},
        "roofline": head["roofline"],
        "targets": head["targets"],
        "parity": par,
        "cpu_baseline": cpu,
        "graph": ({"ms_per_step": round(res["graph_ms_per_step"], 4),
                   "value": round(wl.flops() / (res["graph_ms_per_step"] * 1e-3) / 1e12, 3)}
                  if "graph_ms_per_step" in res else None),
        "modes": head["modes"],
        **{k: head[k] for k in ("exposed_reduce_ms", "exposed_over_fused", "exposed_over_reduce_only",
                                "fused_over_unfused", "model_pipeline_ms", "model_serial_ms", "chunked_best")
           if k in head},
        "configs": configs,
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


def cpu_baseline(wl, inp, seconds, runner=None):
    """Time the plain C oracle (float64, OpenMP over output rows) on a bounded
    sample of the workload's output rows, on the same inputs; where the timed
    GPU output of those rows is at hand, also report its largest deviation
    from them."""
    import numpy as np
    from oracle import c_oracle
    from tensor_gemm_reduction_amd import inputs

    C = c_oracle.default()
    threads = C.threads()
    Xb = [inputs.bf16_to_bits(x) for x in inp.X]
    Wb = [inputs.bf16_to_bits(w) for w in inp.W]
    kind = "oracle"
    if wl.op in ("allreduce", "reducescatter"):
        M, fn = wl.M, lambda r: C.matmul_allreduce(Xb, Wb, rows=r)
    elif wl.op == "dx":
        M, fn = wl.M, lambda r: C.matmul_dx(Xb, Wb, rows=r)
    elif wl.op == "allgather":
        M, fn = wl.M, lambda r: C.allgather_matmul(Xb, Wb[0], rows=r)[1]
    elif wl.op == "rowpar_dx":          # dX_k = dY W_k^T: the dX loops with one shard each
        M, fn = wl.M, lambda r: np.stack([C.matmul_dx([Xb[0]], [w], rows=r) for w in Wb], 0)
    else:
        return None                     # the MLP block and weight gradients: no C loops for them

    def run(rows):
        r = np.arange(rows)
        t0 = time.perf_counter()
        y = fn(r)
        return time.perf_counter() - t0, y

    rows = min(M, 8)
    dt, y = run(rows)
    while dt < seconds / 4 and rows < M:
        rows = min(M, rows * 4)
        dt, y = run(rows)
    reps, total = 1, dt
    while total < seconds and rows == M:     # the whole workload is quick: repeat it for a steady figure
        d, _ = run(rows)
        total += d
        reps += 1
    per_row_flops = wl.flops() / M
    out = {"value": round(per_row_flops * rows * reps / total / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
           "kind": kind,
           "sample": f"{rows} of {M} output rows of the same inputs (plain C oracle, float64, OpenMP over rows, "
                     f"{threads} threads), {reps} run(s), {total:.2f} s on {cpu_model()}"}
    if runner is not None and wl.op in ("allreduce", "reducescatter", "dx", "allgather"):
        import torch
        g = runner.output("auto", torch.float32)[:rows].double().cpu().numpy()
        ref = y if y.ndim == 2 else y
        out["gpu_f32_max_abs_over_rms_on_sample"] = float(np.abs(g - ref).max() / np.sqrt(np.mean(ref ** 2)))
    return out


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
