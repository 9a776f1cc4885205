"""Full-size parity for every configured workload, in the launch configuration
the benchmark times (AUTO scheduler, the workload's default chunk count).

Every output row is compared with the float64 oracle (the oracle's matmul
is a library dgemm, so the whole of every configuration takes seconds on
the host).  Properties that hold at any size are checked as well: identical
bits for every scheduler and chunk count, ReduceScatter slices equal to
AllReduce rows, bf16 output equal to the RNE rounding of the fp32 output."""
import numpy as np
import pytest
import torch

from oracle import tpf_oracle as O
from tensor_gemm_reduction_amd import inputs, tpfuse as tp
from tests.parity import assert_bf16, assert_bf16_is_rne_of_f32, assert_bitwise, assert_f32

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def bits(ts):
    return [inputs.bf16_to_bits(t) for t in ts]


# Ops of the reducing / gathering calls this file runs at full size.  Every
# other op has a test of its own below; run() and oracle_rows() refuse them.
FULLSIZE_OPS = ("allreduce", "reducescatter", "dx", "allgather")


def run(wl, inp, out_dtype, n, sched):
    if wl.op == "allreduce":
        return tp.matmul_allreduce(inp.X, inp.W, out_dtype, n_chunks=n, sched=sched)
    if wl.op == "reducescatter":
        return torch.cat(tp.matmul_reducescatter(inp.X, inp.W, out_dtype, n_chunks=n, sched=sched), 0)
    if wl.op == "dx":
        return tp.matmul_dx(inp.X, inp.W, tp.ALLREDUCE, out_dtype, n_chunks=n, sched=sched)
    if wl.op == "allgather":
        return tp.allgather_matmul(inp.X, inp.W[0], out_dtype, n_chunks=n, sched=sched)[1]
    raise ValueError(f"run(): no full-size dispatch for op {wl.op!r} (workload {wl.name})")


def oracle_rows(wl, inp, rows=None):
    """The float64 oracle's output rows (all rows when `rows` is None)."""
    if wl.op in ("allreduce", "reducescatter"):
        return O.matmul_allreduce(bits(inp.X), bits(inp.W), rows=rows)
    if wl.op == "dx":
        return O.matmul_dx(bits(inp.X), bits(inp.W), rows=rows)
    if wl.op == "allgather":
        xg = O.allgather(bits(inp.X))
        if rows is not None:
            xg = xg[rows]
        return xg @ O.bf16_bits_to_f64(bits(inp.W)[0])
    raise ValueError(f"oracle_rows(): no oracle for op {wl.op!r} (workload {wl.name})")


REDUCING = [n for n, w in inputs.WORKLOADS.items() if w.op in FULLSIZE_OPS]
WGRAD = [n for n, w in inputs.WORKLOADS.items() if w.op.startswith("wgrad")]


@pytest.mark.parametrize("name", REDUCING)
def test_fullsize_parity(name):
    wl = inputs.WORKLOADS[name]
    n = wl.default_chunks
    say(f"full-size {name}: op={wl.op} p={wl.p} M={wl.M} N={wl.N} K={wl.K} n={n}")
    inp = inputs.make_inputs(wl, seed=0, device="cuda")
    y16 = run(wl, inp, torch.bfloat16, n, "auto")
    y32 = run(wl, inp, torch.float32, n, "auto")
    torch.cuda.synchronize()
    ref = oracle_rows(wl, inp)                      # every row
    assert ref.shape == tuple(y16.shape)
    what = f"{name} n={n} all {wl.M} rows"
    assert_f32(y32, ref, what)
    assert_bf16(y16, ref, what)
    assert_bf16_is_rne_of_f32(y16, y32, what)
    del ref
    # every other chunk count and scheduler gives the same bits
    for m in wl.chunks:
        for sched in ("persistent", "two_stream", "unfused", "tile", "fold", "stationary"):
            if m == n and sched == "persistent" and n == 1:
                continue
            y = run(wl, inp, torch.bfloat16, m, sched)
            torch.cuda.synchronize()
            assert_bitwise(y, y16, f"{name}: {sched} n={m} vs auto n={n}")


@pytest.mark.parametrize("name", WGRAD)
def test_fullsize_weight_grad(name):
    """Weight gradients at full size: every row of every dW_k against the
    oracle (one shard at a time), bf16 output equal to the RNE rounding of the
    fp32 output."""
    wl = inputs.WORKLOADS[name]
    say(f"full-size {name}: p={wl.p} M={wl.M} R={wl.K} C={wl.N}")
    inp = inputs.make_inputs(wl, seed=0, device="cuda")
    A, B = inputs.weight_grad_operands(inp)
    d32 = tp.weight_grad(A, B, torch.float32)
    d16 = tp.weight_grad(A, B, torch.bfloat16)
    torch.cuda.synchronize()
    for k in range(wl.p):
        ref = O.weight_grad([inputs.bf16_to_bits(A[k])], [inputs.bf16_to_bits(B[k])])[0]     # [R, C]
        what = f"{name} dW_{k} all {ref.shape[0]} rows"
        assert_f32(d32[k], ref, what)
        assert_bf16(d16[k], ref, what)
        assert_bf16_is_rne_of_f32(d16[k], d32[k], what)
        del ref


def test_fullsize_rowpar_dx():
    """Row-parallel input gradients at the dx_row size (dY [4096,4096] shared
    by p = 4 shards, W_k [4096,4096]): every row of every dX_k against the
    oracle, bf16 output equal to the RNE rounding of the fp32 output."""
    wl = inputs.WORKLOADS["dx_row"]
    say(f"full-size dx_row: p={wl.p} M={wl.M} K_shard={wl.K} N={wl.N}")
    inp = inputs.make_inputs(wl, seed=0, device="cuda")
    dY = inp.X[0]
    d32 = tp.rowpar_dx(dY, inp.W, torch.float32)
    d16 = tp.rowpar_dx(dY, inp.W, torch.bfloat16)
    torch.cuda.synchronize()
    dYb = inputs.bf16_to_bits(dY)
    for k in range(wl.p):
        ref = O.rowpar_dx(dYb, [inputs.bf16_to_bits(inp.W[k])])[0]
        what = f"dx_row dX_{k} all {wl.M} rows"
        assert_f32(d32[k], ref, what)
        assert_bf16(d16[k], ref, what)
        assert_bf16_is_rne_of_f32(d16[k], d32[k], what)
        del ref


def test_fullsize_mlp_sp():
    """The MLP block at full size: the gathered input exactly, every
    activation against the float64 GeLU of the exact FC1 product, every output
    row against FC2 evaluated on the GPU's own activations, and identical bits
    for every FC2 scheduler."""
    wl = inputs.WORKLOADS["mlp_sp"]
    p, S, Hd, F = wl.p, wl.M, wl.N, wl.K
    say(f"full-size mlp_sp: p={p} S={S} Hd={Hd} F={F}")
    inp = inputs.make_inputs(wl, seed=0, device="cuda")
    W1, W2 = inp.W[:p], inp.W[p:]
    xg, H, Y = tp.mlp_sp(inp.X, W1, W2, torch.bfloat16, n_chunks=wl.default_chunks)
    _, _, Y32 = tp.mlp_sp(inp.X, W1, W2, torch.float32, n_chunks=wl.default_chunks)
    torch.cuda.synchronize()
    assert torch.equal(xg, torch.cat(inp.X, 0))
    x = O.bf16_bits_to_f64(inputs.bf16_to_bits(xg))
    Hb = []
    for k in range(p):
        g = O.gelu(x @ O.bf16_bits_to_f64(inputs.bf16_to_bits(W1[k])))
        hb = inputs.bf16_to_bits(H[k])
        h = O.bf16_bits_to_f64(hb)
        # half a bf16 ulp of the rounding plus an fp32-accumulation slack
        tol = 0.5 * np.ldexp(1.0, np.frexp(np.abs(g))[1] - 8) * (1 + 2.0 ** -7) + 1e-5 * np.sqrt(np.mean(g * g))
        assert (np.abs(h - g) <= tol).all(), f"activation {k}"
        Hb.append(hb)
        del g, h
    del x
    ref = O.matmul_allreduce(Hb, [inputs.bf16_to_bits(w) for w in W2])    # sum_k H_k W2_k, every row
    assert_f32(torch.cat(Y32, 0), ref, f"mlp_sp all {S} rows")
    assert_bf16(torch.cat(Y, 0), ref, f"mlp_sp all {S} rows")
    assert_bf16_is_rne_of_f32(torch.cat(Y, 0), torch.cat(Y32, 0), "mlp_sp")
    del ref
    for sched in ("persistent", "two_stream", "tile", "fold", "stationary"):
        _, _, Ys = tp.mlp_sp(inp.X, W1, W2, torch.bfloat16, n_chunks=wl.default_chunks, sched=sched)
        torch.cuda.synchronize()
        assert_bitwise(torch.cat(Ys, 0), torch.cat(Y, 0), f"mlp_sp {sched}")


def test_fullsize_reducescatter_equals_allreduce_rows():
    wl = inputs.WORKLOADS["sp_rs"]
    say("sp_rs: ReduceScatter slices vs AllReduce rows at full size")
    inp = inputs.make_inputs(wl, seed=1, device="cuda")
    sl = tp.matmul_reducescatter(inp.X, inp.W, torch.bfloat16, n_chunks=wl.default_chunks)
    ar = tp.matmul_allreduce(inp.X, inp.W, torch.bfloat16, n_chunks=wl.default_chunks)
    torch.cuda.synchronize()
    s = wl.M // wl.p
    for r in range(wl.p):
        assert_bitwise(sl[r], ar[r * s:(r + 1) * s], f"slice {r}")


def test_fullsize_dx_reducescatter():
    wl = inputs.WORKLOADS["dx_bwd"]
    say("dx_bwd: ReduceScatter layout vs AllReduce rows at full size")
    inp = inputs.make_inputs(wl, seed=2, device="cuda")
    full = tp.matmul_dx(inp.X, inp.W, tp.ALLREDUCE, torch.bfloat16, n_chunks=wl.default_chunks)
    sl = tp.matmul_dx(inp.X, inp.W, tp.REDUCESCATTER, torch.bfloat16, n_chunks=wl.default_chunks)
    torch.cuda.synchronize()
    s = wl.M // wl.p
    for r in range(wl.p):
        assert_bitwise(sl[r], full[r * s:(r + 1) * s], f"dX slice {r}")


def test_fullsize_allgather_copy_exact():
    wl = inputs.WORKLOADS["ag_fwd"]
    say("ag_fwd: gathered input equals the slices in rank order")
    inp = inputs.make_inputs(wl, seed=3, device="cuda")
    xg, _ = tp.allgather_matmul(inp.X, inp.W[0], torch.bfloat16, n_chunks=wl.default_chunks)
    torch.cuda.synchronize()
    assert torch.equal(xg, torch.cat(inp.X, 0))


def test_tile_timeline_reduces_each_tile_once_and_overlaps():
    """Tile scheduler: every output tile is summed exactly once, by the
    workgroup that finished its last shard, and those sums run while GEMM
    tiles of other output tiles are still being computed."""
    wl = inputs.WORKLOADS["mlp_down"]
    say("mlp_down: tile-scheduler timeline")
    inp = inputs.make_inputs(wl, seed=0, device="cuda")
    h = tp.Handle(0)
    tiles = (wl.M // 256) * (wl.N // 256)
    ev = torch.zeros(32 * wl.p * tiles, dtype=torch.uint8, device="cuda")
    h.set_timeline(ev)
    y = tp.matmul_allreduce(inp.X, inp.W, n_chunks=wl.default_chunks, sched="tile", handle=h)
    torch.cuda.synchronize()
    h.set_timeline(None)
    assert h.sync_status() == tp.OK
    e = tp.timeline_events(ev, wl.p * tiles)
    assert (e["t_end"] > 0).all()
    red = e[e["mid"] > 0]
    assert sorted(red["chunk"].tolist()) == list(range(tiles))    # each output tile summed once
    r0 = red["t_start"] + red["mid"]
    r1 = red["t_end"]
    g_end = np.where(e["mid"] > 0, e["t_start"] + e["mid"], e["t_end"])
    hit = (r0[:, None] < g_end[None, :]) & (e["t_start"][None, :] < r1[:, None])
    overlapped = hit.any(axis=1).mean()
    assert overlapped > 0.5, f"only {overlapped:.2f} of the tile sums overlap a GEMM tile"
    ref = tp.matmul_allreduce(inp.X, inp.W, n_chunks=1, sched="unfused")
    torch.cuda.synchronize()
    assert_bitwise(y, ref, "tile vs unfused")
    h.close()


def test_timeline_shows_chunk_overlap():
    """The persistent kernel overlaps each chunk's reduction with GEMM work of
    later chunks: for every chunk but the last, some interval in which a
    slice of its reduction runs intersects an interval in which a GEMM tile
    of a later chunk runs.  (With two chunks in flight on the GPU at a time,
    chunk c's reduction typically overlaps chunk c+2's GEMM.)"""
    wl = inputs.WORKLOADS["mlp_down"]
    say("mlp_down: persistent-kernel timeline")
    inp = inputs.make_inputs(wl, seed=0, device="cuda")
    h = tp.Handle(0)
    ev = torch.zeros(32 * 8192, dtype=torch.uint8, device="cuda")
    h.set_timeline(ev)
    tp.matmul_allreduce(inp.X, inp.W, n_chunks=wl.default_chunks, sched="persistent", handle=h)
    torch.cuda.synchronize()
    h.set_timeline(None)
    assert h.sync_status() == tp.OK
    e = tp.timeline_events(ev, 8192)
    e = e[e["t_end"] > 0]
    n = wl.default_chunks
    gemm = e[e["kind"] == 0]
    assert len(gemm) == wl.p * (wl.M // 256) * (wl.N // 256)
    # GEMM part of each tile: [t_start, t_start + mid] (whole task when mid == 0)
    g_end = np.where(gemm["mid"] > 0, gemm["t_start"] + gemm["mid"], gemm["t_end"])
    overlapped = 0
    for c in range(n - 1):
        carriers = gemm[gemm["chunk"] == c + 1]     # tiles that reduce a slice of chunk c
        assert (carriers["mid"] > 0).all()
        r0 = carriers["t_start"] + carriers["mid"]
        r1 = carriers["t_end"]
        later = gemm["chunk"] > c
        gs, ge = gemm["t_start"][later], g_end[later]
        # any reduce interval [r0, r1] intersecting any later GEMM interval [gs, ge]
        hit = (r0[:, None] < ge[None, :]) & (gs[None, :] < r1[:, None])
        if hit.any():
            overlapped += 1
    assert overlapped == n - 1, f"{overlapped} of {n - 1} chunks overlapped"
    h.close()


@pytest.mark.parametrize("name", REDUCING)
def test_fullsize_against_plain_c_oracle(name):
    """The plain C oracle (float64 loops, OpenMP over rows) on sampled rows of
    every configuration at full size, against the timed launch configuration
    (AUTO, default chunks): first and last rows, both sides of every chunk
    boundary and seeded random rows, fp32 and bf16 outputs."""
    from oracle import c_oracle
    C = c_oracle.default()
    wl = inputs.WORKLOADS[name]
    n = wl.default_chunks
    say(f"C oracle {name}: op={wl.op} p={wl.p} M={wl.M} N={wl.N} K={wl.K} n={n}")
    inp = inputs.make_inputs(wl, seed=5, device="cuda")
    y32 = run(wl, inp, torch.float32, n, "auto")
    y16 = run(wl, inp, torch.bfloat16, n, "auto")
    torch.cuda.synchronize()
    rows = {0, 1, wl.M - 2, wl.M - 1}
    for r0, r1 in O.chunk_bounds(wl.M, n):
        rows.update({r0, max(0, r1 - 1)})
    rows.update(int(r) for r in np.random.default_rng(17).integers(0, wl.M, 16))
    rows = np.array(sorted(r for r in rows if 0 <= r < wl.M))
    X, W = bits(inp.X), bits(inp.W)
    if wl.op in ("allreduce", "reducescatter"):
        ref = C.matmul_allreduce(X, W, rows=rows)
    elif wl.op == "dx":
        ref = C.matmul_dx(X, W, rows=rows)
    else:
        ref = C.allgather_matmul(X, W[0], rows=rows)[1]
    idx = torch.as_tensor(rows, device="cuda")
    what = f"{name} vs C oracle, {len(rows)} rows"
    assert_f32(y32.index_select(0, idx), ref, what)
    assert_bf16(y16.index_select(0, idx), ref, what)
