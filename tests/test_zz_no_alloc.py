"""The no-allocation MatMul->AllReduce (tpf_matmul_allreduce_noalloc), called
through the C ABI, against the existing entry point (tpf_matmul_allreduce
with a caller workspace): identical bits on consecutive calls, each later
call smaller than the one before, so each runs over a static workspace that
the previous call left filled; a request beyond the static workspace is
refused with nothing enqueued; the calls change no device allocation; and a
captured call replays correctly."""
import pytest
import torch

from tensor_gemm_reduction_amd import inputs, tpfuse as tp
from tests.parity import assert_bitwise

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def noalloc(h, X, W, Y, n, sched, stream=None):
    """One call of the entry point through the C ABI (ctypes)."""
    lib = tp.load()
    p = len(X)
    M, K = X[0].shape
    N = W[0].shape[1]
    s = (stream or torch.cuda.current_stream()).cuda_stream
    return lib.tpf_matmul_allreduce_noalloc(h.ptr, p, M, N, K, tp.ptr_array([x.data_ptr() for x in X]),
                                            tp.ptr_array([w.data_ptr() for w in W]), Y.data_ptr(),
                                            tp._dtype_code(Y.dtype), n, tp._sched(sched), s)


def test_noalloc_matches_allreduce_on_consecutive_calls():
    h = tp.Handle(0)
    # (workload, out dtype, chunks, scheduler): partials of 16.8 MB, then 2 MB, then 2 MB again
    cases = [("decode64", torch.bfloat16, 1, "auto"), ("worked", torch.float32, 4, "fold"),
             ("worked", torch.bfloat16, 4, "persistent"), ("decode16", torch.bfloat16, 2, "unfused")]
    for name, dt, n, sched in cases:
        wl = inputs.WORKLOADS[name]
        say(f"noalloc {name}: p={wl.p} M={wl.M} N={wl.N} K={wl.K} {dt} n={n} {sched}")
        inp = inputs.make_inputs(wl, seed=3, device="cuda")
        ref = tp.matmul_allreduce(inp.X, inp.W, dt, n_chunks=n, sched=sched, handle=h)
        Y = torch.full((wl.M, wl.N), float("nan"), dtype=dt, device="cuda")
        assert noalloc(h, inp.X, inp.W, Y, n, sched) == tp.OK, tp.load().tpf_last_error()
        torch.cuda.synchronize()
        assert h.sync_status() == tp.OK
        assert_bitwise(Y, ref, f"noalloc vs allreduce, {name} {sched}")
    h.close()


def test_noalloc_refuses_beyond_its_workspace_and_allocates_nothing():
    h = tp.Handle(0)
    wl = inputs.WORKLOADS["decode64"]
    inp = inputs.make_inputs(wl, seed=4, device="cuda")
    Y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    assert noalloc(h, inp.X, inp.W, Y, 1, "unfused") == tp.OK           # first use on this device
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(20):
        assert noalloc(h, inp.X, inp.W, Y, 1, "unfused") == tp.OK
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "device memory changed across no-allocation calls"
    # p = 4 shards of [1024, 4096] x [4096, 4096]: 64 MiB of fp32 partials fit exactly, one more row does not
    p, K, N = 4, 256, 4096
    X = [torch.zeros((1025, K), dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    W = [torch.zeros((K, N), dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    Ybig = torch.full((1025, N), 7.0, dtype=torch.bfloat16, device="cuda")
    assert noalloc(h, X, W, Ybig, 1, "unfused") == tp.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((Ybig == 7.0).all()), "a refused call wrote its output"
    Yfit = torch.full((1024, N), 7.0, dtype=torch.bfloat16, device="cuda")
    assert noalloc(h, [x[:1024] for x in X], W, Yfit, 1, "unfused") == tp.OK
    torch.cuda.synchronize()
    assert bool((Yfit == 0).all())
    h.close()


def test_noalloc_single_launch_needs_no_workspace_at_any_size():
    # the output-stationary scheduler keeps the partials on chip, so a call
    # whose partials (p = 4, [1536, 512] x [512, 4096]: 96 MiB) exceed the
    # static workspace still runs, bit-identical to the existing entry point
    h = tp.Handle(0)
    p, M, K, N = 4, 1536, 512, 4096
    g = torch.Generator().manual_seed(5)
    X = [(torch.randn((M, K), generator=g)).to(torch.bfloat16).cuda() for _ in range(p)]
    W = [(0.05 * torch.randn((K, N), generator=g)).to(torch.bfloat16).cuda() for _ in range(p)]
    say(f"noalloc stationary p={p} M={M} N={N} K={K}")
    ref = tp.matmul_allreduce(X, W, torch.bfloat16, sched="unfused", handle=h)
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    assert noalloc(h, X, W, Y, 1, "stationary") == tp.OK, tp.load().tpf_last_error()
    torch.cuda.synchronize()
    assert_bitwise(Y, ref, "noalloc stationary vs allreduce")
    # the same call with a scheduler that needs the partials in memory is refused
    Y2 = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    assert noalloc(h, X, W, Y2, 1, "unfused") == tp.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((Y2 == 7.0).all())
    h.close()


@pytest.mark.parametrize("sched", ["unfused", "persistent"])
def test_noalloc_call_replays_from_a_graph(sched):
    """Captured in a HIP graph (the calls enqueue only kernels), several
    replays with eager work and synchronisation between them each give the
    eager bits."""
    h = tp.Handle(0)
    wl = inputs.WORKLOADS["decode16"]
    inp = inputs.make_inputs(wl, seed=5, device="cuda")
    ref = tp.matmul_allreduce(inp.X, inp.W, torch.bfloat16, n_chunks=2, sched=sched, handle=h).clone()
    Y = torch.empty((wl.M, wl.N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert noalloc(h, inp.X, inp.W, Y, 2, sched, stream=side) == tp.OK
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert noalloc(h, inp.X, inp.W, Y, 2, sched) == tp.OK
    for _ in range(3):
        Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(Y, ref, f"replay {sched}")
    assert h.sync_status() == tp.OK
    del g
    h.close()
