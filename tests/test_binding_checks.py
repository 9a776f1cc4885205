"""The Python binding refuses tensors the library cannot be handed (host
tensors, a wrong shard count, a shard of another shape, dtype or layout)
with ValueError before any library call: the library derives every extent
from the shape arguments, so such a tensor would be accessed out of bounds
on the GPU.  The host-tensor and shard-count cases need no GPU; the rest
build GPU tensors but launch nothing."""
import pytest
import torch

from tensor_gemm_reduction_amd import tpfuse as tp

BF = torch.bfloat16


def host(*shape, dtype=BF):
    return torch.zeros(shape, dtype=dtype)


OPS_ON_HOST = {
    "allreduce": lambda: tp.matmul_allreduce([host(64, 32)] * 2, [host(32, 16)] * 2),
    "reducescatter": lambda: tp.matmul_reducescatter([host(64, 32)] * 2, [host(32, 16)] * 2),
    "allgather": lambda: tp.allgather_matmul([host(32, 32)] * 2, host(32, 16)),
    "dx": lambda: tp.matmul_dx([host(64, 16)] * 2, [host(32, 16)] * 2),
    "weight_grad": lambda: tp.weight_grad([host(64, 32)] * 2, [host(64, 16)] * 2),
    "mlp_sp": lambda: tp.mlp_sp([host(32, 16)] * 2, [host(16, 24)] * 2, [host(24, 16)] * 2),
    "rowpar_dx": lambda: tp.rowpar_dx(host(64, 16), [host(32, 16)] * 2),
}


@pytest.mark.parametrize("op", sorted(OPS_ON_HOST))
def test_host_tensors_are_refused(op):
    with pytest.raises(ValueError, match="not on a GPU"):
        OPS_ON_HOST[op]()


@pytest.mark.parametrize("call", [
    lambda: tp.matmul_allreduce([host(64, 32)] * 2, [host(32, 16)] * 3),
    lambda: tp.matmul_reducescatter([host(64, 32)] * 2, [host(32, 16)]),
    lambda: tp.matmul_dx([host(64, 16)] * 3, [host(32, 16)] * 2),
    lambda: tp.weight_grad([host(64, 32)] * 2, [host(64, 16)] * 4),
    lambda: tp.mlp_sp([host(32, 16)] * 2, [host(16, 24)] * 2, [host(24, 16)]),
])
def test_shard_count_mismatch_is_refused(call):
    with pytest.raises(ValueError, match="one per shard"):
        call()


@pytest.mark.gpu
def test_device_tensor_checks():
    d = "cuda"

    def dev(*shape, dtype=BF):
        return torch.zeros(shape, dtype=dtype, device=d)

    X, W = [dev(64, 32)] * 2, [dev(32, 16)] * 2
    cases = [
        (lambda: tp.matmul_allreduce([dev(64, 32), dev(48, 32)], W), "X\\[1\\] has shape"),
        (lambda: tp.matmul_allreduce([dev(64, 32, dtype=torch.float32)] * 2, W), "dtype"),
        (lambda: tp.matmul_allreduce(X, [dev(16, 32).t()] * 2), "not contiguous"),
        (lambda: tp.matmul_allreduce(X, W, Y=dev(64, 16, dtype=torch.float16)), "Y has dtype"),
        (lambda: tp.matmul_allreduce(X, W, Y=dev(64, 8)), "Y has shape"),
        (lambda: tp.matmul_allreduce(X, W, ws=torch.zeros(1 << 20, dtype=torch.uint8)), "ws is on cpu"),
        (lambda: tp.matmul_allreduce(X, [host(32, 16)] * 2), "W\\[0\\] is on cpu"),
        (lambda: tp.matmul_reducescatter(X, W, Y=[dev(32, 16), dev(32, 16, dtype=torch.float32)]),
         "differ in dtype"),
        (lambda: tp.allgather_matmul([dev(32, 32)] * 2, W[0], X_gathered=dev(32, 32)), "X_gathered has shape"),
        (lambda: tp.matmul_dx([dev(64, 16)] * 2, [dev(32, 8)] * 2), "W\\[0\\] has shape"),
        (lambda: tp.matmul_dx([dev(64, 16)] * 2, [dev(32, 16)] * 2, tp.REDUCESCATTER, dX=[dev(64, 32)] * 2),
         "dX\\[0\\] has shape"),
        (lambda: tp.weight_grad([dev(64, 32)] * 2, [dev(60, 16)] * 2), "B\\[0\\] has shape"),
        (lambda: tp.rowpar_dx(dev(64, 16), [dev(32, 16), dev(32, 8)]), "W\\[1\\] has shape"),
        (lambda: tp.rowpar_dx(dev(64, 16), [dev(32, 16)] * 2, dX=[dev(64, 32)]), "one per shard"),
        (lambda: tp.mlp_sp([dev(32, 16)] * 2, [dev(16, 24)] * 2, [dev(16, 24)] * 2), "W2\\[0\\] has shape"),
        (lambda: tp.mlp_sp([dev(32, 16)] * 2, [dev(16, 24)] * 2, [dev(24, 16)] * 2,
                           H=[dev(64, 24, dtype=torch.float32)] * 2), "H\\[0\\] has dtype"),
    ]
    for call, msg in cases:
        with pytest.raises(ValueError, match=msg):
            call()


def test_default_handles_are_per_stream(monkeypatch):
    """A handle runs one call at a time, so the binding keeps one default
    handle per (device, stream): calls on two streams never share the work
    queue or readiness counters of one handle.  Host-only (fake handles)."""
    created = []

    class FakeHandle:
        def __init__(self, dev):
            created.append(dev)
            self.device = dev

    class FakeStream:
        def __init__(self, ptr):
            self.cuda_stream = ptr

    monkeypatch.setattr(tp, "Handle", FakeHandle)
    monkeypatch.setattr(tp, "_default_handles", {})
    a = tp.default_handle(0, FakeStream(0x10))
    b = tp.default_handle(0, FakeStream(0x20))
    c = tp.default_handle(0, FakeStream(0x10))
    d = tp.default_handle(1, FakeStream(0x10))
    assert a is c and a is not b and d is not a
    assert created == [0, 0, 1]


@pytest.mark.gpu
def test_side_stream_call_allocates_on_its_stream():
    """A call on a side stream with binding-allocated workspace and output
    gives the same bits as the same call on the current stream (the buffers
    belong to the side stream's allocator pool, and the call uses that
    stream's own default handle)."""
    p, M, N, K = 4, 512, 512, 256
    g = torch.Generator(device="cuda").manual_seed(5)
    X = [torch.randn(M, K, device="cuda", generator=g).to(BF) for _ in range(p)]
    W = [(torch.randn(K, N, device="cuda", generator=g) * 0.02).to(BF) for _ in range(p)]
    ref = tp.matmul_allreduce(X, W, n_chunks=4, sched="persistent")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for sched in ("persistent", "tile", "unfused", "fold"):
        outs.append(tp.matmul_allreduce(X, W, n_chunks=4, sched=sched, stream=side))
    side.synchronize()
    torch.cuda.synchronize()
    assert tp.default_handle(0, side) is not tp.default_handle(0)
    for y in outs:
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
