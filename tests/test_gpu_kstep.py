"""K-step edges of the large GEMM tile (more than 64 output rows): reduction
lengths of 1 to 13 whole 64-wide steps (the interleaved loads, the
three-slot A ring and its six-step unroll, the loads repeated past the last
step) and lengths with a tail step (the checked path), for every operand
layout: row-major weights (MatMul -> AllReduce), transposed weights (dX and
row-parallel dX) and transposed activations (weight gradients).  Integer
inputs make every fp32 result exact, so each output element is compared for
equality with the float64 oracle, and the schedulers are compared bit for
bit with each other."""
import numpy as np
import pytest
import torch

from oracle import tpf_oracle as O
from tensor_gemm_reduction_amd import inputs, tpfuse as tp

pytestmark = pytest.mark.gpu

DEV = "cuda"
# whole 64-wide steps: 1 .. 7 and 13; with a tail step: 8, 72, 200, 392
KS = [64, 128, 192, 256, 320, 384, 448, 832, 8, 72, 200, 392]


def ints(rng, shape):
    return torch.from_numpy(rng.integers(-2, 3, shape).astype(np.float32)).to(torch.bfloat16)


def bits(ts):
    return [inputs.bf16_to_bits(t) for t in ts]


def exact(t, ref, what):
    got = t.cpu().double().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} elements differ, first at {tuple(bad[0])}: {got[tuple(bad[0])]} vs " \
                          f"{ref[tuple(bad[0])]}"


@pytest.mark.parametrize("K", KS)
def test_allreduce_kstep(K):
    p, M, N = 3, 520, 264
    print(f"kstep allreduce p={p} M={M} N={N} K={K}", flush=True)
    rng = np.random.default_rng(1000 + K)
    Xh = [ints(rng, (M, K)) for _ in range(p)]
    Wh = [ints(rng, (K, N)) for _ in range(p)]
    ref = O.matmul_allreduce(bits(Xh), bits(Wh))
    X, W = [t.to(DEV) for t in Xh], [t.to(DEV) for t in Wh]
    outs = {}
    for sched in ("unfused", "fold", "tile", "persistent", "two_stream", "stationary"):
        y = tp.matmul_allreduce(X, W, torch.float32, n_chunks=2, sched=sched)
        torch.cuda.synchronize()
        exact(y, ref, f"allreduce K={K} {sched}")
        outs[sched] = y
    for sched, y in outs.items():
        assert torch.equal(y, outs["unfused"]), f"allreduce K={K} {sched} vs unfused"


@pytest.mark.parametrize("K", KS)
def test_dx_kstep(K):
    # dX = sum_k dY_k W_k^T: the reduction runs over the shard width K
    p, M, C = 3, 520, 264
    print(f"kstep dx p={p} M={M} K_in={C} N_shard={K}", flush=True)
    rng = np.random.default_rng(2000 + K)
    dYh = [ints(rng, (M, K)) for _ in range(p)]
    Wh = [ints(rng, (C, K)) for _ in range(p)]
    ref = O.matmul_dx(bits(dYh), bits(Wh))
    dY, W = [t.to(DEV) for t in dYh], [t.to(DEV) for t in Wh]
    outs = {}
    for sched in ("unfused", "fold", "persistent", "stationary"):
        y = tp.matmul_dx(dY, W, tp.ALLREDUCE, torch.float32, n_chunks=2, sched=sched)
        torch.cuda.synchronize()
        exact(y, ref, f"dx K={K} {sched}")
        outs[sched] = y
    for sched, y in outs.items():
        assert torch.equal(y, outs["unfused"]), f"dx K={K} {sched} vs unfused"


@pytest.mark.parametrize("K", KS)
def test_rowpar_dx_kstep(K):
    # dX_k = dY W_k^T: the reduction runs over the output width N = K here
    p, M, Ks = 2, 300, 264
    print(f"kstep row-parallel dx p={p} M={M} K_shard={Ks} N={K}", flush=True)
    rng = np.random.default_rng(3000 + K)
    dYh = ints(rng, (M, K))
    Wh = [ints(rng, (Ks, K)) for _ in range(p)]
    refs = O.rowpar_dx(inputs.bf16_to_bits(dYh), bits(Wh))
    d = tp.rowpar_dx(dYh.to(DEV), [w.to(DEV) for w in Wh], torch.float32)
    torch.cuda.synchronize()
    for k in range(p):
        exact(d[k], refs[k], f"row-parallel dx K={K} shard {k}")


@pytest.mark.parametrize("K", KS)
def test_weight_grad_kstep(K):
    # dW_k = A_k^T B_k: the reduction runs over the rows M = K here
    p, R, C = 2, 304, 264
    print(f"kstep weight gradient p={p} rows={K} R={R} C={C}", flush=True)
    rng = np.random.default_rng(4000 + K)
    Ah = [ints(rng, (K, R)) for _ in range(p)]
    Bh = [ints(rng, (K, C)) for _ in range(p)]
    refs = O.weight_grad(bits(Ah), bits(Bh))
    d = tp.weight_grad([a.to(DEV) for a in Ah], [b.to(DEV) for b in Bh], torch.float32)
    torch.cuda.synchronize()
    for k in range(p):
        exact(d[k], refs[k], f"weight gradient K={K} shard {k}")
