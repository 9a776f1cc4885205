"""The algorithmic counts that bench.py's roofline divides by: FLOPs of each
workload and the HBM bytes of one launch of its dominant kernel, checked
against an inventory of the tensors that launch touches (shape x element
size, each read or written once)."""
import pytest

import bench
from tensor_gemm_reduction_amd.inputs import WORKLOADS

BF16, F32 = 2, 4


def nbytes(shape, es):
    n = 1
    for d in shape:
        n *= d
    return n * es


def test_headline_counts_by_hand():
    # MLP down projection: p = 4 shards of X_k [4096, 4096] . W_k [4096, 4096]
    wl = WORKLOADS["mlp_down"]
    assert wl.flops() == 2 * 4096 ** 3 * 4 == 549_755_813_888
    # fold pair: operands once (4 x 2 x 32 MiB), 3 fp32 partials written and
    # read back (3 x 2 x 64 MiB), one bf16 result (32 MiB)
    MiB = 1 << 20
    assert bench.kernel_bytes(wl, 4, "fold") == 4 * 2 * 32 * MiB + 3 * 2 * 64 * MiB + 32 * MiB == 704_643_072


@pytest.mark.parametrize("name", ["worked", "mlp_down", "sp_rs", "decode16", "decode64"])
@pytest.mark.parametrize("part", [F32, BF16])
def test_reducing_gemm_bytes(name, part):
    wl = WORKLOADS[name]
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    X = [nbytes((M, K), BF16)] * p
    W = [nbytes((K, N), BF16)] * p
    partials = [nbytes((M, N), part)] * p
    assert bench.kernel_bytes(wl, part, "unfused") == sum(X) + sum(W) + sum(partials)
    # fold: the last shard's partial is never stored; the other p - 1 are
    # written by the first launch and read by the second, which writes Y
    fold = sum(X) + sum(W) + 2 * sum(partials[:-1]) + nbytes((M, N), BF16)
    assert bench.kernel_bytes(wl, part, "fold") == fold


def test_dx_bytes():
    wl = WORKLOADS["dx_bwd"]        # dY_k [M, N_shard], W_k [K_in, N_shard], dX [M, K_in]
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    ops = p * (nbytes((M, N), BF16) + nbytes((K, N), BF16))
    assert bench.kernel_bytes(wl, F32, "unfused") == ops + p * nbytes((M, K), F32)
    assert bench.kernel_bytes(wl, F32, "fold") == ops + 2 * (p - 1) * nbytes((M, K), F32) + nbytes((M, K), BF16)
    assert wl.flops() == 2 * M * N * K * p


def test_allgather_and_wgrad_bytes():
    ag = WORKLOADS["ag_fwd"]        # X_gathered [M, K], W [K, N_shard], Y [M, N_shard]
    assert bench.kernel_bytes(ag) == nbytes((ag.M, ag.K), BF16) + nbytes((ag.K, ag.N), BF16) + nbytes((ag.M, ag.N), BF16)
    assert ag.flops() == 2 * ag.M * ag.K * ag.N
    for name in ("dw_col", "dw_row"):
        wl = WORKLOADS[name]        # A_k [M, K], B_k [M, N], dW_k [K, N] fp32
        p, M, N, K = wl.p, wl.M, wl.N, wl.K
        assert bench.kernel_bytes(wl) == p * (nbytes((M, K), BF16) + nbytes((M, N), BF16) + nbytes((K, N), F32))
        assert wl.flops() == 2 * M * N * K * p


def test_mlp_sp_bytes():
    wl = WORKLOADS["mlp_sp"]        # FC2 launch: H_k [M, K], W2_k [K, N], partials [M, N]
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    ops = p * (nbytes((M, K), BF16) + nbytes((K, N), BF16))
    assert bench.kernel_bytes(wl, F32, "unfused") == ops + p * nbytes((M, N), F32)
    assert bench.kernel_bytes(wl, F32, "fold") == ops + 2 * (p - 1) * nbytes((M, N), F32) + nbytes((M, N), BF16)
    assert wl.flops() == 2 * (2 * M * N * K * p)     # FC1 and FC2


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says so,
    before it touches a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_rowpar_dx_bytes():
    wl = WORKLOADS["dx_row"]        # dY [M, N] read once for every shard, W_k [K, N], dX_k [M, K] bf16
    p, M, N, K = wl.p, wl.M, wl.N, wl.K
    assert bench.kernel_bytes(wl) == nbytes((M, N), BF16) + p * (nbytes((K, N), BF16) + nbytes((M, K), BF16))
    assert wl.flops() == 2 * M * N * K * p
