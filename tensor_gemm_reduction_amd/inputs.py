"""Seeded synthetic inputs for the fused tensor-parallel Linear workloads.

This module only draws random numbers and shapes them; it holds none of the
arithmetic of the method (no products, no sums, no reductions).  Both the CPU
oracle (via the tests) and the HIP path consume exactly the tensors produced
here, so parity compares like with like.

Every workload is defined by the shapes and value distributions of the
tensor-parallel Linear it stands for:

* ``worked``  – the two-shard worked example of the ai-infra-kb M027 page
  (section 03 "两卡与四个输出块"): X_r [128,1024], W_r [1024,2048], M split
  into four 32-row chunks, AllReduce semantics.  X ~ U(-1,1), W ~ N(0, 1/32).
* ``mlp_down`` – a Llama-style MLP down projection, row-parallel over p=4:
  X_k [4096,4096], W_k [4096,4096], X ~ N(0,1), W ~ N(0,0.02), 8 chunks.
* ``sp_rs``   – a sequence-parallel MatMul+ReduceScatter, p=8: X_k [8192,3584],
  W_k [3584,8192], both N(0,0.02), 16 chunks, output as 8 row slices.
* ``ag_fwd``  – GPT-3-shaped AllGather->MatMul, p=8: slices [256,12288]
  N(0,1), one column shard W_0 [12288,6144] N(0,0.02), 8 chunks (one per
  slice).
* ``dx_bwd``  – the column-parallel backward dX = sum_k dY_k W_k^T for the same
  layer: dY_k [2048,6144] N(0,1), W_k [12288,6144] N(0,0.02), 8 chunks.
* ``decode16`` / ``decode64`` – decode-shaped row-parallel GEMMs, p=8:
  X_k [M,1024], W_k [1024,8192], both N(0,0.02), chunk counts 1/2/4.
* ``mlp_sp`` – the MLP block of the same GPT-3 layer under sequence
  parallelism, p=8: slices [256,12288] N(0,1), W1_k [12288,6144] and
  W2_k [6144,12288] N(0,0.02).
* ``dw_col`` – the weight gradient of the ``ag_fwd`` column shard layer,
  dW_k = X^T dY_k: gathered X [2048,12288], dY_k [2048,6144], both N(0,1).
* ``dw_row`` – the weight gradient of the ``mlp_down`` row-parallel layer,
  dW_k = X_k^T dY: X_k [4096,4096], dY [4096,4096], both N(0,1).

``N(0, s)`` is read as standard deviation ``s``.

Values are drawn in float32 from torch's counter-free CPU Mersenne-Twister
generator (or a CUDA generator for speed when ``device`` is a GPU) and then
rounded to bfloat16 by torch's round-to-nearest-even conversion.  The integer
mode draws integers uniformly from {-2,...,2}; those are exact in bfloat16
and every partial sum of the configured sizes stays exact in float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import torch

# A fixed base so that the seed of each tensor is a plain function of
# (workload, role, shard) and no two tensors share a stream.
_SEED_BASE = 0x7470660000
_ROLE = {"X": 0, "W": 1, "dY": 2, "Xs": 3}


@dataclass(frozen=True)
class Workload:
    """Shapes and value distributions of one tensor-parallel Linear workload."""

    name: str
    op: str                  # "allreduce" | "reducescatter" | "allgather" | "dx"
    p: int                   # number of simulated ranks (shards)
    M: int                   # rows (tokens)
    N: int                   # output columns (per shard for allgather / dx: see below)
    K: int                   # reduction length per shard (full K for allgather)
    chunks: tuple            # chunk counts exercised; the first one is the default
    x_dist: tuple            # ("uniform", a) -> U(-a, a); ("normal", s) -> N(0, s)
    w_dist: tuple
    index: int = 0           # stable workload number used in seeds
    out_dtypes: tuple = ("bf16",)
    note: str = ""

    @property
    def default_chunks(self) -> int:
        return self.chunks[0]

    def flops(self) -> float:
        """Algorithmic multiply-add FLOPs of the whole op (2 per MAC)."""
        if self.op == "allgather":
            return 2.0 * self.M * self.K * self.N
        if self.op in ("wgrad_col", "wgrad_row"):
            # p GEMMs dW_k [K, N] = A_k^T B_k over M rows
            return 2.0 * self.M * self.K * self.N * self.p
        if self.op == "mlp_sp":
            # FC1 [M, N] x [N, K] and FC2 [M, K] x [K, N] on each of p shards
            return 4.0 * self.M * self.N * self.K * self.p
        if self.op == "dx":
            # dX [M, K] = sum over p shards of dY_k [M, N] . W_k^T
            return 2.0 * self.M * self.N * self.K * self.p
        return 2.0 * self.M * self.K * self.N * self.p


# dx_bwd: M rows, N = N_shard (reduction length per shard), K = K_in (output cols)
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("worked", "allreduce", 2, 128, 2048, 1024, (4, 1, 2),
                 ("uniform", 1.0), ("normal", 1.0 / 32.0), index=1,
                 out_dtypes=("f32", "bf16"),
                 note="two-shard worked example, four 32-row chunks"),
        Workload("mlp_down", "allreduce", 4, 4096, 4096, 4096, (8, 1, 2, 4),
                 ("normal", 1.0), ("normal", 0.02), index=2,
                 out_dtypes=("bf16", "f32"),
                 note="Llama-style MLP down projection, ffn 16384 -> h 4096"),
        Workload("sp_rs", "reducescatter", 8, 8192, 8192, 3584, (16, 1, 4),
                 ("normal", 0.02), ("normal", 0.02), index=3,
                 note="sequence-parallel MatMul+ReduceScatter, ffn 28672 -> h 8192"),
        Workload("ag_fwd", "allgather", 8, 2048, 6144, 12288, (8, 1, 4),
                 ("normal", 1.0), ("normal", 0.02), index=4,
                 note="GPT-3 FC1 column shard, sequence slices [256,12288]"),
        Workload("dx_bwd", "dx", 8, 2048, 6144, 12288, (8, 1, 4),
                 ("normal", 1.0), ("normal", 0.02), index=4,
                 note="column-parallel backward dX for the GPT-3 FC1 shard"),
        Workload("decode16", "allreduce", 8, 16, 8192, 1024, (1, 2, 4),
                 ("normal", 0.02), ("normal", 0.02), index=5,
                 note="decode step, 16 tokens"),
        Workload("decode64", "allreduce", 8, 64, 8192, 1024, (1, 2, 4),
                 ("normal", 0.02), ("normal", 0.02), index=6,
                 note="decode step, 64 tokens"),
        Workload("mlp_sp", "mlp_sp", 8, 2048, 12288, 6144, (8, 1, 4),
                 ("normal", 1.0), ("normal", 0.02), index=9,
                 note="GPT-3 MLP block under sequence parallelism: AllGather, FC1 column shard + GeLU, "
                      "FC2 row shard, ReduceScatter (N = hidden, K = ffn shard)"),
        Workload("dw_col", "wgrad_col", 8, 2048, 6144, 12288, (1,),
                 ("normal", 1.0), ("normal", 1.0), index=7, out_dtypes=("f32",),
                 note="column-parallel weight gradient dW_k = X^T dY_k of the GPT-3 FC1 shard"),
        Workload("dw_row", "wgrad_row", 4, 4096, 4096, 4096, (1,),
                 ("normal", 1.0), ("normal", 1.0), index=8, out_dtypes=("f32",),
                 note="row-parallel weight gradient dW_k = X_k^T dY of the MLP down projection"),
        Workload("dx_row", "rowpar_dx", 4, 4096, 4096, 4096, (1,),
                 ("normal", 1.0), ("normal", 0.02), index=10,
                 note="row-parallel input gradient dX_k = dY W_k^T of the MLP down projection "
                      "(N = the layer's output width, K = the shard's input width)"),
    ]
}


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw(shape, dist, seed: int, mode: str = "random", device: str = "cpu") -> torch.Tensor:
    """One bfloat16 tensor of ``shape``.

    ``dist`` is ("uniform", a) for U(-a, a) or ("normal", s) for N(0, s).
    ``mode == "int"`` ignores ``dist`` and draws integers in {-2, ..., 2}.
    """
    g = _gen(seed, device)
    if mode == "int":
        t = torch.randint(-2, 3, tuple(shape), generator=g, device=device, dtype=torch.int32)
        return t.to(torch.bfloat16)
    if mode != "random":
        raise ValueError(f"unknown input mode {mode!r}")
    kind, scale = dist
    if kind == "uniform":
        t = torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)
        t = (t * 2.0 - 1.0) * scale
    elif kind == "normal":
        t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32) * scale
    else:
        raise ValueError(f"unknown distribution {kind!r}")
    return t.to(torch.bfloat16)


def tensor_seed(workload_index: int, role: str, shard: int, seed: int = 0) -> int:
    return _SEED_BASE + 100000 * seed + 1000 * workload_index + 10 * _ROLE[role] + shard


@dataclass
class Inputs:
    """The bf16 operands of one workload instance (row-major, contiguous)."""

    workload: Workload
    M: int
    N: int
    K: int
    p: int
    X: List[torch.Tensor] = field(default_factory=list)    # per-shard activations / dY / slices
    W: List[torch.Tensor] = field(default_factory=list)    # per-shard weights (one for allgather)


def make_inputs(wl: Workload, seed: int = 0, mode: str = "random", device: str = "cpu",
                M: Optional[int] = None, N: Optional[int] = None, K: Optional[int] = None,
                p: Optional[int] = None) -> Inputs:
    """Draw the operands of ``wl`` (optionally with overridden sizes).

    Layouts (all row-major bf16):
      allreduce / reducescatter: X[k] [M, K], W[k] [K, N]     (k < p)
      allgather:                 X[r] [M/p, K] (slices), W[0] [K, N]
      dx:                        X[k] = dY_k [M, N], W[k] [K, N]  (K = K_in, N = N_shard)
      mlp_sp:                    X[r] [M/p, N] (slices), W[k] = W1_k [N, K], W[p + k] = W2_k [K, N]
      wgrad_col:                 X[0] = gathered input [M, K], W[k] = dY_k [M, N]
      wgrad_row:                 X[k] = X_k [M, K], W[0] = dY [M, N]
      rowpar_dx:                 X[0] = dY [M, N], W[k] = W_k [K, N]
    """
    M = wl.M if M is None else M
    N = wl.N if N is None else N
    K = wl.K if K is None else K
    p = wl.p if p is None else p
    inp = Inputs(wl, M, N, K, p)
    idx = wl.index
    if wl.op in ("allreduce", "reducescatter"):
        for k in range(p):
            inp.X.append(draw((M, K), wl.x_dist, tensor_seed(idx, "X", k, seed), mode, device))
            inp.W.append(draw((K, N), wl.w_dist, tensor_seed(idx, "W", k, seed), mode, device))
    elif wl.op == "allgather":
        if M % p:
            raise ValueError("allgather needs M divisible by p")
        for r in range(p):
            inp.X.append(draw((M // p, K), wl.x_dist, tensor_seed(idx, "Xs", r, seed), mode, device))
        inp.W.append(draw((K, N), wl.w_dist, tensor_seed(idx, "W", 0, seed), mode, device))
    elif wl.op == "dx":
        for k in range(p):
            inp.X.append(draw((M, N), wl.x_dist, tensor_seed(idx, "dY", k, seed), mode, device))
            inp.W.append(draw((K, N), wl.w_dist, tensor_seed(idx, "W", k, seed), mode, device))
    elif wl.op == "mlp_sp":
        if M % p:
            raise ValueError("mlp_sp needs M divisible by p")
        for r in range(p):
            inp.X.append(draw((M // p, N), wl.x_dist, tensor_seed(idx, "Xs", r, seed), mode, device))
        for k in range(p):
            inp.W.append(draw((N, K), wl.w_dist, tensor_seed(idx, "W", k, seed), mode, device))
        for k in range(p):
            inp.W.append(draw((K, N), wl.w_dist, tensor_seed(idx, "W", 100 + k, seed), mode, device))
    elif wl.op == "wgrad_col":
        inp.X.append(draw((M, K), wl.x_dist, tensor_seed(idx, "X", 0, seed), mode, device))
        for k in range(p):
            inp.W.append(draw((M, N), wl.w_dist, tensor_seed(idx, "dY", k, seed), mode, device))
    elif wl.op == "wgrad_row":
        for k in range(p):
            inp.X.append(draw((M, K), wl.x_dist, tensor_seed(idx, "X", k, seed), mode, device))
        inp.W.append(draw((M, N), wl.w_dist, tensor_seed(idx, "dY", 0, seed), mode, device))
    elif wl.op == "rowpar_dx":
        inp.X.append(draw((M, N), wl.x_dist, tensor_seed(idx, "dY", 0, seed), mode, device))
        for k in range(p):
            inp.W.append(draw((K, N), wl.w_dist, tensor_seed(idx, "W", k, seed), mode, device))
    else:
        raise ValueError(f"unknown op {wl.op!r}")
    return inp


def weight_grad_operands(inp: Inputs):
    """The per-shard (A, B) lists of a weight-gradient workload: dW_k = A_k^T B_k."""
    if inp.workload.op == "wgrad_col":
        return [inp.X[0]] * inp.p, list(inp.W)
    return list(inp.X), [inp.W[0]] * inp.p


def bf16_to_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bit patterns (copied to CPU)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
