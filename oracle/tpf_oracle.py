"""CPU oracle for the fused tensor-parallel Linear (MatMul + cross-shard reduction).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library
and its Python binding) never calls it and shares no code with it.

It is plain and slow on purpose: every result is the textbook definition,
computed in float64 with numpy, so that a reader can check it against the
pages by eye.  Inputs are bfloat16 bit patterns (numpy ``uint16``) exactly as
the GPU receives them; products of two bf16 values are exact in float64 and
the sums carry ~2^-53 relative error, far below every tolerance used.

Sources (web pages; section names as printed on them):

* ai-infra-kb M027 "compute-communication fusion" page:
  - §01 一层里的计算和通信依赖: row-parallel Linear, Y_r = X_r W_r, Y = Y_0 + Y_1;
    AllReduce (every rank holds Y) versus ReduceScatter (each rank holds its
    slice) are different output layouts; AllGather then MatMul.
  - §02 MC² 的计算—通信协同: MatMul->AllReduce chunked along output rows;
    AllGather->MatMul starts compute once enough input blocks arrived.
  - §03 两卡与四个输出块: the worked example (X_r [128,1024], W_r [1024,2048],
    four 32-row chunks, 512 KiB local output and 128 KiB per chunk at two bytes
    per element) and the timeline model (serial 20 ms, pipelined 14 ms).
* cnblogs "张量并行：列并行与行并行的前向/反向传播…" tutorial page:
  - §2.3 列并行 / §三: column shards A_k = A[:, k*out/p:(k+1)*out/p], Y_k = X A_k,
    Y = [Y_0 | ... | Y_{p-1}]; backward dX = sum_k dY_k A_k^T.
  - §2.4 行并行 / §四: row shards A_k = A[k*in/p:(k+1)*in/p, :],
    X_k = X[:, k*in/p:(k+1)*in/p], Y = sum_k X_k A_k.
  - §2.5-2.7: AllReduce sums, AllGather concatenates, ReduceScatter = reduce
    then scatter a slice to each rank.
  - §6.1 / §6.4: the column-parallel dX needs the sum over shards.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  R4  partial results are summed from exact per-shard products (the oracle
      keeps them in float64; it has no "message" precision).  The separate
      2-byte message functions at the end round each rank's local output to
      bfloat16 and sum in binary32 in rank order.
  R5  reduction order is irrelevant to the oracle (float64, exact-enough).
  R6  shard k owns the k-th contiguous block of the split dimension.
  R7  chunks are contiguous row ranges in order; the last takes the remainder.
  R8  ReduceScatter slice r is the r-th contiguous block of M/p rows.
  R10 AllGather concatenates the p slices in rank order.
  R13 the reduction is a sum, not a mean.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

import numpy as np

# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns as float64.

    A bfloat16 is the upper 16 bits of an IEEE binary32; shifting the pattern
    left by 16 gives the binary32 with the same value, which float64 holds
    exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest, ties to even) in one step.

    bfloat16 keeps 8 significant bits and binary32's exponent range, so a
    finite x with 2^(e-1) <= |x| < 2^e has quantum 2^(e-8), never finer than
    the subnormal quantum 2^-133.  Dividing by the quantum is an exact power-of
    -two scaling, numpy's ``rint`` rounds half to even, and multiplying back is
    exact.  Rounding directly from float64 avoids the double rounding of going
    through float32 first.  Results at or beyond 2^128 become infinity; NaN
    stays NaN.  Returns the uint16 bit patterns.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    _, e = np.frexp(xf)                       # xf = m * 2**e, 0.5 <= |m| < 1
    q_exp = np.maximum(e - 8, -133)           # quantum exponent
    scaled = np.ldexp(xf, -q_exp)             # exact
    y = np.ldexp(np.rint(scaled), q_exp)      # exact
    y = np.where(np.abs(y) >= 2.0 ** 128, np.copysign(np.inf, y), y)
    out[...] = np.where(finite, y, np.where(np.isnan(x), 0.0, x))
    # Every value is now exactly representable as bfloat16, hence as binary32,
    # so its bfloat16 pattern is the top half of its binary32 pattern.
    bits = (out.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)


# --------------------------------------------------------------------------
# Chunking and message sizes (M027 page §02-§03)
# --------------------------------------------------------------------------


def chunk_bounds(M: int, n: int) -> List[Tuple[int, int]]:
    """Contiguous row ranges of the n output chunks, in order.

    Each chunk has floor(M/n) rows; the last one also takes the remainder
    (reading R7 of the worked example "M=128 cut into 4 blocks of 32 rows").
    """
    if n < 1 or n > M:
        raise ValueError("need 1 <= n <= M")
    base = M // n
    return [(c * base, (c + 1) * base if c < n - 1 else M) for c in range(n)]


def message_bytes(rows: int, cols: int, elt_bytes: int) -> int:
    """Bytes of one rows x cols block of the local output (the message)."""
    return rows * cols * elt_bytes


def serial_time(n: int, t_compute: float, t_comm: float) -> float:
    """Serial schedule of the M027 page §03: every chunk computes, then communicates."""
    return n * (t_compute + t_comm)


def pipeline_time(n: int, t_compute: float, t_comm: float) -> float:
    """Ideal two-engine pipeline of the M027 page §03.

    The first chunk's compute, then n-1 stages each bounded by the slower of
    compute and communication, then the last chunk's communication.
    """
    return t_compute + (n - 1) * max(t_compute, t_comm) + t_comm


# --------------------------------------------------------------------------
# The operations (plain definitions)
# --------------------------------------------------------------------------


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def shard_products(X_shards: Sequence, W_shards: Sequence, rows=None) -> List[np.ndarray]:
    """Per-rank local outputs Y_k = X_k W_k (row-parallel, cnblogs §2.4), float64.

    ``rows`` optionally restricts the result to a subset of output rows.
    """
    if len(X_shards) != len(W_shards):
        raise ValueError("X and W need one block per shard")
    out = []
    for Xk, Wk in zip(X_shards, W_shards):
        xk = _f64(Xk)
        if rows is not None:
            xk = xk[np.asarray(rows)]
        out.append(xk @ _f64(Wk))
    return out


def matmul_allreduce(X_shards: Sequence, W_shards: Sequence, rows=None) -> np.ndarray:
    """Row-parallel Linear with AllReduce semantics: Y = sum_k X_k W_k (full Y).

    M027 page §01 (Y = Y_0 + Y_1); cnblogs §2.4 / §四 (Y = sum_k X_k A_k),
    §2.5 (AllReduce is an element-wise sum; reading R13: sum, not mean).
    """
    parts = shard_products(X_shards, W_shards, rows)
    y = np.zeros_like(parts[0])
    for part in parts:
        y = y + part
    return y


def matmul_allreduce_chunked(X_shards: Sequence, W_shards: Sequence, n: int) -> np.ndarray:
    """The same result assembled chunk by chunk, in the pages' loop order.

    M027 page §03: for each chunk (same order on every rank) each rank forms its
    local output rows, and the ranks' blocks for the same chunk are summed.
    """
    M = np.asarray(X_shards[0]).shape[0]
    N = np.asarray(W_shards[0]).shape[1]
    y = np.zeros((M, N), dtype=np.float64)
    for r0, r1 in chunk_bounds(M, n):
        local = shard_products(X_shards, W_shards, rows=np.arange(r0, r1))
        acc = np.zeros((r1 - r0, N), dtype=np.float64)
        for blk in local:
            acc = acc + blk
        y[r0:r1] = acc
    return y


def scatter_rows(Y: np.ndarray, p: int) -> List[np.ndarray]:
    """Slices of a reduced result as ReduceScatter hands them out.

    cnblogs §2.7: each rank receives one slice of the reduced data; reading R8:
    rank r owns rows [r*M/p, (r+1)*M/p).
    """
    M = Y.shape[0]
    if M % p:
        raise ValueError("ReduceScatter needs M divisible by p")
    s = M // p
    return [Y[r * s:(r + 1) * s] for r in range(p)]


def matmul_reducescatter(X_shards: Sequence, W_shards: Sequence) -> List[np.ndarray]:
    """Row-parallel Linear with ReduceScatter semantics (M027 page §01)."""
    return scatter_rows(matmul_allreduce(X_shards, W_shards), len(X_shards))


def allgather(X_slices: Sequence) -> np.ndarray:
    """AllGather of row slices in rank order (cnblogs §2.6: concatenation, no reduction)."""
    return np.concatenate([_f64(s) for s in X_slices], axis=0)


def allgather_matmul(X_slices: Sequence, W) -> Tuple[np.ndarray, np.ndarray]:
    """AllGather of sequence slices, then the column-parallel GEMM Y_k = X W_k.

    M027 page §01 / §02 (gather the input, then MatMul); cnblogs §2.3 (column
    shard, Y_k = X A_k, no reduction).  Returns (X_gathered, Y_k), float64.
    """
    xg = allgather(X_slices)
    return xg, xg @ _f64(W)


def matmul_dx(dY_shards: Sequence, W_shards: Sequence, rows=None) -> np.ndarray:
    """Column-parallel input gradient dX = sum_k dY_k W_k^T.

    cnblogs §三 and §6.1 / §6.4: every column shard contributes dY_k A_k^T to
    dX, so the shards' contributions are summed (AllReduce).  W_k is stored
    [K_in, N_shard] (the forward's A_k), used transposed.
    """
    dx = None
    for dYk, Wk in zip(dY_shards, W_shards):
        d = _f64(dYk)
        if rows is not None:
            d = d[np.asarray(rows)]
        term = d @ _f64(Wk).T
        dx = term if dx is None else dx + term
    return dx


def matmul_dx_reducescatter(dY_shards: Sequence, W_shards: Sequence) -> List[np.ndarray]:
    """dX delivered as p row slices (sequence-parallel layout, reading R11)."""
    return scatter_rows(matmul_dx(dY_shards, W_shards), len(dY_shards))


# --------------------------------------------------------------------------
# The 2-byte message variant (M027 page §03: a rank's local output is sized
# at two bytes per element, 512 KiB per rank and 128 KiB per 32-row chunk in
# the worked example)
# --------------------------------------------------------------------------


def bf16_message(part: np.ndarray) -> np.ndarray:
    """A rank's local output as sent at two bytes per element.

    Each value is rounded once, to nearest with ties to even, to bfloat16
    (reading: the 2-byte element of the worked example is bfloat16, the
    inputs' format); returned as float64 (exact).
    """
    return bf16_bits_to_f64(round_to_bf16_bits(part))


def sum_messages_f32(messages: Sequence) -> np.ndarray:
    """Fixed-order binary32 sum of received messages: ((m_0 + m_1) + m_2) + ...

    Every addition is rounded to binary32 (numpy float32 arithmetic rounds to
    nearest even), in rank order k = 0..p-1 (reading R5).  The messages are
    bfloat16 values, hence exact in binary32.  Returned as float64 (exact).
    """
    acc = np.asarray(messages[0], dtype=np.float64).astype(np.float32)
    for m in messages[1:]:
        acc = (acc + np.asarray(m, dtype=np.float64).astype(np.float32)).astype(np.float32)
    return acc.astype(np.float64)


def matmul_allreduce_msg_bf16(X_shards: Sequence, W_shards: Sequence, rows=None) -> np.ndarray:
    """Y = sum_k bf16(X_k W_k): the row-parallel sum over 2-byte messages.

    M027 page §01 (Y = Y_0 + Y_1) with each rank's local output Y_k sent as a
    bfloat16 message (§03) and summed in binary32 in rank order.  The result is
    the binary32 sum before the final rounding to the output type.
    """
    return sum_messages_f32([bf16_message(part) for part in shard_products(X_shards, W_shards, rows)])


def matmul_dx_msg_bf16(dY_shards: Sequence, W_shards: Sequence, rows=None) -> np.ndarray:
    """dX = sum_k bf16(dY_k W_k^T) (cnblogs §三, §6.4) over 2-byte messages."""
    terms = []
    for dYk, Wk in zip(dY_shards, W_shards):
        d = _f64(dYk)
        if rows is not None:
            d = d[np.asarray(rows)]
        terms.append(bf16_message(d @ _f64(Wk).T))
    return sum_messages_f32(terms)


# --------------------------------------------------------------------------
# Weight gradients (cnblogs §三 / §四 backward: local GEMMs, no communication)
# --------------------------------------------------------------------------


def weight_grad(A_shards: Sequence, B_shards: Sequence) -> List[np.ndarray]:
    """dW_k = A_k^T B_k for every shard, float64.

    Row-parallel Linear Y = sum_k X_k W_k: dL/dW_k = X_k^T dY (A_k = X_k,
    B_k = dY for every k).  Column-parallel Y_k = X W_k: dL/dW_k = X^T dY_k
    (A_k = the gathered X for every k, B_k = dY_k).
    """
    if len(A_shards) != len(B_shards):
        raise ValueError("A and B need one block per shard")
    return [_f64(a).T @ _f64(b) for a, b in zip(A_shards, B_shards)]


def rowpar_dx(dY, W_shards: Sequence) -> List[np.ndarray]:
    """dX_k = dY W_k^T for every shard, float64.

    Row-parallel Linear Y = sum_k X_k W_k (cnblogs §四): the output gradient
    dY reaches every rank whole, and dL/dX_k = dY W_k^T is each rank's local
    product; no communication.
    """
    d = _f64(dY)
    return [d @ _f64(w).T for w in W_shards]


# --------------------------------------------------------------------------
# The MLP block under sequence parallelism (cnblogs §7.1 and §11.3):
# AllGather -> column-parallel FC1 -> GeLU -> row-parallel FC2 -> ReduceScatter
# --------------------------------------------------------------------------


def gelu(x: np.ndarray) -> np.ndarray:
    """GeLU(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt(2))), float64.

    Reading: the exact (erf) form; the pages name the activation without
    choosing between it and the tanh approximation.
    """
    import math
    x = np.asarray(x, dtype=np.float64)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def mlp_sp_hidden(X_slices: Sequence, W1_shards: Sequence) -> List[np.ndarray]:
    """H_k = bf16(GeLU(X W1_k)): the column shards' activations.

    X is the AllGather of the sequence slices in rank order (cnblogs §2.6);
    each rank's FC1 is a column shard (§2.3, §7.1), the activation is applied
    element-wise to its own columns, and the activation is kept as bfloat16
    (reading: FC2's input has the inputs' format).  Returns bf16 bit patterns.
    """
    x = allgather(X_slices)
    return [round_to_bf16_bits(gelu(x @ _f64(w))) for w in W1_shards]


def mlp_sp(X_slices: Sequence, W1_shards: Sequence, W2_shards: Sequence, H_shards=None) -> List[np.ndarray]:
    """Output slices of the MLP block: ReduceScatter of sum_k H_k W2_k.

    FC2 is row-parallel (§2.4, §7.1): rank k multiplies its activation shard
    H_k by its row shard W2_k; the partial sums are reduced and scattered
    along the sequence (§11.3).  ``H_shards`` (bf16 bit patterns) may be given
    to evaluate FC2 on a particular set of activations.
    """
    H = mlp_sp_hidden(X_slices, W1_shards) if H_shards is None else H_shards
    return matmul_reducescatter(H, W2_shards)
