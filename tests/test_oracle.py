"""Pins for the CPU oracle: values, identities and brute force that hold independently of it.

Each pin is written so that a plausible slip in the oracle (a dropped shard,
a wrong slice index, a transposed operand, a wrong rounding rule) fails at
least one of them; ``test_pins_catch_planted_mistakes`` plants such slips in
copies of the oracle functions and checks that the pins notice.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import tpf_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bits(a):
    """bf16 bit patterns of small exact values (integers here)."""
    return O.round_to_bf16_bits(np.asarray(a, dtype=np.float64))


# ---------------------------------------------------------------------------
# Pins as functions of an oracle-like namespace, so they can be re-run on
# deliberately broken copies.
# ---------------------------------------------------------------------------


def pin_tiny_row_parallel(o):
    g = _load("tiny_tp_example.json")
    X = np.array(g["X"], float)
    A = np.array(g["A"], float)
    Xs = [_bits(X[:, 0:2]), _bits(X[:, 2:4])]
    As = [_bits(A[0:2]), _bits(A[2:4])]
    parts = o.shard_products(Xs, As)
    ok = np.array_equal(parts[0], g["row_parallel"]["Y_0"]) and \
        np.array_equal(parts[1], g["row_parallel"]["Y_1"])
    ok = ok and np.array_equal(o.matmul_allreduce(Xs, As), g["row_parallel"]["Y"])
    return ok


def pin_tiny_reducescatter(o):
    g = _load("tiny_tp_example.json")
    X = np.array(g["reducescatter"]["X"], float)
    A = np.array(g["A"], float)
    Xs = [_bits(X[:, 0:2]), _bits(X[:, 2:4])]
    As = [_bits(A[0:2]), _bits(A[2:4])]
    sl = o.matmul_reducescatter(Xs, As)
    return len(sl) == 2 and all(np.array_equal(s, e) for s, e in zip(sl, g["reducescatter"]["slices"]))


def pin_tiny_column_backward(o):
    g = _load("tiny_tp_example.json")
    A = np.array(g["A"], float)
    cb = g["column_backward"]
    dY = [_bits(cb["dY_0"]), _bits(cb["dY_1"])]
    W = [_bits(A[:, 0:3]), _bits(A[:, 3:6])]      # column shards, stored [K_in, N_shard]
    return np.array_equal(o.matmul_dx(dY, W), cb["dX"])


def pin_tiny_allgather(o):
    g = _load("tiny_tp_example.json")
    A = np.array(g["A"], float)
    sl = [_bits(s) for s in g["allgather"]["X_slices"]]
    xg, y = o.allgather_matmul(sl, _bits(A[:, 0:3]))
    return np.array_equal(xg, np.concatenate([np.array(s) for s in g["allgather"]["X_slices"]])) and \
        np.array_equal(y, g["allgather"]["Y_0"])


def pin_worked_example(o):
    g = _load("worked_example.json")
    M, N = g["Y_r"]
    ok = o.message_bytes(M, N, g["elt_bytes"]) == g["local_output_bytes"]
    cb = o.chunk_bounds(M, g["chunks"])
    ok = ok and all(r1 - r0 == g["chunk_rows"] for r0, r1 in cb)
    ok = ok and all(o.message_bytes(r1 - r0, N, g["elt_bytes"]) == g["chunk_bytes"] for r0, r1 in cb)
    t = g["timeline"]
    ok = ok and o.serial_time(t["n"], t["t_compute_ms"], t["t_comm_ms"]) == t["serial_ms"]
    ok = ok and o.pipeline_time(t["n"], t["t_compute_ms"], t["t_comm_ms"]) == t["pipeline_ms"]
    ok = ok and abs(1 - t["pipeline_ms"] / t["serial_ms"] - t["saving"]) < 1e-12
    return ok


def _rand_shards(rng, M, K, N, p, scale=1.0):
    Xs = [O.round_to_bf16_bits(rng.standard_normal((M, K)) * scale) for _ in range(p)]
    Ws = [O.round_to_bf16_bits(rng.standard_normal((K, N)) * scale) for _ in range(p)]
    return Xs, Ws


def _exact_matmul(A, B):
    """Brute-force exact product of small float matrices with rationals."""
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for t in range(K):
                s += Fraction(float(A[i, t])) * Fraction(float(B[t, j]))
            out[i][j] = s
    return out


def pin_brute_force_unsharded(o):
    """sum_k X_k W_k equals the exact unsharded X W (cnblogs §四 identity), brute force."""
    rng = np.random.default_rng(5)
    M, K, N, p = 3, 5, 4, 3
    Xs, Ws = _rand_shards(rng, M, K, N, p)
    X = np.concatenate([O.bf16_bits_to_f64(x) for x in Xs], axis=1)      # [M, p*K]
    W = np.concatenate([O.bf16_bits_to_f64(w) for w in Ws], axis=0)      # [p*K, N]
    exact = _exact_matmul(X, W)
    y = o.matmul_allreduce(Xs, Ws)
    for i in range(M):
        for j in range(N):
            e = float(exact[i][j])
            if abs(y[i, j] - e) > 1e-14 * max(1.0, abs(e)):
                return False
    # the same with one row selected
    yr = o.matmul_allreduce(Xs, Ws, rows=[2])
    return np.allclose(yr[0], y[2], rtol=0, atol=1e-14)


def pin_brute_force_dx(o):
    """dX = sum_k dY_k W_k^T equals [dY_0|..]·[W_0|..]^T (cnblogs §6.4), brute force."""
    rng = np.random.default_rng(6)
    M, Kin, Ns, p = 3, 4, 5, 2
    dY = [O.round_to_bf16_bits(rng.standard_normal((M, Ns))) for _ in range(p)]
    W = [O.round_to_bf16_bits(rng.standard_normal((Kin, Ns))) for _ in range(p)]
    dYc = np.concatenate([O.bf16_bits_to_f64(d) for d in dY], axis=1)    # [M, p*Ns]
    Wc = np.concatenate([O.bf16_bits_to_f64(w) for w in W], axis=1)      # [Kin, p*Ns]
    exact = _exact_matmul(dYc, Wc.T)
    d = o.matmul_dx(dY, W)
    return all(abs(d[i, j] - float(exact[i][j])) <= 1e-14 * max(1.0, abs(float(exact[i][j])))
               for i in range(M) for j in range(Kin))


def pin_brute_force_dx_reducescatter(o):
    """dX in the sequence-parallel layout: slice r holds rows [r*M/p, (r+1)*M/p)
    of sum_k dY_k W_k^T (cnblogs §2.7 ReduceScatter applied to the §6.4
    backward), checked row by row against the exact rational product."""
    rng = np.random.default_rng(16)
    M, Kin, Ns, p = 6, 4, 3, 3
    dY = [O.round_to_bf16_bits(rng.standard_normal((M, Ns))) for _ in range(p)]
    W = [O.round_to_bf16_bits(rng.standard_normal((Kin, Ns))) for _ in range(p)]
    dYc = np.concatenate([O.bf16_bits_to_f64(d) for d in dY], axis=1)    # [M, p*Ns]
    Wc = np.concatenate([O.bf16_bits_to_f64(w) for w in W], axis=1)      # [Kin, p*Ns]
    exact = _exact_matmul(dYc, Wc.T)
    sl = o.matmul_dx_reducescatter(dY, W)
    if len(sl) != p or any(s.shape != (M // p, Kin) for s in sl):
        return False
    return all(abs(sl[r][i, j] - float(exact[r * (M // p) + i][j])) <= 1e-14 * max(1.0, abs(float(exact[r * (M // p) + i][j])))
               for r in range(p) for i in range(M // p) for j in range(Kin))


def pin_brute_force_rowpar_dx(o):
    """Row-parallel input gradients side by side equal dY W^T with the
    unsharded W = [W_0; ...; W_{p-1}] (cnblogs §四), exact rational brute force."""
    rng = np.random.default_rng(26)
    M, Ks, N, p = 3, 2, 5, 3
    dY = O.round_to_bf16_bits(rng.standard_normal((M, N)))
    W = [O.round_to_bf16_bits(rng.standard_normal((Ks, N))) for _ in range(p)]
    Wc = np.concatenate([O.bf16_bits_to_f64(w) for w in W], axis=0)      # [p*Ks, N]
    exact = _exact_matmul(O.bf16_bits_to_f64(dY), Wc.T)                  # [M, p*Ks]
    d = o.rowpar_dx(dY, W)
    if len(d) != p or any(x.shape != (M, Ks) for x in d):
        return False
    return all(abs(d[k][i, j] - float(exact[i][k * Ks + j])) <= 1e-14 * max(1.0, abs(float(exact[i][k * Ks + j])))
               for k in range(p) for i in range(M) for j in range(Ks))


def pin_rowpar_dx_autograd(o):
    """The oracle's dX_k equals autograd's gradient of Y = sum_k X_k W_k with
    respect to X_k (float64), for loss = <G, Y>."""
    rng = np.random.default_rng(27)
    M, Ks, N, p = 4, 3, 6, 2
    W = [O.round_to_bf16_bits(rng.standard_normal((Ks, N))) for _ in range(p)]
    G = O.round_to_bf16_bits(rng.standard_normal((M, N)))
    Xt = [torch.tensor(rng.standard_normal((M, Ks)), requires_grad=True) for _ in range(p)]
    Y = sum(x @ torch.tensor(O.bf16_bits_to_f64(w)) for x, w in zip(Xt, W))
    (Y * torch.tensor(O.bf16_bits_to_f64(G))).sum().backward()
    d = o.rowpar_dx(G, W)
    return all(np.allclose(dk, x.grad.numpy(), rtol=1e-13, atol=1e-13) for dk, x in zip(d, Xt))


def pin_dx_autograd(o):
    """The oracle's dX equals autograd's gradient of the column-parallel forward.

    Forward Y_k = X A_k on every shard (cnblogs §2.3), loss = sum_k <G_k, Y_k>;
    the gradient with respect to the replicated X is what the backward must
    all-reduce (cnblogs §6.4).
    """
    rng = np.random.default_rng(7)
    M, Kin, Ns, p = 6, 10, 7, 3
    G = [O.round_to_bf16_bits(rng.standard_normal((M, Ns))) for _ in range(p)]
    A = [O.round_to_bf16_bits(rng.standard_normal((Kin, Ns))) for _ in range(p)]
    X = torch.tensor(rng.standard_normal((M, Kin)), dtype=torch.float64, requires_grad=True)
    loss = 0
    for g, a in zip(G, A):
        loss = loss + (torch.tensor(O.bf16_bits_to_f64(g)) * (X @ torch.tensor(O.bf16_bits_to_f64(a)))).sum()
    loss.backward()
    return np.allclose(o.matmul_dx(G, A), X.grad.numpy(), rtol=1e-13, atol=1e-13)


def pin_column_identity(o):
    """Gathered input times column shard k equals column block k of X A (cnblogs §三)."""
    rng = np.random.default_rng(8)
    p, Ms, K, N = 4, 3, 8, 12
    slices = [O.round_to_bf16_bits(rng.standard_normal((Ms, K))) for _ in range(p)]
    Afull = O.round_to_bf16_bits(rng.standard_normal((K, N)))
    xg, yfull = o.allgather_matmul(slices, Afull)
    exact = _exact_matmul(xg, O.bf16_bits_to_f64(Afull))
    if not all(abs(yfull[i, j] - float(exact[i][j])) < 1e-13 for i in range(p * Ms) for j in range(N)):
        return False
    # rows must follow rank order: row r*Ms + i comes from slice r
    for r in range(p):
        if not np.array_equal(xg[r * Ms:(r + 1) * Ms], O.bf16_bits_to_f64(slices[r])):
            return False
    w = N // 2
    _, y1 = o.allgather_matmul(slices, Afull[:, w:])
    return np.allclose(y1, yfull[:, w:], rtol=0, atol=1e-13)


def pin_chunked_equals_whole(o):
    rng = np.random.default_rng(9)
    Xs, Ws = _rand_shards(rng, 37, 16, 9, 2)
    whole = o.matmul_allreduce(Xs, Ws)
    for n in (1, 2, 4, 5, 37):
        if not np.allclose(o.matmul_allreduce_chunked(Xs, Ws, n), whole, rtol=0, atol=1e-12):
            return False
    return True


def pin_rs_slices(o):
    """ReduceScatter slice r is row block r of the AllReduce result (M027 §01)."""
    rng = np.random.default_rng(10)
    Xs, Ws = _rand_shards(rng, 12, 8, 5, 4)
    ar = o.matmul_allreduce(Xs, Ws)
    sl = o.matmul_reducescatter(Xs, Ws)
    return len(sl) == 4 and all(np.array_equal(sl[r], ar[3 * r:3 * (r + 1)]) for r in range(4))


def pin_chunk_bounds(o):
    ok = o.chunk_bounds(128, 4) == [(0, 32), (32, 64), (64, 96), (96, 128)]
    ok = ok and o.chunk_bounds(10, 3) == [(0, 3), (3, 6), (6, 10)]
    ok = ok and o.chunk_bounds(7, 1) == [(0, 7)]
    ok = ok and o.chunk_bounds(5, 5) == [(i, i + 1) for i in range(5)]
    return ok


def _nearest_bf16_bruteforce(x):
    """Nearest bf16 to x among all finite patterns, ties to the even pattern."""
    pats = np.arange(0, 0x7F80, dtype=np.uint32)          # non-negative finite patterns
    vals = (pats << 16).view(np.float32).astype(np.float64)
    ax = abs(x)
    d = np.abs(vals - ax)
    best = np.flatnonzero(d == d.min())
    if len(best) == 2:
        b = best[0] if pats[best[0]] % 2 == 0 else best[1]
    else:
        b = best[0]
    bits = int(pats[b])
    # beyond the largest finite value by half an ulp or more: infinity
    maxv = float(vals[-1])
    ulp_top = maxv - float(vals[-2])
    if ax >= maxv + ulp_top / 2:
        bits = 0x7F80
    return bits | (0x8000 if np.signbit(x) else 0)


def pin_round_bf16(o):
    rng = np.random.default_rng(11)
    # (a) against torch's binary32 -> bfloat16 RNE for values exact in binary32
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    edge = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -126, 2 ** -130,
                     3.0e38, 65504.0, 1.5 * 2 ** -133], dtype=np.float32)
    f = np.concatenate([f, edge])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if not np.array_equal(o.round_to_bf16_bits(f.astype(np.float64)), ref):
        return False
    # (b) brute force over all patterns for doubles that binary32 cannot hold
    xs = list(rng.standard_normal(200) * np.exp(rng.uniform(-20, 20, 200)))
    # exact ties and values just off a tie, which double rounding through binary32 gets wrong
    xs += [1.0 + 2 ** -8, 1.0 + 2 ** -8 + 2 ** -40, 1.0 + 3 * 2 ** -8 - 2 ** -40, -2.5 * 2 ** -100]
    xs += [1.0 + 2 ** -8 + 2 ** -30]      # rounds to 1.0 via binary32 (tie), up to 1+2^-7 directly
    got = o.round_to_bf16_bits(np.array(xs))
    return all(int(g) == _nearest_bf16_bruteforce(x) for g, x in zip(got, xs))


def pin_message_bf16_golden(o):
    """Hand-worked 2-byte message cases (ties, binary32 absorption, rank order)."""
    g = _load("message_bf16.json")
    for case in g["cases"]:
        Xs = [_bits(x) for x in case["X"]]
        Ws = [_bits(w) for w in case["W"]]
        if not np.array_equal(o.matmul_allreduce_msg_bf16(Xs, Ws), case["Y"]):
            return False
        if not np.array_equal(o.matmul_allreduce(Xs, Ws), case["Y_exact"]):
            return False
        if not all(np.array_equal(o.bf16_message(part), m)
                   for part, m in zip(o.shard_products(Xs, Ws), case["messages"])):
            return False
    return True


def pin_message_bf16_integer_exact(o):
    """Small integers with short shards: every local output is an integer of
    magnitude <= 2*2*8 = 32 (exact in bfloat16) and every partial sum of p <= 4
    of them is exact in binary32, so the 2-byte-message result is the exact sum."""
    rng = np.random.default_rng(5)
    for p in (1, 2, 3, 4):
        Xs = [_bits(rng.integers(-2, 3, (9, 8))) for _ in range(p)]
        Ws = [_bits(rng.integers(-2, 3, (8, 7))) for _ in range(p)]
        if not np.array_equal(o.matmul_allreduce_msg_bf16(Xs, Ws), o.matmul_allreduce(Xs, Ws)):
            return False
    return True


def pin_message_bf16_error_bound(o):
    """Against the exact sum, each element is off by at most half a bfloat16
    ulp of every local output plus the binary32 fold's rounding (p - 1
    additions, each within 2^-24 of a partial sum bounded by sum_k |m_k|)."""
    rng = np.random.default_rng(6)
    p, M, K, N = 4, 24, 40, 20
    Xs = [_bits(rng.standard_normal((M, K))) for _ in range(p)]
    Ws = [_bits(rng.standard_normal((K, N)) * 0.1) for _ in range(p)]
    parts = o.shard_products(Xs, Ws)
    got = o.matmul_allreduce_msg_bf16(Xs, Ws)
    exact = sum(parts)
    half_ulp = sum(np.ldexp(1.0, np.frexp(np.abs(q))[1] - 9) for q in parts)
    fold = (p - 1) * 2.0 ** -24 * sum(np.abs(q) for q in parts) * (1 + 2.0 ** -8)
    err = np.abs(got - exact)
    # the bound is attained only in rare corners; it must hold everywhere and not be vacuous
    return bool(np.all(err <= half_ulp + fold)) and float(err.max()) > 0.0


def pin_message_bf16_dx(o):
    """dX over 2-byte messages equals the row-parallel message sum with the
    transposed weight shards (cnblogs §6.4: dX = sum_k dY_k A_k^T)."""
    rng = np.random.default_rng(7)
    dY = [_bits(rng.standard_normal((6, 5))) for _ in range(3)]
    W = [_bits(rng.standard_normal((9, 5))) for _ in range(3)]
    Wt = [np.ascontiguousarray(w.T) for w in W]
    return np.array_equal(o.matmul_dx_msg_bf16(dY, W), o.matmul_allreduce_msg_bf16(dY, Wt))


def pin_weight_grad_golden(o):
    g = _load("tiny_tp_example.json")["weight_grad"]
    c = g["column"]
    got = o.weight_grad([_bits(c["X"])] * 2, [_bits(d) for d in c["dY"]])
    if not all(np.array_equal(a, e) for a, e in zip(got, c["dW"])):
        return False
    r = g["row"]
    got = o.weight_grad([_bits(x) for x in r["X_shards"]], [_bits(r["dY"])] * 2)
    return all(np.array_equal(a, e) for a, e in zip(got, r["dW"]))


def pin_weight_grad_autograd(o):
    """torch float64 autograd of the row- and column-parallel forwards."""
    rng = np.random.default_rng(8)
    p, M, K, N = 3, 5, 4, 6
    X = [_bits(rng.standard_normal((M, K))) for _ in range(p)]
    W = [_bits(rng.standard_normal((K, N))) for _ in range(p)]
    G = _bits(rng.standard_normal((M, N)))
    Wt = [torch.tensor(O.bf16_bits_to_f64(w), requires_grad=True) for w in W]
    Y = sum(torch.tensor(O.bf16_bits_to_f64(x)) @ w for x, w in zip(X, Wt))
    (Y * torch.tensor(O.bf16_bits_to_f64(G))).sum().backward()
    row = o.weight_grad(X, [G] * p)
    if not all(np.allclose(r, w.grad.numpy(), rtol=1e-12, atol=1e-12) for r, w in zip(row, Wt)):
        return False
    # column-parallel: Y_k = X W_k, upstream gradient G_k per shard
    Xg = _bits(rng.standard_normal((M, K)))
    Gk = [_bits(rng.standard_normal((M, N))) for _ in range(p)]
    Wt = [torch.tensor(O.bf16_bits_to_f64(w), requires_grad=True) for w in W]
    loss = sum(((torch.tensor(O.bf16_bits_to_f64(Xg)) @ w) * torch.tensor(O.bf16_bits_to_f64(g))).sum()
               for w, g in zip(Wt, Gk))
    loss.backward()
    col = o.weight_grad([Xg] * p, Gk)
    return all(np.allclose(c, w.grad.numpy(), rtol=1e-12, atol=1e-12) for c, w in zip(col, Wt))


def pin_gelu(o):
    """GeLU against the normal distribution's tabulated values (Phi(1) =
    0.841344746068543, Phi(2) = 0.977249868051821), its symmetry
    GeLU(x) - GeLU(-x) = x, the limits, and torch's erf-form GeLU."""
    g = o.gelu(np.array([0.0, 1.0, -1.0, 2.0, -2.0, 40.0, -40.0]))
    tab = [0.0, 0.841344746068543, -(1 - 0.841344746068543), 2 * 0.977249868051821,
           -2 * (1 - 0.977249868051821), 40.0, 0.0]
    if not np.allclose(g, tab, rtol=1e-14, atol=1e-15):
        return False
    x = np.random.default_rng(10).standard_normal(1000) * 3
    if not np.allclose(o.gelu(x) - o.gelu(-x), x, rtol=0, atol=1e-14):
        return False
    ref = torch.nn.functional.gelu(torch.from_numpy(x)).numpy()   # float64, erf form
    return np.allclose(o.gelu(x), ref, rtol=1e-14, atol=1e-15)


def pin_mlp_sp_unsharded(o):
    """The sharded MLP block equals the unsharded one (cnblogs §7.1: FC1 split
    by columns and FC2 by rows needs no communication in between): with the
    activation kept in float64, sum_k GeLU(X W1_k) W2_k == GeLU(X [W1_0|..]) [W2_0;..].
    The oracle's bf16 activation is compared in the same way through the
    same rounding applied to the unsharded activation."""
    rng = np.random.default_rng(12)
    p, s, h, f = 2, 8, 6, 4
    Xs = [_bits(rng.standard_normal((s // p, h))) for _ in range(p)]
    W1 = [_bits(rng.standard_normal((h, f)) * 0.5) for _ in range(p)]
    W2 = [_bits(rng.standard_normal((f, h)) * 0.5) for _ in range(p)]
    x = np.concatenate([O.bf16_bits_to_f64(a) for a in Xs])
    w1 = np.concatenate([O.bf16_bits_to_f64(w) for w in W1], axis=1)
    w2 = np.concatenate([O.bf16_bits_to_f64(w) for w in W2], axis=0)
    hid = O.bf16_bits_to_f64(O.round_to_bf16_bits(0.5 * (x @ w1) * (1 + np.vectorize(__import__("math").erf)(
        (x @ w1) / np.sqrt(2.0)))))
    y = hid @ w2
    got_h = o.mlp_sp_hidden(Xs, W1)
    if not np.array_equal(np.concatenate(got_h, axis=1), O.round_to_bf16_bits(hid)):
        return False
    sl = o.mlp_sp(Xs, W1, W2)
    return len(sl) == p and np.allclose(np.concatenate(sl), y, rtol=1e-13, atol=1e-13)


PINS = [pin_tiny_row_parallel, pin_tiny_reducescatter, pin_tiny_column_backward, pin_tiny_allgather,
        pin_worked_example, pin_brute_force_unsharded, pin_brute_force_dx, pin_brute_force_dx_reducescatter,
        pin_dx_autograd, pin_brute_force_rowpar_dx, pin_rowpar_dx_autograd,
        pin_column_identity, pin_chunked_equals_whole, pin_rs_slices, pin_chunk_bounds,
        pin_round_bf16, pin_message_bf16_golden, pin_message_bf16_integer_exact,
        pin_message_bf16_error_bound, pin_message_bf16_dx, pin_weight_grad_golden, pin_weight_grad_autograd,
        pin_gelu, pin_mlp_sp_unsharded]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    assert pin(O)


def test_pipeline_exercise_closed_form():
    # M027 §07 exercise: compute 1 ms, communication 5 ms, four chunks -> the
    # communication-dominated ceiling 1 + 3*5 + 5 = 21 ms against 24 ms serial.
    assert O.pipeline_time(4, 1, 5) == 21
    assert O.serial_time(4, 1, 5) == 24
    # with one chunk there is nothing to overlap
    assert O.pipeline_time(1, 3, 2) == O.serial_time(1, 3, 2)


def test_bf16_bits_roundtrip():
    pats = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(O.round_to_bf16_bits(O.bf16_bits_to_f64(pats)), pats)
    assert np.array_equal(O.round_to_bf16_bits(O.bf16_bits_to_f64(pats | 0x8000)), pats | 0x8000)


# ---------------------------------------------------------------------------
# Planted mistakes: each broken copy must fail at least one pin.
# ---------------------------------------------------------------------------


class _Mutant:
    def __init__(self, **over):
        self.__dict__.update({k: getattr(O, k) for k in dir(O) if not k.startswith("__")})
        self.__dict__.update(over)


def _m_dropped_shard():
    def shard_products(Xs, Ws, rows=None):
        return O.shard_products(Xs[1:], Ws[1:], rows) + [0 * O.shard_products(Xs[:1], Ws[:1], rows)[0]]

    m = _Mutant(shard_products=shard_products)

    def matmul_allreduce(Xs, Ws, rows=None):
        parts = shard_products(Xs, Ws, rows)
        y = np.zeros_like(parts[0])
        for q in parts:
            y = y + q
        return y
    m.matmul_allreduce = matmul_allreduce
    m.matmul_reducescatter = lambda Xs, Ws: O.scatter_rows(matmul_allreduce(Xs, Ws), len(Xs))
    return m


def _m_sign():
    def matmul_allreduce(Xs, Ws, rows=None):
        parts = O.shard_products(Xs, Ws, rows)
        return parts[0] - sum(parts[1:])
    return _Mutant(matmul_allreduce=matmul_allreduce)


def _m_dx_untransposed():
    def matmul_dx(dY, W, rows=None):
        out = None
        for d, w in zip(dY, W):
            wf = O.bf16_bits_to_f64(w)
            # a transposed operand: contract dY's columns with W's rows (reshape to fit)
            t = O.bf16_bits_to_f64(d) @ wf.reshape(wf.shape[1], wf.shape[0])
            out = t if out is None else out + t
        return out
    return _Mutant(matmul_dx=matmul_dx)


def _m_rowpar_dx_untransposed():
    def rowpar_dx(dY, W):
        d = O.bf16_bits_to_f64(dY)
        return [d @ O.bf16_bits_to_f64(w).reshape(w.shape[1], w.shape[0]) for w in W]
    return _Mutant(rowpar_dx=rowpar_dx)


def _m_slices_reversed():
    def scatter_rows(Y, p):
        return O.scatter_rows(Y, p)[::-1]
    m = _Mutant(scatter_rows=scatter_rows)
    m.matmul_reducescatter = lambda Xs, Ws: scatter_rows(O.matmul_allreduce(Xs, Ws), len(Xs))
    m.matmul_dx_reducescatter = lambda dY, W: scatter_rows(O.matmul_dx(dY, W), len(dY))
    return m


def _m_gather_reversed():
    def allgather_matmul(sl, W):
        return O.allgather_matmul(list(sl)[::-1], W)
    return _Mutant(allgather_matmul=allgather_matmul)


def _m_round_truncate():
    def round_to_bf16_bits(x):
        x = np.asarray(x, np.float64).astype(np.float32)
        return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return _Mutant(round_to_bf16_bits=round_to_bf16_bits)


def _m_round_via_f32():
    def round_to_bf16_bits(x):
        f = np.asarray(x, np.float64).astype(np.float32)
        return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return _Mutant(round_to_bf16_bits=round_to_bf16_bits)


def _m_chunk_lastshort():
    def chunk_bounds(M, n):
        base = -(-M // n)
        return [(c * base, min(M, (c + 1) * base)) for c in range(n)]
    return _Mutant(chunk_bounds=chunk_bounds)


def _m_pipeline_serial():
    # forgetting the pipeline fill and drain
    return _Mutant(pipeline_time=lambda n, tc, tm: n * max(tc, tm))


def _msg_mutant(message=None, fold=None):
    """Copies of the 2-byte-message functions with one step replaced."""
    message = message or O.bf16_message
    fold = fold or O.sum_messages_f32

    def matmul_allreduce_msg_bf16(Xs, Ws, rows=None):
        return fold([message(q) for q in O.shard_products(Xs, Ws, rows)])

    def matmul_dx_msg_bf16(dY, W, rows=None):
        return fold([message(O.bf16_bits_to_f64(d) @ O.bf16_bits_to_f64(w).T) for d, w in zip(dY, W)])
    return _Mutant(bf16_message=message, sum_messages_f32=fold, matmul_allreduce_msg_bf16=matmul_allreduce_msg_bf16,
                   matmul_dx_msg_bf16=matmul_dx_msg_bf16)


def _m_message_truncated():
    # round toward zero instead of to nearest even
    return _msg_mutant(message=lambda q: np.trunc(np.ldexp(q, 7 - np.frexp(q)[1] + 1)) *
                       np.ldexp(1.0, np.frexp(q)[1] - 8))


def _m_message_unrounded():
    # the message kept in binary32 (no 2-byte rounding)
    return _msg_mutant(message=lambda q: np.asarray(q, np.float64).astype(np.float32).astype(np.float64))


def _m_message_fold_f64():
    # the sum carried in float64 instead of binary32
    return _msg_mutant(fold=lambda ms: sum(np.asarray(m, np.float64) for m in ms))


def _m_message_fold_reversed():
    return _msg_mutant(fold=lambda ms: O.sum_messages_f32(list(ms)[::-1]))


def _m_weight_grad_swapped():
    # the operands' roles swapped: B_k^T A_k (the transposed gradient)
    return _Mutant(weight_grad=lambda A, B: [O.bf16_bits_to_f64(b).T @ O.bf16_bits_to_f64(a) for a, b in zip(A, B)])


def _m_weight_grad_shard_shift():
    # shard k paired with the next shard's B
    return _Mutant(weight_grad=lambda A, B: O.weight_grad(A, list(B[1:]) + list(B[:1])))


def _m_gelu_tanh():
    # the tanh approximation instead of the erf form
    def gelu(x):
        x = np.asarray(x, np.float64)
        return 0.5 * x * (1 + np.tanh(np.sqrt(2 / np.pi) * (x + 0.044715 * x ** 3)))
    m = _Mutant(gelu=gelu)
    m.mlp_sp_hidden = lambda Xs, W1: [O.round_to_bf16_bits(gelu(O.allgather(Xs) @ O.bf16_bits_to_f64(w))) for w in W1]
    m.mlp_sp = lambda Xs, W1, W2, H=None: O.matmul_reducescatter(m.mlp_sp_hidden(Xs, W1) if H is None else H, W2)
    return m


def _m_mlp_w2_transposed_shards():
    # FC2 applied with the shards in reverse order
    m = _Mutant()
    m.mlp_sp = lambda Xs, W1, W2, H=None: O.matmul_reducescatter(O.mlp_sp_hidden(Xs, W1), list(W2)[::-1])
    return m


MUTANTS = [_m_dropped_shard, _m_sign, _m_dx_untransposed, _m_rowpar_dx_untransposed, _m_slices_reversed, _m_gather_reversed,
           _m_round_truncate, _m_round_via_f32, _m_chunk_lastshort, _m_pipeline_serial,
           _m_message_truncated, _m_message_unrounded, _m_message_fold_f64, _m_message_fold_reversed,
           _m_weight_grad_swapped, _m_weight_grad_shard_shift, _m_gelu_tanh, _m_mlp_w2_transposed_shards]


@pytest.mark.parametrize("mut", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_pins_catch_planted_mistakes(mut):
    m = mut()
    failed = []
    for pin in PINS:
        try:
            ok = pin(m)
        except Exception:
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"no pin noticed the planted mistake {mut.__name__}"
