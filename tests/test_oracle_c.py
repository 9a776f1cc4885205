"""Pins for the plain C oracle (oracle/tpf_oracle.c).

The C oracle computes the same definitions as the numpy oracle with its own
loops.  It is pinned the same way, to things other than itself: the
hand-worked tiny examples and exact rational brute force of the pin suite in
test_oracle.py (run here through an adapter that calls only the C library
for every arithmetic step), the column identity, ReduceScatter slices against
AllReduce rows, and the bf16 rounding against torch's binary32 conversion and
a brute-force nearest search.  Mistakes planted in edited copies of the C
source (compiled on the fly) must each fail some pin.  A cross-check against
the numpy oracle on random inputs closes the loop; it is a cross-check, not
a pin.  Host-only.
"""
import os
import re
import shutil
import tempfile

import numpy as np
import pytest

from oracle import build as B
from oracle import c_oracle as C
from oracle import tpf_oracle as O
from tests import test_oracle as T


class _Adapter:
    """The oracle interface the pins expect, every arithmetic step done by the
    C library (the numpy side only reshapes and converts bit patterns)."""

    def __init__(self, c: C.COracle):
        self.c = c

    def shard_products(self, X, W, rows=None):
        return [self.c.matmul_allreduce([x], [w], rows) for x, w in zip(X, W)]

    def matmul_allreduce(self, X, W, rows=None):
        return self.c.matmul_allreduce(X, W, rows)

    def matmul_reducescatter(self, X, W):
        return self.c.matmul_reducescatter(X, W)

    def matmul_dx(self, dY, W, rows=None):
        return self.c.matmul_dx(dY, W, rows)

    def matmul_dx_reducescatter(self, dY, W):
        p, M = len(dY), dY[0].shape[0]
        per = M // p
        return [self.c.matmul_dx(dY, W, rows=np.arange(r * per, (r + 1) * per)) for r in range(p)]

    def allgather_matmul(self, slices, W):
        xg, y = self.c.allgather_matmul(slices, W)
        return O.bf16_bits_to_f64(xg), y

    def round_to_bf16_bits(self, x):
        return self.c.round_to_bf16_bits(x)


# Pins of test_oracle.py that exercise only what the C oracle computes.
C_PINS = [T.pin_tiny_row_parallel, T.pin_tiny_reducescatter, T.pin_tiny_column_backward, T.pin_tiny_allgather,
          T.pin_brute_force_unsharded, T.pin_brute_force_dx, T.pin_brute_force_dx_reducescatter,
          T.pin_column_identity, T.pin_rs_slices, T.pin_round_bf16]


def pin_integer_exact(o):
    """Integer operands in {-2..2}: every partial sum is an integer below
    2^24, so the result equals the exact integer product, computed here with
    Python integers from the unsharded operands (cnblogs §四: the sharded sum
    is the unsharded product)."""
    rng = np.random.default_rng(21)
    p, M, K, N = 3, 5, 7, 6
    Xi = [rng.integers(-2, 3, (M, K)) for _ in range(p)]
    Wi = [rng.integers(-2, 3, (K, N)) for _ in range(p)]
    X = np.concatenate(Xi, axis=1).tolist()
    W = np.concatenate(Wi, axis=0).tolist()
    exact = [[sum(X[i][t] * W[t][j] for t in range(p * K)) for j in range(N)] for i in range(M)]
    y = o.matmul_allreduce([O.round_to_bf16_bits(x) for x in Xi], [O.round_to_bf16_bits(w) for w in Wi])
    return np.array_equal(y, np.array(exact, dtype=np.float64))


def pin_selected_rows(o):
    """A request for a subset of rows returns exactly those rows, in order."""
    rng = np.random.default_rng(22)
    X = [O.round_to_bf16_bits(rng.standard_normal((9, 8))) for _ in range(2)]
    W = [O.round_to_bf16_bits(rng.standard_normal((8, 8))) for _ in range(2)]
    full = o.matmul_allreduce(X, W)
    rows = [7, 0, 3]
    dY = [O.round_to_bf16_bits(rng.standard_normal((9, 8))) for _ in range(2)]
    return np.array_equal(o.matmul_allreduce(X, W, rows=rows), full[rows]) and \
        np.array_equal(o.matmul_dx(dY, W, rows=rows), o.matmul_dx(dY, W)[rows])


ALL_PINS = C_PINS + [pin_integer_exact, pin_selected_rows]


@pytest.fixture(scope="module")
def c_oracle():
    B.build()
    return _Adapter(C.COracle())


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_c_oracle_pin(c_oracle, pin):
    assert pin(c_oracle)


def test_c_oracle_agrees_with_numpy_oracle(c_oracle):
    """Cross-check (not a pin): the two oracles on random bf16 inputs of
    several tiles' size, including ragged shapes."""
    rng = np.random.default_rng(3)
    c = c_oracle.c
    for p, M, K, N in [(2, 37, 40, 24), (4, 64, 96, 40), (3, 5, 8, 16)]:
        X = [O.round_to_bf16_bits(rng.standard_normal((M, K))) for _ in range(p)]
        W = [O.round_to_bf16_bits(rng.standard_normal((K, N)) * 0.1) for _ in range(p)]
        a, b = c.matmul_allreduce(X, W), O.matmul_allreduce(X, W)
        assert np.allclose(a, b, rtol=1e-13, atol=1e-13)
        d = [O.round_to_bf16_bits(rng.standard_normal((M, N))) for _ in range(p)]
        Wd = [O.round_to_bf16_bits(rng.standard_normal((K, N)) * 0.1) for _ in range(p)]
        assert np.allclose(c.matmul_dx(d, Wd), O.matmul_dx(d, Wd), rtol=1e-13, atol=1e-13)
    v = rng.standard_normal(50000) * 10.0 ** rng.integers(-44, 39, 50000)
    assert np.array_equal(c.round_to_bf16_bits(v), O.round_to_bf16_bits(v))


# Mistakes planted in copies of the C source: (name, regex, replacement).
PLANTS = [
    ("dropped_shard", r"for \(int k = 0; k < p; \+\+k\) \{\n      const uint16_t\* x = X\[k\]",
     "for (int k = 0; k < p - 1; ++k) {\n      const uint16_t* x = X[k]"),
    ("sign", r"acc\[j\] \+= a \* bf16\(w\[j\]\);\n      \}\n    \}\n  \}\n\}\n\n/\*\n \* Column",
     "acc[j] -= a * bf16(w[j]);\n      }\n    }\n  }\n}\n\n/*\n * Column"),
    ("dx_untransposed", r"s \+= bf16\(g\[t\]\) \* bf16\(w\[t\]\);",
     "s += bf16(g[t]) * bf16(W[k][t * K_in + j]);"),
    ("gather_reversed", r"slices\[i / per\]", "slices[p - 1 - i / per]"),
    ("rows_ignored", r"return rows \? rows\[r\] : r;", "return r;"),
    ("round_truncate", r"nearbyint\(ldexp\(v, -q\)\)", "trunc(ldexp(v, -q))"),
    ("round_via_f32", r"nearbyint\(ldexp\(v, -q\)\)", "nearbyint(ldexp((double)(float)v, -q))"),
    ("dx_shard_twice", r"const uint16_t\* g = dY\[k\] \+ i \* Ns;", "const uint16_t* g = dY[0] + i * Ns;"),
]


@pytest.mark.parametrize("name,pattern,repl", PLANTS, ids=[p[0] for p in PLANTS])
def test_c_pins_catch_planted_mistakes(name, pattern, repl):
    if shutil.which("gcc") is None and shutil.which("cc") is None:
        pytest.skip("no C compiler")
    src = open(B.SRC).read()
    bad, n = re.subn(pattern, repl, src, count=1)
    assert n == 1, f"plant {name} did not apply"
    d = tempfile.mkdtemp(prefix="tpfo_plant_")
    try:
        path = os.path.join(d, f"tpf_oracle_{name}.c")
        with open(path, "w") as f:
            f.write(bad)
        lib = B.build_source(path, os.path.join(d, f"lib_{name}.so"))
        o = _Adapter(C.COracle(lib))
        failed = []
        for pin in ALL_PINS:
            try:
                ok = pin(o)
            except Exception:
                ok = False
            if not ok:
                failed.append(pin.__name__)
        assert failed, f"no pin noticed the planted mistake {name}"
    finally:
        shutil.rmtree(d, ignore_errors=True)
