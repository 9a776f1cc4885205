"""ctypes loader of the plain C oracle (oracle/tpf_oracle.c).

TEST INFRASTRUCTURE, like the rest of oracle/: only the tests, the smoke
check and the benchmark's CPU-baseline leg use it.  Argument marshalling
only; every value is computed by the C loops.  Inputs are bfloat16 bit
patterns (numpy uint16), outputs float64 (or uint16 bit patterns).
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libtpf_oracle.so")

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SIGS = {
    "tpfo_threads": (_I, []),
    "tpfo_matmul_allreduce": (None, [_I, _I64, _I64, _I64, _P, _P, _P, _I64, _P]),
    "tpfo_matmul_dx": (None, [_I, _I64, _I64, _I64, _P, _P, _P, _I64, _P]),
    "tpfo_allgather_matmul": (None, [_I, _I64, _I64, _I64, _P, _P, _P, _I64, _P, _P]),
    "tpfo_round_bf16": (None, [_P, _I64, _P]),
}

_libs = {}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (building first if needed) the oracle library at `path`."""
    lib = _libs.get(path)
    if lib is not None:
        return lib
    if not os.path.exists(path):
        if path != LIB_PATH:
            raise RuntimeError(f"{path} is missing")
        from oracle import build as _b
        _b.build()
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _libs[path] = lib
    return lib


class COracle:
    """The oracle's operations, bound to one built library (the default one,
    or a test's deliberately broken copy)."""

    def __init__(self, path: str = LIB_PATH):
        self.lib = load(path)

    def threads(self) -> int:
        return int(self.lib.tpfo_threads())

    @staticmethod
    def _u16(a) -> np.ndarray:
        a = np.ascontiguousarray(a)
        if a.dtype != np.uint16:
            raise TypeError("inputs are bfloat16 bit patterns (uint16)")
        return a

    @staticmethod
    def _ptrs(arrs) -> ctypes.Array:
        ptrs = (ctypes.c_void_p * len(arrs))()
        for i, a in enumerate(arrs):
            ptrs[i] = a.ctypes.data
        return ptrs

    @staticmethod
    def _rows(rows, M):
        if rows is None:
            return None, M
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if r.size and (r.min() < 0 or r.max() >= M):
            raise IndexError("row out of range")
        return r, r.size

    def matmul_allreduce(self, X: Sequence, W: Sequence, rows=None) -> np.ndarray:
        """Y = sum_k X_k W_k (all rows, or the requested ones), float64."""
        X = [self._u16(x) for x in X]
        W = [self._u16(w) for w in W]
        p = len(X)
        if p < 1 or len(W) != p:
            raise ValueError("need one X and one W per shard")
        M, K = X[0].shape
        N = W[0].shape[1]
        for x, w in zip(X, W):
            if x.shape != (M, K) or w.shape != (K, N):
                raise ValueError("shard shapes differ")
        r, n = self._rows(rows, M)
        Y = np.empty((n, N), dtype=np.float64)
        self.lib.tpfo_matmul_allreduce(p, M, N, K, self._ptrs(X), self._ptrs(W),
                                       r.ctypes.data if r is not None else None, n, Y.ctypes.data)
        return Y

    def matmul_reducescatter(self, X: Sequence, W: Sequence) -> List[np.ndarray]:
        """Slice s = rows [s*M/p, (s+1)*M/p) of sum_k X_k W_k."""
        p = len(X)
        M = X[0].shape[0]
        if M % p:
            raise ValueError("M must be divisible by p")
        per = M // p
        return [self.matmul_allreduce(X, W, rows=np.arange(s * per, (s + 1) * per)) for s in range(p)]

    def matmul_dx(self, dY: Sequence, W: Sequence, rows=None) -> np.ndarray:
        """dX = sum_k dY_k W_k^T, float64 (W_k [K_in, Ns] read transposed)."""
        dY = [self._u16(d) for d in dY]
        W = [self._u16(w) for w in W]
        p = len(dY)
        if p < 1 or len(W) != p:
            raise ValueError("need one dY and one W per shard")
        M, Ns = dY[0].shape
        Kin = W[0].shape[0]
        for d, w in zip(dY, W):
            if d.shape != (M, Ns) or w.shape != (Kin, Ns):
                raise ValueError("shard shapes differ")
        r, n = self._rows(rows, M)
        out = np.empty((n, Kin), dtype=np.float64)
        self.lib.tpfo_matmul_dx(p, M, Kin, Ns, self._ptrs(dY), self._ptrs(W),
                                r.ctypes.data if r is not None else None, n, out.ctypes.data)
        return out

    def allgather_matmul(self, slices: Sequence, W, rows=None):
        """(X_gathered rows as bit patterns, X_gathered W rows in float64)."""
        S = [self._u16(s) for s in slices]
        W = self._u16(W)
        p = len(S)
        per, K = S[0].shape
        N = W.shape[1]
        if W.shape[0] != K or any(s.shape != (per, K) for s in S):
            raise ValueError("slice or weight shapes differ")
        M = per * p
        r, n = self._rows(rows, M)
        xg = np.empty((n, K), dtype=np.uint16)
        Y = np.empty((n, N), dtype=np.float64)
        self.lib.tpfo_allgather_matmul(p, M, N, K, self._ptrs(S), W.ctypes.data,
                                       r.ctypes.data if r is not None else None, n, xg.ctypes.data, Y.ctypes.data)
        return xg, Y

    def round_to_bf16_bits(self, x) -> np.ndarray:
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.tpfo_round_bf16(x.ctypes.data, x.size, out.ctypes.data)
        return out


_default: Optional[COracle] = None


def default() -> COracle:
    global _default
    if _default is None:
        _default = COracle()
    return _default
