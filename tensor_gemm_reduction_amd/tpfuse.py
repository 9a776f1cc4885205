"""Python binding of libtpfuse (ctypes).

Argument marshalling only: every step of the fused path runs in the HIP
kernels of ``libtpfuse.so``.  PyTorch supplies device memory (tensors) and
the stream (``torch.cuda.current_stream()``).  If the library is not built
the import of a call fails loudly; there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libtpfuse.so")

# Status codes, dtypes, schedulers, semantics and op ids (include/tpfuse.h).
OK = 0
ERR_INVALID_ARG, ERR_SHAPE, ERR_ALIGNMENT, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_HIP, ERR_TIMEOUT = range(-1, -8, -1)
BF16, F32 = 0, 1
(SCHED_AUTO, SCHED_PERSISTENT, SCHED_TWO_STREAM, SCHED_UNFUSED, SCHED_GEMM_ONLY, SCHED_REDUCE_ONLY, SCHED_TILE,
 SCHED_FOLD, SCHED_STATIONARY) = range(9)
ALLREDUCE, REDUCESCATTER = 0, 1
OP_MATMUL_ALLREDUCE, OP_MATMUL_REDUCESCATTER, OP_ALLGATHER_MATMUL, OP_MATMUL_DX, OP_MLP_SP = range(5)
MAX_SHARDS = 16
MAX_CHUNKS = 64
NOALLOC_SCRATCH_BYTES = 64 << 20

SCHEDS = {"auto": SCHED_AUTO, "persistent": SCHED_PERSISTENT, "two_stream": SCHED_TWO_STREAM,
          "unfused": SCHED_UNFUSED, "gemm_only": SCHED_GEMM_ONLY, "reduce_only": SCHED_REDUCE_ONLY,
          "tile": SCHED_TILE, "fold": SCHED_FOLD, "stationary": SCHED_STATIONARY}

_VP = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); the set of exported functions of include/tpfuse.h
SIGNATURES = {
    "tpf_create": (_I, [ctypes.POINTER(_VP), _I]),
    "tpf_destroy": (_I, [_VP]),
    "tpf_workspace_size": (_SZ, [_I, _I, _I64, _I64, _I64, _I, _I]),
    "tpf_matmul_allreduce": (_I, [_VP, _I, _I64, _I64, _I64, _PP, _PP, _VP, _I, _I, _I, _VP, _SZ, _VP]),
    "tpf_matmul_allreduce_noalloc": (_I, [_VP, _I, _I64, _I64, _I64, _PP, _PP, _VP, _I, _I, _I, _VP]),
    "tpf_matmul_reducescatter": (_I, [_VP, _I, _I64, _I64, _I64, _PP, _PP, _PP, _I, _I, _I, _VP, _SZ, _VP]),
    "tpf_allgather_matmul": (_I, [_VP, _I, _I64, _I64, _I64, _PP, _VP, _VP, _VP, _I, _I, _I, _VP, _SZ, _VP]),
    "tpf_matmul_dx": (_I, [_VP, _I, _I, _I64, _I64, _I64, _PP, _PP, _PP, _I, _I, _I, _VP, _SZ, _VP]),
    "tpf_weight_grad": (_I, [_VP, _I, _I64, _I64, _I64, _PP, _PP, _PP, _I, _VP]),
    "tpf_mlp_sp": (_I, [_VP, _I, _I64, _I64, _I64, _PP, _PP, _PP, _VP, _PP, _PP, _I, _I, _I, _VP, _SZ, _VP]),
    "tpf_sync_status": (_I, [_VP, _VP]),
    "tpf_debug_set_wait": (_I, [_VP, _I64, _I]),
    "tpf_debug_set_delay": (_I, [_VP, ctypes.c_uint32, _I, _I]),
    "tpf_debug_set_timeline": (_I, [_VP, _VP, _I]),
    "tpf_debug_set_kernel_timing": (_I, [_VP, _I]),
    "tpf_debug_kernel_times": (_I, [_VP, ctypes.POINTER(ctypes.c_float), _I]),
    "tpf_debug_last_sched": (_I, [_VP]),
    "tpf_rowpar_dx": (_I, [_VP, _I, _I64, _I64, _I64, _VP, _VP, _VP, _I, _VP]),
    "tpf_status_string": (ctypes.c_char_p, [_I]),
    "tpf_last_error": (ctypes.c_char_p, []),
    "tpf_version": (_I, []),
}

_lib: Optional[ctypes.CDLL] = None


class TpfError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libtpfuse error {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load the in-tree libtpfuse.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m tensor_gemm_reduction_amd.build`")
    lib = ctypes.CDLL(LIB_PATH, mode=ctypes.RTLD_GLOBAL)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(code: int) -> None:
    if code != OK:
        msg = load().tpf_last_error().decode(errors="replace")
        raise TpfError(code, msg)


def ptr_array(ptrs: Sequence[int]):
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float32:
        return F32
    raise ValueError(f"output dtype must be bfloat16 or float32, got {dt}")


MSG_BF16 = 0x100           # TPF_MSG_BF16: shard partials ("messages") kept as bf16
MESSAGES = {"fp32": 0, "bf16": MSG_BF16}


def _sched(s, message: str = "fp32") -> int:
    return (SCHEDS[s] if isinstance(s, str) else int(s)) | MESSAGES[message]


def _stream_ptr(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _on(stream):
    """Allocation context for buffers the library writes on `stream`.

    torch's caching allocator ties a block to the stream that was current
    when it was allocated and may hand it out again as soon as the tensor is
    freed, ordered only against that stream.  Buffers the binding allocates
    for a call (outputs, workspace) are therefore allocated with the call's
    stream current, so a freed workspace cannot be reused while the library's
    kernels on that stream still write it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


class Handle:
    """A libtpfuse handle bound to one device (owns a side stream, events, counters)."""

    def __init__(self, device: int = 0):
        lib = load()
        h = ctypes.c_void_p()
        check(lib.tpf_create(ctypes.byref(h), int(device)))
        self._h = h
        self.device = device

    @property
    def ptr(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value:
            load().tpf_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def sync_status(self, stream=None) -> int:
        return load().tpf_sync_status(self._h, _stream_ptr(stream))

    def debug_set_wait(self, spins: int, unreachable: bool) -> None:
        check(load().tpf_debug_set_wait(self._h, int(spins), 1 if unreachable else 0))

    def set_delay(self, seed: int, period: int, sleeps: int) -> None:
        """Perturb producer timing (a seeded subset of tasks sleeps before
        publishing); period = 0 turns it off."""
        check(load().tpf_debug_set_delay(self._h, int(seed) & 0xFFFFFFFF, int(period), int(sleeps)))

    def set_timeline(self, events: Optional[torch.Tensor]) -> None:
        """Record persistent-kernel task events into `events` (uint8 device tensor, 32 B per event)."""
        if events is None:
            check(load().tpf_debug_set_timeline(self._h, None, 0))
        else:
            check(load().tpf_debug_set_timeline(self._h, events.data_ptr(), events.numel() // 32))

    def set_kernel_timing(self, enable: bool) -> None:
        """Record timing events around each later call's dominant kernel launch."""
        check(load().tpf_debug_set_kernel_timing(self._h, 1 if enable else 0))

    def last_sched(self) -> str:
        """Name of the scheduler the last reducing or AllGather call on this
        handle ran (AUTO resolved), or "" before the first."""
        v = load().tpf_debug_last_sched(self._h)
        if v < -1:
            check(v)
        names = {code: name for name, code in SCHEDS.items()}
        return names.get(v, "")

    def kernel_times(self, max_records: int = 256) -> List[float]:
        """Durations (ms) of the recorded launches, oldest first; clears the record."""
        buf = (ctypes.c_float * max_records)()
        n = load().tpf_debug_kernel_times(self._h, buf, max_records)
        if n < 0:
            check(n)
        return [float(buf[i]) for i in range(n)]


TIMELINE_DTYPE = [("ticket", "<u4"), ("kind", "<u2"), ("chunk", "<u2"), ("block", "<u2"), ("xcd", "<u2"),
                  ("mid", "<u4"), ("t_start", "<u8"), ("t_end", "<u8")]


def timeline_events(events: torch.Tensor, count: int):
    """Decode the first `count` timeline records into a numpy structured array."""
    import numpy as np
    raw = events[: count * 32].cpu().numpy()
    return raw.view(np.dtype(TIMELINE_DTYPE))


_default_handles = {}


def default_handle(device: Optional[int] = None, stream=None) -> Handle:
    """The binding's handle for (device, stream).

    A handle runs one call at a time (its persistent and tile schedulers keep
    work-queue and readiness counters in the handle), and calls on different
    streams may run at the same time, so every stream gets its own default
    handle."""
    dev = torch.cuda.current_device() if device is None else device
    key = (int(dev), _stream_ptr(stream) if stream is not None else _stream_ptr(torch.cuda.current_stream(dev)))
    h = _default_handles.get(key)
    if h is None:
        h = Handle(dev)
        _default_handles[key] = h
    return h


OUT_DTYPES = (torch.bfloat16, torch.float32)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check(name: str, ts, shape, dtypes=(torch.bfloat16,), device=None) -> torch.device:
    """Refuse, before any library call, tensors the library cannot be handed.

    The library reads and writes through raw device pointers whose extents it
    derives from the shape arguments alone, so a tensor on the host, on
    another device, of another shape or strided would be accessed out of
    bounds on the GPU.  Every tensor in `ts` must be a contiguous GPU tensor
    on `device` (default: the first one's), of shape `shape` and one of
    `dtypes`.  Returns the device."""
    _need(len(ts) >= 1, f"{name}: no tensors given")
    dev = device if device is not None else getattr(ts[0], "device", None)
    shape = tuple(shape)
    ok = getattr(dev, "type", None) == "cuda"
    for t in ts:        # one combined test per tensor; the message is built only on failure
        if not (ok and isinstance(t, torch.Tensor) and t.device == dev and t.dtype in dtypes
                and t.shape == shape and t.is_contiguous()):
            ok = False
            break
    if not ok:
        for i, t in enumerate(ts):
            lab = f"{name}[{i}]" if len(ts) > 1 else name
            _need(isinstance(t, torch.Tensor), f"{lab} is not a tensor")
            _need(t.device.type == "cuda", f"{lab} is on {t.device}, not on a GPU")
            _need(t.device == dev, f"{lab} is on {t.device}, expected {dev}")
            _need(t.dtype in dtypes, f"{lab} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
            _need(tuple(t.shape) == shape, f"{lab} has shape {tuple(t.shape)}, expected {shape}")
            _need(t.is_contiguous(), f"{lab} is not contiguous")
        _need(False, f"{name}: the device {dev} is not a GPU")
    return dev


def _check_shards(name: str, ts, p: int) -> None:
    _need(len(ts) == p, f"{name}: {len(ts)} tensors given, expected one per shard ({p})")


def _check_ws(ws, dev) -> None:
    if ws is not None:
        _check("ws", [ws], tuple(ws.shape), (ws.dtype,), dev)


def _handle(handle, dev, stream=None) -> "Handle":
    h = handle or default_handle(dev.index, stream)
    _need(h.device == dev.index, f"handle is bound to device {h.device}, tensors are on {dev}")
    return h


def workspace_size(op: int, p: int, M: int, N: int, K: int, n_chunks: int = 1, sched=SCHED_AUTO,
                   message: str = "fp32") -> int:
    return int(load().tpf_workspace_size(op, p, M, N, K, n_chunks, _sched(sched, message)))


def _ws(op, p, M, N, K, n_chunks, sched, ws, device, message="fp32", stream=None):
    need = workspace_size(op, p, M, N, K, n_chunks, sched, message)
    if need == 0:
        return ws, 0 if ws is None else ws.numel() * ws.element_size()
    if ws is None:
        with _on(stream):
            ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def matmul_allreduce(X: List[torch.Tensor], W: List[torch.Tensor], out_dtype=torch.bfloat16, n_chunks: int = 1,
                     sched="auto", Y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                     handle: Optional[Handle] = None, stream=None, message: str = "fp32") -> torch.Tensor:
    """Y = sum_k X[k] @ W[k] (row-parallel Linear, AllReduce layout)."""
    p = len(X)
    _need(p >= 1, "X: no shards given")
    M, K = X[0].shape
    N = W[0].shape[1]
    _check_shards("W", W, p)
    dev = _check("X", X, (M, K))
    _check("W", W, (K, N), device=dev)
    if Y is None:
        with _on(stream):
            Y = torch.empty((M, N), dtype=out_dtype, device=dev)
    _check("Y", [Y], (M, N), OUT_DTYPES, dev)
    _check_ws(ws, dev)
    h = _handle(handle, dev, stream)
    ws, ws_bytes = _ws(OP_MATMUL_ALLREDUCE, p, M, N, K, n_chunks, sched, ws, dev, message, stream)
    check(load().tpf_matmul_allreduce(h.ptr, p, M, N, K, ptr_array([x.data_ptr() for x in X]),
                                      ptr_array([w.data_ptr() for w in W]), Y.data_ptr(), _dtype_code(Y.dtype),
                                      n_chunks, _sched(sched, message), ws.data_ptr() if ws is not None else None, ws_bytes,
                                      _stream_ptr(stream)))
    return Y


def matmul_allreduce_noalloc(X: List[torch.Tensor], W: List[torch.Tensor], Y: torch.Tensor, n_chunks: int = 1,
                             sched="auto", handle: Optional[Handle] = None, stream=None,
                             message: str = "fp32") -> torch.Tensor:
    """Y = sum_k X[k] @ W[k] into the caller's Y with no allocation anywhere:
    the library keeps the partials in its static per-device workspace
    (NOALLOC_SCRATCH_BYTES); calls that overlap on one device race."""
    p = len(X)
    _need(p >= 1, "X: no shards given")
    M, K = X[0].shape
    N = W[0].shape[1]
    _check_shards("W", W, p)
    dev = _check("X", X, (M, K))
    _check("W", W, (K, N), device=dev)
    _check("Y", [Y], (M, N), OUT_DTYPES, dev)
    h = _handle(handle, dev, stream)
    check(load().tpf_matmul_allreduce_noalloc(h.ptr, p, M, N, K, ptr_array([x.data_ptr() for x in X]),
                                              ptr_array([w.data_ptr() for w in W]), Y.data_ptr(),
                                              _dtype_code(Y.dtype), n_chunks, _sched(sched, message),
                                              _stream_ptr(stream)))
    return Y


def matmul_reducescatter(X: List[torch.Tensor], W: List[torch.Tensor], out_dtype=torch.bfloat16, n_chunks: int = 1,
                         sched="auto", Y: Optional[List[torch.Tensor]] = None, ws: Optional[torch.Tensor] = None,
                         handle: Optional[Handle] = None, stream=None, message: str = "fp32") -> List[torch.Tensor]:
    """Slice r = rows [r*M/p, (r+1)*M/p) of sum_k X[k] @ W[k] (ReduceScatter layout)."""
    p = len(X)
    _need(p >= 1, "X: no shards given")
    M, K = X[0].shape
    N = W[0].shape[1]
    _check_shards("W", W, p)
    dev = _check("X", X, (M, K))
    _check("W", W, (K, N), device=dev)
    if Y is None:
        with _on(stream):
            Y = [torch.empty((M // p, N), dtype=out_dtype, device=dev) for _ in range(p)]
    _check_shards("Y", Y, p)
    _check("Y", Y, (M // p, N), OUT_DTYPES, dev)
    _need(len({y.dtype for y in Y}) == 1, "Y: the slices differ in dtype")
    _check_ws(ws, dev)
    h = _handle(handle, dev, stream)
    ws, ws_bytes = _ws(OP_MATMUL_REDUCESCATTER, p, M, N, K, n_chunks, sched, ws, dev, message, stream)
    check(load().tpf_matmul_reducescatter(h.ptr, p, M, N, K, ptr_array([x.data_ptr() for x in X]),
                                          ptr_array([w.data_ptr() for w in W]), ptr_array([y.data_ptr() for y in Y]),
                                          _dtype_code(Y[0].dtype), n_chunks, _sched(sched, message),
                                          ws.data_ptr() if ws is not None else None, ws_bytes, _stream_ptr(stream)))
    return Y


def allgather_matmul(X_slices: List[torch.Tensor], W: torch.Tensor, out_dtype=torch.bfloat16, n_chunks: int = 1,
                     sched="auto", X_gathered: Optional[torch.Tensor] = None, Y: Optional[torch.Tensor] = None,
                     handle: Optional[Handle] = None, stream=None):
    """(X_gathered, Y): slices concatenated in rank order, then Y = X_gathered @ W."""
    p = len(X_slices)
    _need(p >= 1, "X_slices: no slices given")
    Ms, K = X_slices[0].shape
    M = Ms * p
    N = W.shape[1]
    dev = _check("W", [W], (K, N))
    _check("X_slices", X_slices, (Ms, K), device=dev)
    with _on(stream):
        if X_gathered is None:
            X_gathered = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        if Y is None:
            Y = torch.empty((M, N), dtype=out_dtype, device=dev)
    _check("X_gathered", [X_gathered], (M, K), device=dev)
    _check("Y", [Y], (M, N), OUT_DTYPES, dev)
    h = _handle(handle, dev, stream)
    check(load().tpf_allgather_matmul(h.ptr, p, M, N, K, ptr_array([x.data_ptr() for x in X_slices]), W.data_ptr(),
                                      X_gathered.data_ptr(), Y.data_ptr(), _dtype_code(Y.dtype), n_chunks,
                                      _sched(sched), None, 0, _stream_ptr(stream)))
    return X_gathered, Y


def matmul_dx(dY: List[torch.Tensor], W: List[torch.Tensor], semantic: int = ALLREDUCE, out_dtype=torch.bfloat16,
              n_chunks: int = 1, sched="auto", dX=None, ws: Optional[torch.Tensor] = None,
              handle: Optional[Handle] = None, stream=None, message: str = "fp32"):
    """dX = sum_k dY[k] @ W[k]^T; one tensor (ALLREDUCE) or p row slices (REDUCESCATTER)."""
    p = len(dY)
    _need(p >= 1, "dY: no shards given")
    M, Ns = dY[0].shape
    Kin = W[0].shape[0]
    _check_shards("W", W, p)
    dev = _check("dY", dY, (M, Ns))
    _check("W", W, (Kin, Ns), device=dev)
    if dX is None:
        with _on(stream):
            if semantic == ALLREDUCE:
                dX = torch.empty((M, Kin), dtype=out_dtype, device=dev)
            else:
                dX = [torch.empty((M // p, Kin), dtype=out_dtype, device=dev) for _ in range(p)]
    outs = [dX] if semantic == ALLREDUCE else list(dX)
    if semantic == ALLREDUCE:
        _check("dX", outs, (M, Kin), OUT_DTYPES, dev)
    else:
        _check_shards("dX", outs, p)
        _check("dX", outs, (M // p, Kin), OUT_DTYPES, dev)
        _need(len({o.dtype for o in outs}) == 1, "dX: the slices differ in dtype")
    _check_ws(ws, dev)
    h = _handle(handle, dev, stream)
    ws, ws_bytes = _ws(OP_MATMUL_DX, p, M, Kin, Ns, n_chunks, sched, ws, dev, message, stream)
    check(load().tpf_matmul_dx(h.ptr, semantic, p, M, Kin, Ns, ptr_array([d.data_ptr() for d in dY]),
                               ptr_array([w.data_ptr() for w in W]), ptr_array([o.data_ptr() for o in outs]),
                               _dtype_code(outs[0].dtype), n_chunks, _sched(sched, message),
                               ws.data_ptr() if ws is not None else None, ws_bytes, _stream_ptr(stream)))
    return dX


def weight_grad(A: List[torch.Tensor], B: List[torch.Tensor], out_dtype=torch.float32, dW=None,
                handle: Optional[Handle] = None, stream=None) -> List[torch.Tensor]:
    """dW[k] = A[k]^T @ B[k] for every shard k (A[k] [M, R], B[k] [M, C]).

    Row-parallel: A = X_k per shard, B = [dY] * p.  Column-parallel:
    A = [X_gathered] * p, B = dY_k per shard."""
    p = len(A)
    _need(p >= 1, "A: no shards given")
    M, R = A[0].shape
    C = B[0].shape[1]
    _check_shards("B", B, p)
    dev = _check("A", A, (M, R))
    _check("B", B, (M, C), device=dev)
    if dW is None:
        with _on(stream):
            dW = [torch.empty((R, C), dtype=out_dtype, device=dev) for _ in range(p)]
    _check_shards("dW", dW, p)
    _check("dW", dW, (R, C), OUT_DTYPES, dev)
    _need(len({d.dtype for d in dW}) == 1, "dW: the shards differ in dtype")
    h = _handle(handle, dev, stream)
    check(load().tpf_weight_grad(h.ptr, p, M, R, C, ptr_array([a.data_ptr() for a in A]),
                                 ptr_array([b.data_ptr() for b in B]), ptr_array([d.data_ptr() for d in dW]),
                                 _dtype_code(dW[0].dtype), _stream_ptr(stream)))
    return dW


def rowpar_dx(dY: torch.Tensor, W: List[torch.Tensor], out_dtype=torch.bfloat16, dX=None,
              handle: Optional[Handle] = None, stream=None) -> List[torch.Tensor]:
    """dX[k] = dY @ W[k]^T for every shard k: the input gradient of a
    row-parallel Linear (dY [M, N] whole on every rank, W[k] [K_shard, N])."""
    p = len(W)
    _need(p >= 1, "W: no shards given")
    M, N = dY.shape
    Ks = W[0].shape[0]
    dev = _check("dY", [dY], (M, N))
    _check("W", W, (Ks, N), device=dev)
    if dX is None:
        with _on(stream):
            dX = [torch.empty((M, Ks), dtype=out_dtype, device=dev) for _ in range(p)]
    _check_shards("dX", dX, p)
    _check("dX", dX, (M, Ks), OUT_DTYPES, dev)
    _need(len({d.dtype for d in dX}) == 1, "dX: the shards differ in dtype")
    h = _handle(handle, dev, stream)
    check(load().tpf_rowpar_dx(h.ptr, p, M, Ks, N, dY.data_ptr(), ptr_array([w.data_ptr() for w in W]),
                               ptr_array([d.data_ptr() for d in dX]), _dtype_code(dX[0].dtype),
                               _stream_ptr(stream)))
    return dX


def mlp_sp(X_slices: List[torch.Tensor], W1: List[torch.Tensor], W2: List[torch.Tensor], out_dtype=torch.bfloat16,
           n_chunks: int = 1, sched="auto", X_gathered: Optional[torch.Tensor] = None,
           H: Optional[List[torch.Tensor]] = None, Y: Optional[List[torch.Tensor]] = None,
           ws: Optional[torch.Tensor] = None, handle: Optional[Handle] = None, stream=None,
           message: str = "fp32"):
    """MLP block under sequence parallelism: AllGather -> FC1 (column shards) + GeLU
    -> FC2 (row shards) -> ReduceScatter.  Returns (X_gathered, H, Y_slices)."""
    p = len(X_slices)
    _need(p >= 1, "X_slices: no slices given")
    Sp, Hd = X_slices[0].shape
    S = Sp * p
    F = W1[0].shape[1]
    _check_shards("W1", W1, p)
    _check_shards("W2", W2, p)
    dev = _check("X_slices", X_slices, (Sp, Hd))
    _check("W1", W1, (Hd, F), device=dev)
    _check("W2", W2, (F, Hd), device=dev)
    with _on(stream):
        if X_gathered is None:
            X_gathered = torch.empty((S, Hd), dtype=torch.bfloat16, device=dev)
        if H is None:
            H = [torch.empty((S, F), dtype=torch.bfloat16, device=dev) for _ in range(p)]
        if Y is None:
            Y = [torch.empty((Sp, Hd), dtype=out_dtype, device=dev) for _ in range(p)]
    _check("X_gathered", [X_gathered], (S, Hd), device=dev)
    _check_shards("H", H, p)
    _check("H", H, (S, F), device=dev)
    _check_shards("Y", Y, p)
    _check("Y", Y, (Sp, Hd), OUT_DTYPES, dev)
    _need(len({y.dtype for y in Y}) == 1, "Y: the slices differ in dtype")
    _check_ws(ws, dev)
    h = _handle(handle, dev, stream)
    ws, ws_bytes = _ws(OP_MLP_SP, p, S, Hd, F, n_chunks, sched, ws, dev, message, stream)
    check(load().tpf_mlp_sp(h.ptr, p, S, Hd, F, ptr_array([x.data_ptr() for x in X_slices]),
                            ptr_array([w.data_ptr() for w in W1]), ptr_array([w.data_ptr() for w in W2]),
                            X_gathered.data_ptr(), ptr_array([t.data_ptr() for t in H]),
                            ptr_array([y.data_ptr() for y in Y]), _dtype_code(Y[0].dtype), n_chunks,
                            _sched(sched, message), ws.data_ptr() if ws is not None else None, ws_bytes,
                            _stream_ptr(stream)))
    return X_gathered, H, Y
