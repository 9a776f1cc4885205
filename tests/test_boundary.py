"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/tpfuse.h declares, and rejects bad arguments on the host
before touching any device (all calls here use a NULL handle and fake but
aligned pointers; a check that passed would fail on the NULL handle)."""
import ctypes
import os
import re

import pytest

from tensor_gemm_reduction_amd import tpfuse as tp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tpfuse.h")

A16 = 0x1000      # fake, 16-byte aligned, never dereferenced
MIS = 0x1008      # fake, misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tpf_[a-z_]+)\s*\(", text)))


def test_header_matches_binding():
    assert set(declared_functions()) == set(tp.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = tp.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_constants_match_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(TPF_[A-Z0-9_]+)\s+(-?\d+)", text))
    assert int(defs["TPF_OK"]) == tp.OK
    assert int(defs["TPF_ERR_TIMEOUT"]) == tp.ERR_TIMEOUT
    assert int(defs["TPF_ERR_HIP"]) == tp.ERR_HIP
    assert int(defs["TPF_F32"]) == tp.F32 and int(defs["TPF_BF16"]) == tp.BF16
    assert int(defs["TPF_SCHED_REDUCE_ONLY"]) == tp.SCHED_REDUCE_ONLY
    assert int(defs["TPF_SCHED_TILE"]) == tp.SCHED_TILE
    assert int(defs["TPF_SCHED_FOLD"]) == tp.SCHED_FOLD
    assert int(defs["TPF_SCHED_STATIONARY"]) == tp.SCHED_STATIONARY
    assert int(defs["TPF_REDUCESCATTER"]) == tp.REDUCESCATTER
    assert int(defs["TPF_OP_MATMUL_DX"]) == tp.OP_MATMUL_DX
    assert int(defs["TPF_MAX_SHARDS"]) == tp.MAX_SHARDS and int(defs["TPF_MAX_CHUNKS"]) == tp.MAX_CHUNKS
    assert tp.load().tpf_version() == int(defs["TPF_VERSION"])


def test_status_strings():
    lib = tp.load()
    for code in range(0, -8, -1):
        s = lib.tpf_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.tpf_status_string(-99).decode() == "unknown status"


def test_workspace_size():
    ws = tp.workspace_size
    assert ws(tp.OP_MATMUL_ALLREDUCE, 4, 4096, 4096, 4096, 8) == 4 * 4096 * 4096 * 4
    assert ws(tp.OP_MATMUL_REDUCESCATTER, 8, 8192, 8192, 3584, 16) == 8 * 8192 * 8192 * 4
    assert ws(tp.OP_MATMUL_DX, 8, 2048, 12288, 6144, 8) == 8 * 2048 * 12288 * 4
    assert ws(tp.OP_ALLGATHER_MATMUL, 8, 2048, 6144, 12288, 8) == 0
    # invalid arguments give 0
    assert ws(tp.OP_MATMUL_ALLREDUCE, 0, 16, 16, 16, 1) == 0
    assert ws(tp.OP_MATMUL_REDUCESCATTER, 3, 16, 16, 16, 1) == 0      # M % p
    assert ws(tp.OP_MATMUL_ALLREDUCE, 2, 16, 12, 16, 1) == 0          # N % 8
    assert ws(tp.OP_MATMUL_ALLREDUCE, 2, 16, 16, 16, 17) == 0         # n_chunks > M
    # 2-byte messages halve the partials' workspace
    assert ws(tp.OP_MATMUL_ALLREDUCE, 4, 4096, 4096, 4096, 8, message="bf16") == 4 * 4096 * 4096 * 2
    assert ws(tp.OP_MATMUL_DX, 8, 2048, 12288, 6144, 8, "unfused", "bf16") == 8 * 2048 * 12288 * 2
    assert ws(tp.OP_ALLGATHER_MATMUL, 8, 2048, 6144, 12288, 8, message="bf16") == 0
    assert ws(tp.OP_MATMUL_ALLREDUCE, 4, 64, 64, 64, 1, tp.SCHED_TILE | 0x200) == 0   # unknown flag
    assert ws(tp.OP_MATMUL_ALLREDUCE, 4, 64, 64, 64, 1, tp.SCHED_STATIONARY + 1) == 0  # unknown scheduler
    # the output-stationary single launch keeps the partials on chip (row-parallel
    # calls and the MLP block); dX runs unfused under it and needs the full size
    assert ws(tp.OP_MATMUL_ALLREDUCE, 8, 16, 8192, 1024, 1, "stationary") == 0
    assert ws(tp.OP_MATMUL_REDUCESCATTER, 8, 64, 8192, 1024, 2, "stationary", "bf16") == 0
    assert ws(tp.OP_MLP_SP, 8, 64, 8192, 1024, 1, "stationary") == 0
    assert ws(tp.OP_MATMUL_DX, 8, 64, 1024, 512, 1, "stationary") == 8 * 64 * 1024 * 4
    # with more than 64 rows every reducing call (dX too) runs the large-tile single launch
    assert ws(tp.OP_MATMUL_DX, 8, 65, 1024, 512, 1, "stationary") == 0
    assert ws(tp.OP_MATMUL_ALLREDUCE, 4, 8192, 8192, 7168, 1, "stationary") == 0
    assert ws(tp.OP_MATMUL_ALLREDUCE, 8, 16, 8192, 1024, 1, "auto") == 8 * 16 * 8192 * 4
    assert ws(tp.OP_MATMUL_ALLREDUCE, 4, 64, 64, 64, 1, "fold") == 4 * 64 * 64 * 4


def _ar(p=2, M=64, N=64, K=64, X=None, W=None, Y=A16, dtype=tp.BF16, n=1, sched=tp.SCHED_AUTO, ws=A16,
        ws_bytes=None, handle=None):
    lib = tp.load()
    X = tp.ptr_array([A16] * p) if X is None else X
    W = tp.ptr_array([A16] * p) if W is None else W
    if ws_bytes is None:
        ws_bytes = p * M * N * 4
    return lib.tpf_matmul_allreduce(handle, p, M, N, K, X, W, Y, dtype, n, sched, ws, ws_bytes, None)


def _err(call):
    return tp.load().tpf_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(p=0), tp.ERR_SHAPE),
    (dict(p=17), tp.ERR_SHAPE),
    (dict(M=0), tp.ERR_SHAPE),
    (dict(N=-8), tp.ERR_SHAPE),
    (dict(K=0), tp.ERR_SHAPE),
    (dict(n=0), tp.ERR_SHAPE),
    (dict(n=65, M=128), tp.ERR_SHAPE),
    (dict(n=9, M=8), tp.ERR_SHAPE),
    (dict(N=12), tp.ERR_ALIGNMENT),
    (dict(K=20), tp.ERR_ALIGNMENT),
    (dict(dtype=7), tp.ERR_INVALID_ARG),
    (dict(sched=9), tp.ERR_INVALID_ARG),
    (dict(sched=tp.SCHED_UNFUSED | 0x200), tp.ERR_INVALID_ARG),       # unknown flag bit
    (dict(sched=7 | tp.MSG_BF16), tp.ERR_INVALID_ARG),                # unknown scheduler with the message flag
    (dict(sched=tp.SCHED_UNFUSED | tp.MSG_BF16, ws_bytes=2 * 64 * 64 * 2 - 1), tp.ERR_WORKSPACE),
    (dict(sched=tp.SCHED_UNFUSED | tp.MSG_BF16, ws_bytes=2 * 64 * 64 * 2), tp.ERR_INVALID_ARG),  # enough: NULL handle
    (dict(Y=None), tp.ERR_INVALID_ARG),
    (dict(Y=MIS), tp.ERR_ALIGNMENT),
    (dict(ws=None), tp.ERR_WORKSPACE),
    (dict(ws=MIS), tp.ERR_ALIGNMENT),
    (dict(ws_bytes=100), tp.ERR_WORKSPACE),
    ({}, tp.ERR_INVALID_ARG),            # everything valid: the NULL handle is reported last
])
def test_allreduce_argument_checks(kw, code):
    assert _ar(**kw) == code, _err(None)


def test_pointer_array_checks():
    lib = tp.load()
    assert _ar(X=tp.ptr_array([A16, 0])) == tp.ERR_INVALID_ARG
    assert "X[1]" in lib.tpf_last_error().decode()
    assert _ar(W=tp.ptr_array([A16, MIS])) == tp.ERR_ALIGNMENT
    assert "W[1]" in lib.tpf_last_error().decode()
    assert lib.tpf_matmul_allreduce(None, 2, 64, 64, 64, None, tp.ptr_array([A16] * 2), A16, 0, 1, 0, A16,
                                    1 << 20, None) == tp.ERR_INVALID_ARG


def test_reducescatter_checks():
    lib = tp.load()
    arr = tp.ptr_array([A16] * 4)
    # M not divisible by p
    assert lib.tpf_matmul_reducescatter(None, 4, 30, 64, 64, arr, arr, arr, 0, 1, 0, A16, 1 << 30, None) == tp.ERR_SHAPE
    # a NULL slice
    assert lib.tpf_matmul_reducescatter(None, 4, 32, 64, 64, arr, arr, tp.ptr_array([A16, A16, 0, A16]), 0, 1, 0, A16,
                                        1 << 30, None) == tp.ERR_INVALID_ARG
    assert lib.tpf_matmul_reducescatter(None, 4, 32, 64, 64, arr, arr, arr, 0, 1, 0, A16, 1 << 30,
                                        None) == tp.ERR_INVALID_ARG


def test_allgather_checks():
    lib = tp.load()
    arr = tp.ptr_array([A16] * 8)
    assert lib.tpf_allgather_matmul(None, 8, 100, 64, 64, arr, A16, A16, A16, 0, 1, 0, None, 0, None) == tp.ERR_SHAPE
    assert lib.tpf_allgather_matmul(None, 8, 128, 64, 64, arr, None, A16, A16, 0, 1, 0, None, 0,
                                    None) == tp.ERR_INVALID_ARG
    assert lib.tpf_allgather_matmul(None, 8, 128, 64, 64, arr, A16, MIS, A16, 0, 1, 0, None, 0,
                                    None) == tp.ERR_ALIGNMENT
    # no workspace needed: everything valid ends at the NULL handle
    assert lib.tpf_allgather_matmul(None, 8, 128, 64, 64, arr, A16, A16, A16, 0, 1, 0, None, 0,
                                    None) == tp.ERR_INVALID_ARG
    assert "handle" in lib.tpf_last_error().decode()


def test_dx_checks():
    lib = tp.load()
    arr = tp.ptr_array([A16] * 8)
    big = 1 << 40
    assert lib.tpf_matmul_dx(None, 5, 8, 64, 64, 64, arr, arr, arr, 0, 1, 0, A16, big, None) == tp.ERR_INVALID_ARG
    assert lib.tpf_matmul_dx(None, tp.REDUCESCATTER, 8, 60, 64, 64, arr, arr, arr, 0, 1, 0, A16, big,
                             None) == tp.ERR_SHAPE
    # AllReduce semantics reads one output pointer only
    one = tp.ptr_array([A16])
    assert lib.tpf_matmul_dx(None, tp.ALLREDUCE, 8, 60, 64, 64, arr, arr, one, 0, 1, 0, A16, big,
                             None) == tp.ERR_INVALID_ARG
    assert "handle" in lib.tpf_last_error().decode()
    # workspace is sized by the output width K_in
    assert lib.tpf_matmul_dx(None, tp.ALLREDUCE, 2, 64, 128, 64, arr, arr, one, 0, 1, 0, A16, 2 * 64 * 128 * 4 - 16,
                             None) == tp.ERR_WORKSPACE


def test_weight_grad_checks():
    lib = tp.load()
    P2 = tp.ptr_array([A16] * 2)

    def call(p=2, M=64, R=64, C=64, A=P2, B=P2, D=P2, dtype=tp.F32):
        return lib.tpf_weight_grad(None, p, M, R, C, A, B, D, dtype, None)
    assert call(p=0) == tp.ERR_SHAPE
    assert call(M=0) == tp.ERR_SHAPE
    assert call(R=12) == tp.ERR_ALIGNMENT
    assert call(C=20) == tp.ERR_ALIGNMENT
    assert call(dtype=5) == tp.ERR_INVALID_ARG
    assert call(A=None) == tp.ERR_INVALID_ARG
    assert call(B=tp.ptr_array([A16, MIS])) == tp.ERR_ALIGNMENT
    assert call(D=tp.ptr_array([A16, 0])) == tp.ERR_INVALID_ARG
    assert call(M=1 << 20, R=1 << 12) == tp.ERR_UNSUPPORTED       # 8 GiB operand
    assert call() == tp.ERR_INVALID_ARG                             # all valid: the NULL handle
    assert "handle" in _err(None)


def test_rowpar_dx_checks():
    lib = tp.load()
    P2 = tp.ptr_array([A16] * 2)

    def call(p=2, M=64, K=64, N=64, dY=A16, W=P2, D=P2, dtype=tp.BF16):
        return lib.tpf_rowpar_dx(None, p, M, K, N, dY, W, D, dtype, None)
    assert call(p=0) == tp.ERR_SHAPE
    assert call(p=17) == tp.ERR_SHAPE
    assert call(M=0) == tp.ERR_SHAPE
    assert call(K=12) == tp.ERR_ALIGNMENT
    assert call(N=20) == tp.ERR_ALIGNMENT
    assert call(dtype=5) == tp.ERR_INVALID_ARG
    assert call(dY=None) == tp.ERR_INVALID_ARG
    assert call(dY=MIS) == tp.ERR_ALIGNMENT
    assert call(W=tp.ptr_array([A16, MIS])) == tp.ERR_ALIGNMENT
    assert call(D=tp.ptr_array([A16, 0])) == tp.ERR_INVALID_ARG
    assert call(M=1 << 20, N=1 << 12) == tp.ERR_UNSUPPORTED       # 8 GiB operand
    assert call() == tp.ERR_INVALID_ARG                             # all valid: the NULL handle
    assert "handle" in _err(None)


def test_handle_calls_reject_null():
    lib = tp.load()
    assert lib.tpf_sync_status(None, None) == tp.ERR_INVALID_ARG
    assert lib.tpf_debug_set_wait(None, 10, 1) == tp.ERR_INVALID_ARG
    assert lib.tpf_debug_set_kernel_timing(None, 1) == tp.ERR_INVALID_ARG
    assert lib.tpf_debug_kernel_times(None, None, 0) == tp.ERR_INVALID_ARG
    assert lib.tpf_debug_last_sched(None) == tp.ERR_INVALID_ARG
    assert lib.tpf_create(None, 0) == tp.ERR_INVALID_ARG
    assert lib.tpf_destroy(None) == tp.OK


def test_noalloc_entry_point_checks_on_host():
    """The no-allocation MatMul->AllReduce refuses, before touching a device,
    a request whose partials exceed its static workspace, and otherwise
    reaches the (NULL) handle check; it takes no workspace arguments."""
    lib = tp.load()
    X = tp.ptr_array([A16] * 4)
    W = tp.ptr_array([A16] * 4)
    # 4 x 4096 x 4096 fp32 partials = 256 MiB > 64 MiB
    st = lib.tpf_matmul_allreduce_noalloc(None, 4, 4096, 4096, 4096, X, W, A16, tp.BF16, 1, tp.SCHED_AUTO, None)
    assert st == tp.ERR_UNSUPPORTED
    assert "64" in lib.tpf_last_error().decode() or "67108864" in lib.tpf_last_error().decode()
    # 2-byte messages halve the need: 4 x 1024 x 4096 x 2 = 32 MiB fits, so the
    # next check (the NULL handle) is the one that fails
    st = lib.tpf_matmul_allreduce_noalloc(None, 4, 1024, 4096, 4096, X, W, A16, tp.BF16, 1,
                                          tp.SCHED_AUTO | tp.MSG_BF16, None)
    assert st == tp.ERR_INVALID_ARG and "handle" in lib.tpf_last_error().decode()
    # the stationary scheduler needs no workspace at all
    st = lib.tpf_matmul_allreduce_noalloc(None, 4, 4096, 4096, 4096, X, W, A16, tp.BF16, 1, tp.SCHED_STATIONARY, None)
    assert st == tp.ERR_INVALID_ARG
    # ordinary argument checks still apply
    assert lib.tpf_matmul_allreduce_noalloc(None, 4, 64, 60, 64, X, W, A16, tp.BF16, 1, 0, None) == tp.ERR_ALIGNMENT
    assert lib.tpf_matmul_allreduce_noalloc(None, 4, 64, 64, 64, X, W, MIS, tp.BF16, 1, 0, None) == tp.ERR_ALIGNMENT
    text = open(HEADER).read()
    assert "#define TPF_NOALLOC_SCRATCH_BYTES (64u << 20)" in text and tp.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_debug_delay_argument_checks():
    """The timing-perturbation knob checks its arguments before the handle."""
    lib = tp.load()
    assert lib.tpf_debug_set_delay(None, 1, -1, 1) == tp.ERR_INVALID_ARG
    assert lib.tpf_debug_set_delay(None, 1, 2, 1025) == tp.ERR_INVALID_ARG
    assert lib.tpf_debug_set_delay(None, 1, 2, -1) == tp.ERR_INVALID_ARG
    assert lib.tpf_debug_set_delay(None, 1, 2, 4) == tp.ERR_INVALID_ARG      # valid arguments, NULL handle
    assert "handle" in lib.tpf_last_error().decode()
