/*
 * libtpfuse — fused tensor-parallel Linear (GEMM + cross-shard reduction) for
 * AMD Instinct MI355X (gfx950).
 *
 * One GPU holds all p shards of a tensor-parallel layer ("simulated ranks"):
 * the library computes every shard's local GEMM with bf16 matrix-core tiles,
 * keeps each shard's fp32 local output (the message a rank would send) in a
 * caller-provided workspace, and produces the cross-shard sum in the layout
 * that the collective's semantics require.  Several schedulers order that
 * work: chunked ones that cut the output into contiguous row chunks and
 * overlap the reduction of chunk c with the GEMM of later chunks (a
 * persistent kernel with per-chunk ready counters, two HIP streams with
 * per-chunk events, or readiness per output tile), the unfused
 * GEMM-then-reduce baseline, a fold of the reduction into the last shard's
 * GEMM epilogue, and a single launch that keeps every shard's partial of an
 * output tile on chip.  The default (AUTO) picks between the fold and the
 * unfused baseline by shape (see TPF_SCHED_AUTO).  The sum over
 * shards is a left fold in shard order k = 0..p-1 in fp32, rounded once to
 * the output type, so results are bit-identical for every chunk count and
 * every scheduler.
 *
 * Sources (web pages, cited by title and section):
 *  - ai-infra-kb M027 "compute-communication fusion" page, §01 (row-parallel
 *    Linear: Y = Y_0 + Y_1; AllReduce vs ReduceScatter layouts; AllGather
 *    then MatMul), §02 (MatMul->AllReduce chunked along output rows, the
 *    reduction of chunk 1 overlapping the GEMM of chunk 2; AllGather->MatMul
 *    computing once enough input blocks have arrived), §03 (same chunk order
 *    on every rank, a ready signal per chunk, a final wait for all chunks),
 *    §04 (measure the whole GEMM and the whole collective separately),
 *    §06 (record workspace peak).
 *  - cnblogs tensor-parallel tutorial (列并行与行并行的前向/反向传播), §2.3 / §三
 *    (column shards, backward dX = sum_k dY_k A_k^T), §2.4 / §四 (row shards,
 *    Y = sum_k X_k A_k), §2.5-2.7 (AllReduce, AllGather, ReduceScatter).
 *
 * Conventions for every call:
 *  - All matrices are row-major and contiguous; inputs are bfloat16.
 *  - Every device pointer must be 16-byte aligned; the reduction length and
 *    the output width must be multiples of 8 elements.
 *  - Pointers are checked for alignment only, not for where they live or
 *    how large their buffers are: host memory, another device's memory or a
 *    buffer shorter than the shape arguments imply is undefined behaviour
 *    (a GPU memory fault).  The Python binding checks the device, shape,
 *    dtype and layout of every tensor before it calls in.
 *  - Pointer arrays (X[], W[], slices[]) are host arrays read during the call
 *    only; the device buffers they name are owned by the caller.  The library
 *    never allocates or frees caller memory.  Outputs must not alias inputs
 *    or each other.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream) after any work already on it; the call returns without waiting.
 *    Internal forks onto the handle's side streams join back into `stream`
 *    before the call returns, so callers see single-stream semantics.
 *  - A handle runs at most one call at a time; use one handle per concurrent
 *    stream.
 *  - Return value: TPF_OK (0) or a negative TPF_ERR_* code; the message of
 *    the last failure on the calling thread is tpf_last_error().  Argument
 *    checks run on the host before anything is enqueued; a failed check
 *    enqueues nothing.  Arguments are checked before the handle, so the
 *    checks work without a GPU.
 */
#ifndef TPFUSE_H
#define TPFUSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TPF_VERSION 100          /* 1.0.0 */
#define TPF_MAX_SHARDS 16        /* largest p accepted */
#define TPF_MAX_CHUNKS 64        /* largest n_chunks accepted */

/* Status codes. */
#define TPF_OK 0
#define TPF_ERR_INVALID_ARG -1   /* null pointer, unknown enum, bad handle */
#define TPF_ERR_SHAPE -2         /* non-positive size, p or n_chunks out of range, M % p != 0 where required */
#define TPF_ERR_ALIGNMENT -3     /* pointer not 16-byte aligned, N or K not a multiple of 8 */
#define TPF_ERR_WORKSPACE -4     /* workspace missing or smaller than tpf_workspace_size() */
#define TPF_ERR_UNSUPPORTED -5   /* valid request the library cannot run (size limits) */
#define TPF_ERR_HIP -6           /* a HIP runtime call failed (message in tpf_last_error) */
#define TPF_ERR_TIMEOUT -7       /* a bounded wait inside the persistent kernel gave up */

/* Output element type (inputs are always bfloat16). */
#define TPF_BF16 0
#define TPF_F32 1

/* Schedulers.  Every scheduler computes the same bits. */
#define TPF_SCHED_AUTO 0         /* library's choice.  With every shard on one GPU the reduction shares HBM
                                    and L2 with the GEMM, and overlapping it chunk by chunk costs more
                                    than it hides; folding it into the last shard's GEMM epilogue does
                                    pay when the last shard's tiles fill whole waves of the GPU.  AUTO
                                    runs TPF_SCHED_FOLD for the reducing calls (MatMul->AllReduce,
                                    MatMul->ReduceScatter, dX, the MLP block's FC2) on the large tiles
                                    (M > 64) when the p-1 shards' tiles and the last shard's tiles take
                                    no more waves of one-tile-per-CU workgroups than all p shards'
                                    tiles together, and TPF_SCHED_UNFUSED otherwise (and for
                                    decode-shaped M and AllGather->MatMul); tpf_debug_last_sched
                                    reports the choice.  Every scheduler gives the same bits. */
#define TPF_SCHED_PERSISTENT 1   /* one persistent kernel: work queue + per-chunk ready counters */
#define TPF_SCHED_TWO_STREAM 2   /* per-chunk launches alternating between the caller's stream and a second
                                    handle stream, so that chunk c's reduction runs beside chunk c+1's
                                    GEMM: for the large tiles (M > 64) each chunk runs as TPF_SCHED_FOLD
                                    over its rows (the first p-1 shards' tiles, then the last shard's
                                    tiles with the chunk's reduction folded into their epilogue); for
                                    decode-shaped M each chunk's GEMM is followed, on a side stream after a
                                    per-chunk event, by that chunk's reduction kernel */
#define TPF_SCHED_UNFUSED 3      /* whole GEMM, then the whole reduction (the serial baseline) */
#define TPF_SCHED_GEMM_ONLY 4    /* measurement: only the shard GEMMs (partials into the workspace; for
                                    AllGather->MatMul: only the GEMM over an already gathered X) */
#define TPF_SCHED_REDUCE_ONLY 5  /* measurement: only the reduction of partials already in the workspace
                                    (for AllGather->MatMul: only the gather copy) */
#define TPF_SCHED_TILE 6         /* readiness per output tile: one kernel (one workgroup per tile) runs the
                                    shard GEMM tiles of the whole output in an L2-friendly order, and the
                                    workgroup
                                    that finishes the last shard of an output tile sums that tile at once
                                    (the M027 page's per-chunk readiness at the finest chunking, every
                                    output tile its own chunk; n_chunks is checked but does not change
                                    the schedule).  At most 131072 output tiles (TPF_ERR_UNSUPPORTED
                                    beyond).  For AllGather->MatMul, which has no reduction, it runs as
                                    TPF_SCHED_PERSISTENT. */
#define TPF_SCHED_FOLD 7         /* the reduction folded into the last shard's GEMM epilogue: one launch
                                    computes the partials of shards 0..p-2, a second computes shard p-1
                                    and, per output element, adds those partials in shard order and then
                                    its own accumulator, writing the result directly (no partial of the
                                    last shard, no separate reduction pass; the same additions in the
                                    same order as TPF_SCHED_UNFUSED, so the same bits).  The M027 page's
                                    pipelining taken to one step: the "communication" of the last shard
                                    is its epilogue.  n_chunks is checked but does not change the
                                    schedule.  For M <= 64 (one shard's tiles could not fill the GPU)
                                    and for AllGather->MatMul it runs as TPF_SCHED_UNFUSED. */
#define TPF_SCHED_STATIONARY 8   /* one launch, output-stationary: each workgroup owns an output tile,
                                    runs every shard's GEMM for it (each the same MFMA chain as the
                                    partials the other schedulers store) and folds the shards' fp32
                                    results on chip in shard order, rounding once: no partial goes to
                                    memory, no workspace, no second launch.  M <= 64: tiles of 32 or 64
                                    rows by 32 columns, the partials folded in LDS, for weights stored
                                    [K][N] only (dX runs as TPF_SCHED_UNFUSED there).  M > 64: tiles of
                                    128 x 256 with the running sum in registers, for every reducing
                                    call including dX.  Same bits as every other scheduler; slower
                                    than TPF_SCHED_UNFUSED or TPF_SCHED_FOLD on the measured shapes
                                    (so AUTO does not pick it), but it needs no workspace at all.
                                    AllGather->MatMul runs as TPF_SCHED_UNFUSED.  n_chunks is checked
                                    but does not change the schedule. */

/* Message precision, OR-ed into the `sched` argument of the reducing calls
 * (tpf_matmul_allreduce, tpf_matmul_reducescatter, tpf_matmul_dx, and
 * tpf_workspace_size; ignored by tpf_allgather_matmul, which reduces
 * nothing).  With TPF_MSG_BF16 each shard's local output (the message a rank
 * would send; the M027 page's worked example sizes it at 2 bytes per element)
 * is rounded once, RNE, from its fp32 tile accumulation to bf16 and kept in a
 * workspace of p * M * N * 2 bytes; the sum over shards is still a left fold
 * in fp32 in shard order, rounded once to the output type.  Every scheduler
 * gives the same bits for the same flag.  Against the exact sum, each
 * element then carries up to half a bf16 ulp of each shard's partial
 * (relative 2^-9) in addition to the fp32-message error, so fp32 outputs no
 * longer meet 1e-4 * rms; without the flag the partials are fp32. */
#define TPF_MSG_BF16 0x100

/* Output semantics of the column-parallel backward. */
#define TPF_ALLREDUCE 0          /* one full [M, K_in] result */
#define TPF_REDUCESCATTER 1      /* p row slices [M/p, K_in] */

/* Operation ids for tpf_workspace_size. */
#define TPF_OP_MATMUL_ALLREDUCE 0
#define TPF_OP_MATMUL_REDUCESCATTER 1
#define TPF_OP_ALLGATHER_MATMUL 2
#define TPF_OP_MATMUL_DX 3
#define TPF_OP_MLP_SP 4

typedef struct tpf_context* tpf_handle;

/* Create a handle bound to HIP device `device`.  The handle owns two side
 * streams (default priority), a pool of events, a small device control block
 * (counters, status word) and 512 KiB of per-output-tile counters; these are
 * allocated here and released by tpf_destroy.  Returns TPF_ERR_HIP if the
 * device cannot be used. */
int tpf_create(tpf_handle* h, int device);

/* Release a handle.  The caller must first let every call made with it
 * finish (for instance by synchronising the streams it passed); the call
 * itself synchronises only the handle's own side streams, never the whole
 * device.  NULL is accepted. */
int tpf_destroy(tpf_handle h);

/* Bytes of workspace a call needs (0 if none), a pure function of its
 * arguments.  For the reducing operations it is p * M * N * 4 (p * M * N * 2
 * with TPF_MSG_BF16 in `sched`): one local output [M, N] per shard (N = output
 * width: N for the row-parallel ops, K_in for tpf_matmul_dx), except that
 * TPF_SCHED_STATIONARY needs none for the row-parallel calls and the MLP
 * block, nor for tpf_matmul_dx with M > 64 (with M <= 64 it runs dX unfused
 * and needs the full size).  AUTO asks for the full size, which covers every
 * scheduler it may pick.  `K` is the per-shard reduction length.  AllGather->MatMul needs
 * none.  Returns 0 for invalid arguments. */
size_t tpf_workspace_size(int op, int p, int64_t M, int64_t N, int64_t K, int n_chunks, int sched);

/* MatMul -> AllReduce (row-parallel Linear, M027 page §01-§03; cnblogs §2.4).
 *   X[k]: [M, K_shard] bf16, W[k]: [K_shard, N] bf16, k = 0..p-1.
 *   Y:    [M, N], y_dtype (TPF_BF16 or TPF_F32).
 *   Y = sum_{k=0}^{p-1} X[k] W[k], summed in fp32 in shard order, rounded once.
 *   n_chunks in [1, min(M, TPF_MAX_CHUNKS)]: chunk c covers rows
 *   [c*floor(M/n), (c+1)*floor(M/n)), the last chunk also takes the remainder.
 *   ws/ws_bytes: at least tpf_workspace_size(TPF_OP_MATMUL_ALLREDUCE, ...). */
int tpf_matmul_allreduce(tpf_handle h, int p, int64_t M, int64_t N, int64_t K_shard,
                         const void* const* X, const void* const* W, void* Y, int y_dtype,
                         int n_chunks, int sched, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static workspace behind tpf_matmul_allreduce_noalloc (64 MiB
 * per device). */
#define TPF_NOALLOC_SCRATCH_BYTES (64u << 20)

/* MatMul -> AllReduce that allocates nothing, for callers that cannot call
 * hipMalloc: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same operands, result, schedulers and errors as
 * tpf_matmul_allreduce, without the workspace arguments: the shard partials
 * go to a library-owned static device array of TPF_NOALLOC_SCRATCH_BYTES per
 * device (each GPU the library runs on holds it until the process ends; its
 * address is looked up when the first handle on that device is created).
 * A call whose scheduler needs more than that (tpf_workspace_size of the same
 * arguments) fails with TPF_ERR_UNSUPPORTED before anything is enqueued;
 * TPF_SCHED_STATIONARY needs none and runs at any size.  The
 * call makes no allocation of any kind.  Every call on one device shares that
 * device's array, which keeps the last call's partials: calls that overlap on
 * one device (other streams, other handles, other threads) race and must be
 * serialised by the caller. */
int tpf_matmul_allreduce_noalloc(tpf_handle h, int p, int64_t M, int64_t N, int64_t K_shard,
                                 const void* const* X, const void* const* W, void* Y, int y_dtype,
                                 int n_chunks, int sched, void* stream);

/* MatMul -> ReduceScatter (M027 page §01; cnblogs §2.7).
 *   Same operands as tpf_matmul_allreduce; M % p == 0.
 *   Y_slices[r] ([M/p, N], y_dtype), r = 0..p-1, receives rows
 *   [r*M/p, (r+1)*M/p) of sum_k X[k] W[k]. */
int tpf_matmul_reducescatter(tpf_handle h, int p, int64_t M, int64_t N, int64_t K_shard,
                             const void* const* X, const void* const* W, void* const* Y_slices,
                             int y_dtype, int n_chunks, int sched, void* ws, size_t ws_bytes,
                             void* stream);

/* AllGather -> MatMul (M027 page §01-§02; cnblogs §2.3, §2.6).
 *   X_slices[r]: [M/p, K] bf16 (sequence slices, r = 0..p-1), M % p == 0.
 *   W: [K, N_shard] bf16 (this rank's column shard).
 *   X_gathered: [M, K] bf16 output, the slices concatenated in rank order.
 *   Y: [M, N_shard] y_dtype output, Y = X_gathered W (no reduction).
 *   Chunk c's GEMM starts once every slice overlapping its rows has landed
 *   in X_gathered.  Needs no workspace (ws may be NULL). */
int tpf_allgather_matmul(tpf_handle h, int p, int64_t M, int64_t N_shard, int64_t K,
                         const void* const* X_slices, const void* W, void* X_gathered, void* Y,
                         int y_dtype, int n_chunks, int sched, void* ws, size_t ws_bytes,
                         void* stream);

/* Column-parallel backward input gradient (cnblogs §三, §6.1, §6.4).
 *   dY[k]: [M, N_shard] bf16, W[k]: [K_in, N_shard] bf16 (the forward's
 *   column shard, used transposed), k = 0..p-1.
 *   dX = sum_k dY[k] W[k]^T, summed in fp32 in shard order, rounded once.
 *   sem == TPF_ALLREDUCE:     dX[0] is one [M, K_in] buffer.
 *   sem == TPF_REDUCESCATTER: dX[r] ([M/p, K_in]) receives rows [r*M/p, (r+1)*M/p); M % p == 0.
 *   ws_bytes >= tpf_workspace_size(TPF_OP_MATMUL_DX, p, M, K_in, N_shard, ...). */
int tpf_matmul_dx(tpf_handle h, int sem, int p, int64_t M, int64_t K_in, int64_t N_shard,
                  const void* const* dY, const void* const* W, void* const* dX, int dx_dtype,
                  int n_chunks, int sched, void* ws, size_t ws_bytes, void* stream);

/* Weight gradients of the tensor-parallel Linear (cnblogs §三 / §四 backward:
 * each rank's weight gradient is a local GEMM, no communication).
 *   dW[k] = A[k]^T B[k], k = 0..p-1, summed over the M rows in fp32 and
 *   rounded once to dw_dtype (TPF_BF16 or TPF_F32):
 *   A[k]: [M, R] bf16, B[k]: [M, C] bf16, dW[k]: [R, C].
 *   Row-parallel layer (W_k [K_shard, N]): A[k] = X_k [M, K_shard] (the
 *   shard's input), B[k] = dY [M, N] (the full output gradient; pass the same
 *   pointer p times).  Column-parallel layer (W_k [K, N_shard]): A[k] = the
 *   gathered input X [M, K] (the same pointer p times, e.g. X_gathered of
 *   tpf_allgather_matmul), B[k] = dY_k [M, N_shard].
 *   R and C must be multiples of 8; no workspace; the kernel timed by
 *   tpf_debug_set_kernel_timing is this call's only launch. */
int tpf_weight_grad(tpf_handle h, int p, int64_t M, int64_t R, int64_t C, const void* const* A,
                    const void* const* B, void* const* dW, int dw_dtype, void* stream);

/* Input gradient of a row-parallel Linear (cnblogs §四 backward: with
 * Y = sum_k X_k W_k the output gradient dY reaches every rank whole, and each
 * rank's input gradient is a local GEMM, no communication).
 *   dX[k] = dY W[k]^T, k = 0..p-1, summed over the N columns in fp32 and
 *   rounded once to dx_dtype (TPF_BF16 or TPF_F32):
 *   dY: [M, N] bf16 (one tensor, read by every shard), W[k]: [K_shard, N]
 *   bf16 (the forward weights, used transposed), dX[k]: [M, K_shard].
 *   K_shard and N must be multiples of 8; no workspace; the kernel timed by
 *   tpf_debug_set_kernel_timing is this call's only launch. */
int tpf_rowpar_dx(tpf_handle h, int p, int64_t M, int64_t K_shard, int64_t N, const void* dY,
                  const void* const* W, void* const* dX, int dx_dtype, void* stream);

/* The MLP block under sequence parallelism (cnblogs §7.1 and §11.3: the
 * column-parallel FC1 and row-parallel FC2 need no communication between
 * them; with sequence parallelism the block's input is all-gathered and its
 * output reduce-scattered along the sequence).  For k = 0..p-1:
 *   X_gathered = [X_slices[0]; ...; X_slices[p-1]]           [S, Hd] bf16 (output)
 *   H[k]       = bf16(GeLU(X_gathered W1[k]))                [S, F] bf16 (output;
 *                GeLU = 0.5 x (1 + erf(x / sqrt 2)) on the fp32 product, one RNE rounding)
 *   Y_slices[r] = rows [r*S/p, (r+1)*S/p) of sum_k H[k] W2[k]   [S/p, Hd] y_dtype
 *   X_slices[r]: [S/p, Hd], W1[k]: [Hd, F] (column shard), W2[k]: [F, Hd] (row shard).
 * FC2 and its ReduceScatter run exactly as tpf_matmul_reducescatter with the
 * same `sched` (flags included) and workspace
 * (tpf_workspace_size(TPF_OP_MLP_SP, p, S, Hd, F, n_chunks, sched)); the gather
 * and FC1 run first.  S % p == 0; Hd and F multiples of 8. */
int tpf_mlp_sp(tpf_handle h, int p, int64_t S, int64_t Hd, int64_t F, const void* const* X_slices,
               const void* const* W1, const void* const* W2, void* X_gathered, void* const* H,
               void* const* Y_slices, int y_dtype, int n_chunks, int sched, void* ws, size_t ws_bytes,
               void* stream);

/* Wait for the handle's work on `stream` to finish and report whether a
 * bounded wait inside the persistent kernel gave up since the last query
 * (TPF_ERR_TIMEOUT; the outputs of that call are then undefined).  Clears
 * the flag.  Synchronises `stream`. */
int tpf_sync_status(tpf_handle h, void* stream);

/* Debug: bound the persistent kernel's waits to `spins` polls (0 restores
 * the default).  With `unreachable` != 0 every wait targets a count that is
 * never reached, so each wait ends by its bound: used to test the timeout
 * path without any kernel hanging. */
int tpf_debug_set_wait(tpf_handle h, int64_t spins, int unreachable);

/* Debug: perturb the timing of the producers that the readiness protocols
 * wait for, to stress them (the M027 page §04 asks for the ready events to be
 * checked).  With period > 0 (and sleeps > 0), every later call on this handle
 * makes each producer task whose index i satisfies mix(seed, i) % period == 0
 * (a fixed integer hash) execute `sleeps` times the longest single sleep
 * instruction (s_sleep 127; about 1 us each, measured) before it stores or
 * publishes its results: the GEMM
 * tiles of the persistent kernel (before they bump a chunk's ready counter),
 * its AllGather copy tasks (before they bump a slice's landed counter), the
 * tile scheduler's tiles (before they bump an output tile's counter) and the
 * plain shard-GEMM tiles (before they store their partials; the two-stream
 * and fold schedulers' producers).  Results must not change.  period = 0
 * turns it off.  Returns TPF_ERR_INVALID_ARG for period < 0 or sleeps outside
 * [0, 1024]. */
int tpf_debug_set_delay(tpf_handle h, uint32_t seed, int period, int sleeps);

/* Debug: record the persistent kernel's task timeline.  `events` is a
 * caller-owned device buffer of `max_events` 32-byte records
 *   { uint32 ticket; uint16 kind (0 GEMM tile, 1 reduce, 2 copy);
 *     uint16 chunk (or slice); uint16 workgroup; uint16 xcd;
 *     uint32 mid (for a GEMM tile that also reduced a slice of the previous
 *                 chunk: clock ticks from t_start to the end of its GEMM part);
 *     uint64 t_start; uint64 t_end }   (little-endian)
 * indexed by ticket, stamped with the GPU's constant 100 MHz clock.  Every
 * later persistent call on this handle writes the events of its first
 * max_events tickets; pass NULL / 0 to stop.  The buffer must stay valid
 * while such calls run. */
int tpf_debug_set_timeline(tpf_handle h, void* events, int max_events);

/* Debug: time each call's dominant kernel launch.  With enable != 0, every
 * later call on this handle records a pair of timing events around that
 * launch, on the stream it is launched on: the shard-GEMM kernel for
 * TPF_SCHED_UNFUSED and TPF_SCHED_GEMM_ONLY (and AUTO, which runs UNFUSED),
 * the reduction kernel for TPF_SCHED_REDUCE_ONLY, the single kernel of
 * TPF_SCHED_PERSISTENT and TPF_SCHED_TILE; TPF_SCHED_TWO_STREAM calls record
 * nothing.  The last 256 records are kept.  Enabling creates the handle's
 * events on first use; both enabling and disabling clear the records. */
int tpf_debug_set_kernel_timing(tpf_handle h, int enable);

/* Debug: wait for the recorded launches and write up to `max` of their
 * durations in milliseconds into `ms` (host array), oldest first.  Returns
 * the number written (>= 0) or a negative status; clears the records. */
int tpf_debug_kernel_times(tpf_handle h, float* ms, int max);

/* The scheduler (a TPF_SCHED_* value, with TPF_SCHED_AUTO resolved and
 * any fallback applied) that the last reducing or AllGather->MatMul call on
 * the handle ran, or -1 before the first; negative status for a NULL handle.
 * For measurement tools that must name the kernels a call ran. */
int tpf_debug_last_sched(tpf_handle h);

/* Static text for a status code. */
const char* tpf_status_string(int code);

/* Message of the last failing call on this thread ("" if none). */
const char* tpf_last_error(void);

/* TPF_VERSION of the built library. */
int tpf_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPFUSE_H */
