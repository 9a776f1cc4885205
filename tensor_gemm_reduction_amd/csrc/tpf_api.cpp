// C ABI of libtpfuse: argument checks, workspace sizing, handles and the three
// schedulers (persistent, two-stream, unfused) plus the measurement modes.
//
// Chunking follows the M027 page §02-§03: the output rows are cut into
// contiguous chunks processed in the same order everywhere; each chunk's
// reduction may start as soon as that chunk's shard GEMMs are done, while the
// GEMMs of later chunks continue.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "../../include/tpfuse.h"
#include "tpf_internal.hpp"
#include "tpf_stationary.hpp"

using namespace tpf;

static_assert(TPF_MAX_SHARDS == kMaxShards, "shard limit mismatch");
static_assert(TPF_MAX_CHUNKS == kMaxChunks, "chunk limit mismatch");

constexpr int kKernelTimes = 256;   // debug kernel-timing records held per handle

// Partial workspace of tpf_matmul_allreduce_noalloc: a file-scope device
// array, one copy per GPU the library runs on, held until the process ends.
// Host code never uses the array's name as an address (in host code it is a
// host-side stand-in); it uses the device address that hipGetSymbolAddress
// returns for the current device, fetched once per device when a handle is
// created on it (noalloc_scratch()).
static_assert(TPF_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[TPF_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// The two-stream scheduler's chunk reductions run on a grid capped at a
// quarter of the usual size (2 workgroups per CU): they then trickle beside
// the next chunks' GEMM tiles instead of taking every CU at once (measured
// 2-3 % faster for that scheduler on sp_rs and dx_bwd; a half or an eighth
// were slower).
constexpr int kSideReduceCuDiv = 4;

struct tpf_context {
  int device = 0;
  int num_cus = 0;
  hipStream_t side = nullptr;           // reductions (reducing ops) or gather copies (AllGather)
  hipStream_t gemm2 = nullptr;          // every other chunk's GEMM (two-stream scheduler)
  hipEvent_t ev_fork = nullptr, ev_join = nullptr, ev_join2 = nullptr;
  hipEvent_t ev_chunk[kMaxChunks] = {};
  hipEvent_t ev_slice[kMaxShards] = {};
  Ctrl* ctrl = nullptr;
  int* tile_cnt = nullptr;             // kTileCounters per-output-tile counters (tile scheduler)
  int64_t spin_limit = 0;
  int unreachable = 0;
  TimelineEvent* timeline = nullptr;   // caller-owned device buffer (debug)
  int timeline_cap = 0;
  // Debug kernel timing: a ring of timing-event pairs around each call's
  // dominant launch.
  bool ktime = false;
  hipEvent_t kt0[kKernelTimes] = {}, kt1[kKernelTimes] = {};
  int kt_next = 0;      // ring slot of the next record
  int kt_count = 0;     // records held (<= kKernelTimes)
  int last_sched = -1;  // scheduler the last call ran (AUTO resolved), -1 before any
  void* scratch = nullptr;  // this device's copy of the no-allocation workspace
  DelayArgs delay{};        // debug: timing perturbation of the producers (tpf_debug_set_delay)
};

namespace {

// Polls before a bounded wait gives up (polls back off to ~4K clocks each,
// so this is a few seconds: far beyond any legitimate wait).
constexpr int64_t kDefaultSpinLimit = (int64_t)1 << 21;

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TPF_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define TPF_HIP(call)                                  \
  do {                                                 \
    hipError_t e_ = (call);                            \
    if (e_ != hipSuccess) return hip_fail(e_, #call);  \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A scheduler id in the low byte, optionally OR-ed with TPF_MSG_BF16.
bool valid_sched(int s) {
  const int base = s & 0xff, flags = s & ~0xff;
  return base >= TPF_SCHED_AUTO && base <= TPF_SCHED_STATIONARY && (flags & ~TPF_MSG_BF16) == 0;
}
bool msg_bf16(int s) { return (s & TPF_MSG_BF16) != 0; }
bool valid_dtype(int d) { return d == TPF_BF16 || d == TPF_F32; }

int out_kind(int dtype) { return dtype == TPF_F32 ? OUT_F32 : OUT_BF16; }

// Tile configuration from the op's total row count only (never from the
// chunking): every configuration runs the same MFMA sequence per element, so
// the choice changes speed, not bits.
int pick_cfg(int64_t M) { return M <= 32 ? CFG_SMALL : M <= 64 ? CFG_MID : CFG_LARGE; }

// Common checks of sizes, chunking, dtype and scheduler.
int check_common(int p, int64_t M, int64_t N, int64_t K, int n_chunks, int dtype, int sched, bool need_div) {
  if (p < 1 || p > kMaxShards) return fail(TPF_ERR_SHAPE, "p must be in [1, " + std::to_string(kMaxShards) + "]");
  if (M <= 0 || N <= 0 || K <= 0) return fail(TPF_ERR_SHAPE, "M, N and K must be positive");
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(TPF_ERR_SHAPE, "M, N and K must fit in 31 bits");
  if (M * N > ((int64_t)1 << 40) || M * K > ((int64_t)1 << 40) || N * K > ((int64_t)1 << 40))
    return fail(TPF_ERR_SHAPE, "operand too large");
  if (need_div && M % p != 0) return fail(TPF_ERR_SHAPE, "M must be divisible by p for this layout");
  // Operands are addressed with 32-bit buffer offsets.
  const int64_t lim = ((int64_t)1 << 31) - 1;
  if (M * K * 2 > lim || N * K * 2 > lim || M * N * 4 > lim)
    return fail(TPF_ERR_UNSUPPORTED, "each operand and each shard's fp32 partial must be smaller than 2 GiB");
  if (n_chunks < 1 || n_chunks > kMaxChunks || n_chunks > M)
    return fail(TPF_ERR_SHAPE, "n_chunks must be in [1, min(M, " + std::to_string(kMaxChunks) + ")]");
  if (N % 8 != 0 || K % 8 != 0) return fail(TPF_ERR_ALIGNMENT, "N and K must be multiples of 8");
  if (!valid_dtype(dtype)) return fail(TPF_ERR_INVALID_ARG, "unknown output dtype");
  if (!valid_sched(sched)) return fail(TPF_ERR_INVALID_ARG, "unknown scheduler");
  return TPF_OK;
}

int check_ptrs(const void* const* arr, int count, const char* name) {
  if (!arr) return fail(TPF_ERR_INVALID_ARG, std::string(name) + " array is NULL");
  for (int i = 0; i < count; ++i) {
    if (!arr[i]) return fail(TPF_ERR_INVALID_ARG, std::string(name) + "[" + std::to_string(i) + "] is NULL");
    if (!aligned16(arr[i]))
      return fail(TPF_ERR_ALIGNMENT, std::string(name) + "[" + std::to_string(i) + "] is not 16-byte aligned");
  }
  return TPF_OK;
}

int check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(TPF_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned16(ptr)) return fail(TPF_ERR_ALIGNMENT, std::string(name) + " is not 16-byte aligned");
  return TPF_OK;
}

// Workspace of the reducing ops: one local output ("message") per shard,
// fp32 or (TPF_MSG_BF16) bf16.  The output-stationary scheduler keeps the
// partials on chip and needs none for weights stored [K][N] (the
// row-parallel calls); with weights used transposed (dX) it runs as
// TPF_SCHED_UNFUSED and needs the full workspace.
size_t partial_bytes(int p, int64_t M, int64_t N, int sched, bool weights_kn = false) {
  if ((sched & 0xff) == TPF_SCHED_STATIONARY && (weights_kn || pick_cfg(M) == CFG_LARGE)) return 0;
  return (size_t)p * (size_t)M * (size_t)N * (msg_bf16(sched) ? 2 : 4);
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return TPF_OK;
  if (!ws) return fail(TPF_ERR_WORKSPACE, "workspace is NULL but " + std::to_string(need) + " bytes are needed");
  if (!aligned16(ws)) return fail(TPF_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(TPF_ERR_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " + std::to_string(need));
  return TPF_OK;
}

int check_handle(tpf_handle h) {
  if (!h) return fail(TPF_ERR_INVALID_ARG, "handle is NULL");
  return TPF_OK;
}

// AUTO.  The M027 page makes fusion conditional: measure the whole GEMM and
// the whole collective separately first (§04), and expect chunking to slow
// the GEMM and decode shapes to lack chunkable work (§03, §05).  Here every
// shard lives on one GPU, so the "messages" travel through the same HBM and
// L2 as the GEMM's operands: overlapping a chunk's reduction with later
// chunks' GEMMs costs per-chunk cross-XCD release/acquire, smaller GEMM
// launches or weights re-read once per chunk, and on MI355X each of those
// costs more than the reduction it hides.  What does pay is folding the
// reduction into the last shard's GEMM epilogue (FOLD): no partial of that
// shard is written or read back, there is no separate reduction pass, and
// its epilogue's partial reads overlap other tiles' MFMA work.  But its
// second launch holds only one shard's tiles, so it pays only when splitting
// the tiles into p-1 shards' and one shard's launches costs no extra wave of
// workgroups (one resident large tile per CU): AUTO runs FOLD for reductions
// on the large tiles when
//   waves((p-1) T) + waves(T) == waves(p T),  T = one shard's output tiles,
// and UNFUSED otherwise.  Measured: FOLD 3-7 % faster than GEMM-then-reduce
// on the Llama down projection (T = 256: 3 + 1 = 4 waves), the
// sequence-parallel ReduceScatter (T = 1024: 28 + 4 = 32) and dX of the same
// kind of shapes (T = 256 and 512); 2-3 % slower on the MLP block's FC2 and
// on the GPT-3-shaped dX (T = 384: 11 + 2 = 13 > 12) and 1.8x slower on the
// 2-shard worked example (T = 8: 1 + 1 > 1).  Decode-shaped M (small tiles)
// runs UNFUSED.  AllGather->MatMul has no reduction and runs UNFUSED.  The
// chunked schedulers are chosen explicitly.
int resolve_sched(int sched, int n_chunks) {
  (void)n_chunks;
  return sched & 0xff;   // AUTO stays AUTO here; each op resolves it below
}

int auto_reduce_sched(int cfg, int bl, int p, int64_t M, int64_t N, int num_cus) {
  (void)bl;
  // Decode-shaped M runs GEMM-then-reduce: measured on the decode shapes
  // (p = 8, [16|64, 1024] x [1024, 8192]) the shard-GEMM kernel plus the
  // reduction (27.5 + 4 us) beat the output-stationary single launch
  // (42.6 us at M = 16, 66 us at M = 64), whose 32-column weight stream and
  // per-shard activation re-reads run well below the HBM rate.
  if (cfg != CFG_LARGE || num_cus <= 0) return TPF_SCHED_UNFUSED;
  const int64_t T = ((M + cfg_bm(cfg) - 1) / cfg_bm(cfg)) * ((N + cfg_bn(cfg) - 1) / cfg_bn(cfg));
  auto waves = [num_cus](int64_t tiles) { return (tiles + num_cus - 1) / num_cus; };
  return waves((p - 1) * T) + waves(T) == waves(p * T) ? TPF_SCHED_FOLD : TPF_SCHED_UNFUSED;
}

// A reducing op (row-parallel AR/RS, or dX with either semantic).
struct ReduceCall {
  int p, M, N, K;
  int bl;                       // B_KN (forward weights) or B_NK (dX: weights used transposed)
  const void* const* A;
  const void* const* B;
  ReduceOut ro;
  int n_chunks, sched;
  void* P;                      // partials: fp32, or bf16 when ro.pbf16
};

int set_device(tpf_handle h) {
  TPF_HIP(hipSetDevice(h->device));
  return TPF_OK;
}

// Debug kernel timing: record the start / stop event of the current call's
// dominant launch on the stream it is launched on.
int ktime_start(tpf_handle h, hipStream_t s) {
  if (h->ktime) TPF_HIP(hipEventRecord(h->kt0[h->kt_next], s));
  return TPF_OK;
}
int ktime_stop(tpf_handle h, hipStream_t s) {
  if (!h->ktime) return TPF_OK;
  TPF_HIP(hipEventRecord(h->kt1[h->kt_next], s));
  h->kt_next = (h->kt_next + 1) % kKernelTimes;
  h->kt_count = std::min(h->kt_count + 1, kKernelTimes);
  return TPF_OK;
}

#define TPF_TIMED(h, s, launch)      \
  do {                               \
    int st_ = ktime_start((h), (s)); \
    if (st_) return st_;             \
    TPF_HIP(launch);                 \
    st_ = ktime_stop((h), (s));      \
    if (st_) return st_;             \
  } while (0)

// The fold scheduler's two launches over output rows [row0, row1): shards
// 0..p-2 into their partials, then shard p-1, whose epilogue adds those
// partials and its own accumulator.
static hipError_t launch_fold(int cfg, int bl, const GemmOperands& g, const ReduceOut& ro, void* P, int64_t stride,
                              int p, int row0, int row1, int N, hipStream_t s) {
  if (p > 1) {
    GemmOperands g0 = g;
    g0.nshard = p - 1;
    const hipError_t e = launch_gemm_rows(cfg, bl, g0, row0, row1, s);
    if (e != hipSuccess) return e;
  }
  TileArgs a{};
  a.g = g;
  a.g.A[0] = g.A[p - 1];
  a.g.B[0] = g.B[p - 1];
  a.g.nshard = 1;
  a.ro = ro;
  a.P = P;
  a.p_stride = stride;
  a.p = p;
  a.row0 = row0;
  a.row1 = row1;
  a.tiles_m = (row1 - row0 + cfg_bm(cfg) - 1) / cfg_bm(cfg);
  a.tiles_n = (N + cfg_bn(cfg) - 1) / cfg_bn(cfg);
  a.tasks = a.tiles_m * a.tiles_n;
  return launch_tiles(cfg, bl, 2 + (ro.dtype == OUT_F32 ? 1 : 0) + 2 * ro.pbf16, a, s);
}

int run_reduce_call(tpf_handle h, const ReduceCall& rc, hipStream_t stream) {
  int st = set_device(h);
  if (st) return st;
  const int cfg = pick_cfg(rc.M);
  GemmOperands g{};
  for (int k = 0; k < rc.p; ++k) {
    g.A[k] = reinterpret_cast<const __bf16*>(rc.A[k]);
    g.B[k] = reinterpret_cast<const __bf16*>(rc.B[k]);
  }
  g.lda = rc.K;
  g.a_rows = rc.M;
  g.ldb = rc.bl == B_KN ? rc.N : rc.K;
  g.dst = rc.P;
  g.dst_shard_stride = (int64_t)rc.M * rc.N;
  g.ldd = rc.N;
  g.dst_dtype = rc.ro.pbf16 ? OUT_BF16 : OUT_F32;   // the message is rounded once, from the fp32 tile
  g.M = rc.M;
  g.N = rc.N;
  g.K = rc.K;
  g.b_rows = rc.bl == B_KN ? rc.K : rc.N;
  g.nshard = rc.p;
  g.delay = h->delay;
  ChunkGeom ch{rc.n_chunks, rc.M / rc.n_chunks, rc.M};
  const int64_t stride = (int64_t)rc.M * rc.N;

  // One shard's tiles of a small-M problem cannot fill the GPU: the fold
  // scheduler then runs as UNFUSED (the same bits either way).
  int sched = rc.sched == TPF_SCHED_AUTO ? auto_reduce_sched(cfg, rc.bl, rc.p, rc.M, rc.N, h->num_cus) : rc.sched;
  if (sched == TPF_SCHED_FOLD && cfg != CFG_LARGE) sched = TPF_SCHED_UNFUSED;
  // The single launch streams weights stored [K][N]; dX's transposed weights
  // run GEMM-then-reduce (the same bits).
  if (sched == TPF_SCHED_STATIONARY && rc.bl != B_KN && cfg != CFG_LARGE) sched = TPF_SCHED_UNFUSED;
  h->last_sched = sched;
  switch (sched) {
    case TPF_SCHED_GEMM_ONLY:
      TPF_TIMED(h, stream, launch_gemm_rows(cfg, rc.bl, g, 0, rc.M, stream));
      return TPF_OK;
    case TPF_SCHED_REDUCE_ONLY:
      TPF_TIMED(h, stream, launch_reduce_rows(rc.P, stride, rc.p, 0, rc.M, rc.N, rc.ro, h->num_cus, stream));
      return TPF_OK;
    case TPF_SCHED_UNFUSED:
      TPF_TIMED(h, stream, launch_gemm_rows(cfg, rc.bl, g, 0, rc.M, stream));
      TPF_HIP(launch_reduce_rows(rc.P, stride, rc.p, 0, rc.M, rc.N, rc.ro, h->num_cus, stream));
      return TPF_OK;
    case TPF_SCHED_TWO_STREAM: {
      if (cfg == CFG_LARGE) {
        // Large tiles: chunk c runs as the fold scheduler over its rows -- the
        // first p-1 shards' tiles into their partials, then the last shard's
        // tiles, whose epilogue folds the chunk's reduction -- on the
        // caller's stream (even c) or the handle's second GEMM stream (odd c).
        // Chunk c's reduction (the partial reads of its fold epilogue) thus
        // runs beside chunk c+1's GEMM tiles instead of after all of them.
        TPF_HIP(hipEventRecord(h->ev_fork, stream));
        TPF_HIP(hipStreamWaitEvent(h->gemm2, h->ev_fork, 0));
        for (int c = 0; c < ch.n; ++c) {
          hipStream_t gs = (c & 1) ? h->gemm2 : stream;
          TPF_HIP(launch_fold(cfg, rc.bl, g, rc.ro, rc.P, stride, rc.p, ch.row0(c), ch.row1(c), rc.N, gs));
        }
        TPF_HIP(hipEventRecord(h->ev_join2, h->gemm2));
        TPF_HIP(hipStreamWaitEvent(stream, h->ev_join2, 0));
        return TPF_OK;
      }
      // Decode-shaped tiles: chunk c's GEMM goes to the caller's stream (even
      // c) or the handle's second GEMM stream (odd c), so the next chunk's
      // tiles fill CUs while the current chunk's last tiles finish; chunk c's
      // reduction runs on the side stream after chunk c's event, concurrently
      // with the GEMMs of later chunks.
      TPF_HIP(hipEventRecord(h->ev_fork, stream));
      TPF_HIP(hipStreamWaitEvent(h->side, h->ev_fork, 0));
      TPF_HIP(hipStreamWaitEvent(h->gemm2, h->ev_fork, 0));
      for (int c = 0; c < ch.n; ++c) {
        hipStream_t gs = (c & 1) ? h->gemm2 : stream;
        TPF_HIP(launch_gemm_rows(cfg, rc.bl, g, ch.row0(c), ch.row1(c), gs));
        TPF_HIP(hipEventRecord(h->ev_chunk[c], gs));
        TPF_HIP(hipStreamWaitEvent(h->side, h->ev_chunk[c], 0));
        TPF_HIP(launch_reduce_rows(rc.P, stride, rc.p, ch.row0(c), ch.row1(c), rc.N, rc.ro,
                                   std::max(1, h->num_cus / kSideReduceCuDiv), h->side));
      }
      TPF_HIP(hipEventRecord(h->ev_join, h->side));
      TPF_HIP(hipEventRecord(h->ev_join2, h->gemm2));
      TPF_HIP(hipStreamWaitEvent(stream, h->ev_join, 0));
      TPF_HIP(hipStreamWaitEvent(stream, h->ev_join2, 0));
      return TPF_OK;
    }
    case TPF_SCHED_FOLD:
      TPF_TIMED(h, stream, launch_fold(cfg, rc.bl, g, rc.ro, rc.P, stride, rc.p, 0, rc.M, rc.N, stream));
      return TPF_OK;
    case TPF_SCHED_STATIONARY: {
      if (cfg == CFG_LARGE) {
        StatLargeArgs a{};
        a.g = g;
        a.ro = rc.ro;
        TPF_TIMED(h, stream, launch_stationary_large(rc.bl, a, stream));
        return TPF_OK;
      }
      StationaryArgs a{};
      for (int k = 0; k < rc.p; ++k) {
        a.A[k] = g.A[k];
        a.B[k] = g.B[k];
      }
      a.M = rc.M;
      a.N = rc.N;
      a.K = rc.K;
      a.p = rc.p;
      a.ro = rc.ro;
      TPF_TIMED(h, stream, launch_stationary(a, rc.ro.pbf16, rc.ro.dtype, stream));
      return TPF_OK;
    }
    case TPF_SCHED_TILE: {
      TileArgs a{};
      a.g = g;
      a.ro = rc.ro;
      a.P = rc.P;
      a.p_stride = stride;
      a.p = rc.p;
      a.row0 = 0;
      a.row1 = rc.M;
      a.tiles_m = (rc.M + cfg_bm(cfg) - 1) / cfg_bm(cfg);
      a.tiles_n = (rc.N + cfg_bn(cfg) - 1) / cfg_bn(cfg);
      if ((int64_t)a.tiles_m * a.tiles_n > kTileCounters)
        return fail(TPF_ERR_UNSUPPORTED, "the tile scheduler handles at most " + std::to_string(kTileCounters) +
                                             " output tiles");
      a.tasks = rc.p * a.tiles_m * a.tiles_n;
      a.cnt = h->tile_cnt;
      a.timeline = h->timeline;
      a.timeline_cap = h->timeline_cap;
      TPF_TIMED(h, stream, launch_tiles(cfg, rc.bl, 1, a, stream));
      return TPF_OK;
    }
    case TPF_SCHED_PERSISTENT: {
      FusedArgs a{};
      a.g = g;
      a.ro = rc.ro;
      a.P = rc.P;
      a.p_stride = stride;
      a.p = rc.p;
      // Reduce tasks small enough that one chunk's reduction spreads over
      // every resident workgroup (between 1 Ki and 8 Ki output elements, i.e.
      // 4 to 32 KiB of fp32 partials per shard).
      const int occ = fused_occupancy(cfg, rc.bl);
      const int64_t chunk_elems = (int64_t)(ch.row1(0) - ch.row0(0)) * rc.N;
      int64_t re = chunk_elems / ((int64_t)h->num_cus * occ);
      re = std::max<int64_t>(1024, std::min<int64_t>(8192, re));
      a.reduce_elems = (re + 255) / 256 * 256;
      a.gather = 0;
      a.ch = ch;
      a.ctrl = h->ctrl;
      a.spin_limit = h->spin_limit > 0 ? h->spin_limit : kDefaultSpinLimit;
      a.unreachable = h->unreachable;
      a.timeline = h->timeline;
      a.timeline_cap = h->timeline_cap;
      const int bm = cfg_bm(cfg), bn = cfg_bn(cfg);
      const int tiles_n = (rc.N + bn - 1) / bn;
      // Queue order: G0, G1, ..., G(n-1), R(n-1).  Each GEMM tile of chunk
      // c > 0 also reduces one slice of chunk c-1 once it is ready (all of
      // chunk c-1's tiles hold smaller tickets), so the reduction of chunk
      // c-1 runs spread over chunk c's GEMM; only the last chunk's
      // reduction has tasks of its own.
      a.piggyback = 1;
      int nseg = 0, t = 0;
      auto add_seg = [&](int kind, int idx, int count) {
        a.seg_start[nseg] = t;
        a.seg_info[nseg] = kind | (idx << 4);
        t += count;
        ++nseg;
      };
      auto gemm_count = [&](int c) { return rc.p * ((ch.row1(c) - ch.row0(c) + bm - 1) / bm) * tiles_n; };
      auto red_count = [&](int c) {
        const int64_t e = (int64_t)(ch.row1(c) - ch.row0(c)) * rc.N;
        return (int)((e + a.reduce_elems - 1) / a.reduce_elems);
      };
      for (int c = 0; c < ch.n; ++c) a.gemm_tasks[c] = gemm_count(c);
      for (int c = 0; c < ch.n; ++c) add_seg(TK_GEMM, c, gemm_count(c));
      add_seg(TK_REDUCE, ch.n - 1, red_count(ch.n - 1));
      a.nseg = nseg;
      a.seg_start[nseg] = t;
      const int grid = std::min(t, h->num_cus * fused_occupancy(cfg, rc.bl));
      TPF_TIMED(h, stream, launch_fused(cfg, rc.bl, a, grid, stream));
      return TPF_OK;
    }
  }
  return fail(TPF_ERR_INVALID_ARG, "unknown scheduler");
}

}  // namespace

extern "C" {

int tpf_version(void) { return TPF_VERSION; }

const char* tpf_last_error(void) { return g_last_error.c_str(); }

const char* tpf_status_string(int code) {
  switch (code) {
    case TPF_OK: return "success";
    case TPF_ERR_INVALID_ARG: return "invalid argument";
    case TPF_ERR_SHAPE: return "invalid shape";
    case TPF_ERR_ALIGNMENT: return "misaligned pointer or size";
    case TPF_ERR_WORKSPACE: return "workspace missing or too small";
    case TPF_ERR_UNSUPPORTED: return "unsupported request";
    case TPF_ERR_HIP: return "HIP runtime error";
    case TPF_ERR_TIMEOUT: return "bounded wait timed out";
    default: return "unknown status";
  }
}

int tpf_create(tpf_handle* out, int device) {
  if (!out) return fail(TPF_ERR_INVALID_ARG, "handle pointer is NULL");
  *out = nullptr;
  int count = 0;
  TPF_HIP(hipGetDeviceCount(&count));
  if (device < 0 || device >= count) return fail(TPF_ERR_INVALID_ARG, "no such device");
  tpf_context* h = new (std::nothrow) tpf_context();
  if (!h) return fail(TPF_ERR_INVALID_ARG, "out of host memory");
  h->device = device;
  auto cleanup = [&](int code) {
    tpf_destroy(h);
    return code;
  };
  hipError_t e = hipSetDevice(device);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipSetDevice"));
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipGetDeviceProperties"));
  h->num_cus = prop.multiProcessorCount;
  // The no-allocation entry point's workspace: this device's copy of the
  // static array, looked up once per device with the device current.
  if (device < kMaxDevices) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
      void* ptr = nullptr;
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return cleanup(hip_fail(e, "hipGetSymbolAddress(scratch)"));
      g_scratch_ptr[device] = ptr;
    }
    h->scratch = g_scratch_ptr[device];
  }
  e = hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&h->gemm2, hipStreamNonBlocking);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipStreamCreateWithFlags"));
  e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_join, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_join2, hipEventDisableTiming);
  for (int c = 0; c < kMaxChunks && e == hipSuccess; ++c) e = hipEventCreateWithFlags(&h->ev_chunk[c], hipEventDisableTiming);
  for (int s = 0; s < kMaxShards && e == hipSuccess; ++s) e = hipEventCreateWithFlags(&h->ev_slice[s], hipEventDisableTiming);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipEventCreateWithFlags"));
  e = hipMalloc(reinterpret_cast<void**>(&h->ctrl), sizeof(Ctrl));
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(control block)"));
  e = hipMalloc(reinterpret_cast<void**>(&h->tile_cnt), sizeof(int) * kTileCounters);
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipMalloc(tile counters)"));
  e = hipMemset(h->ctrl, 0, sizeof(Ctrl));
  if (e == hipSuccess) e = hipMemset(h->tile_cnt, 0, sizeof(int) * kTileCounters);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return cleanup(hip_fail(e, "hipMemset(control block)"));
  *out = h;
  return TPF_OK;
}

int tpf_destroy(tpf_handle h) {
  if (!h) return TPF_OK;
  (void)hipSetDevice(h->device);
  // The caller has let every call made with this handle finish (the
  // handle's contract); only the handle's own side streams are drained here,
  // so destroying one handle does not stall other work on the device.
  if (h->side) (void)hipStreamSynchronize(h->side);
  if (h->gemm2) (void)hipStreamSynchronize(h->gemm2);
  if (h->ctrl) (void)hipFree(h->ctrl);
  if (h->tile_cnt) (void)hipFree(h->tile_cnt);
  for (auto& ev : h->ev_chunk)
    if (ev) (void)hipEventDestroy(ev);
  for (auto& ev : h->ev_slice)
    if (ev) (void)hipEventDestroy(ev);
  for (int i = 0; i < kKernelTimes; ++i) {
    if (h->kt0[i]) (void)hipEventDestroy(h->kt0[i]);
    if (h->kt1[i]) (void)hipEventDestroy(h->kt1[i]);
  }
  if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
  if (h->ev_join) (void)hipEventDestroy(h->ev_join);
  if (h->ev_join2) (void)hipEventDestroy(h->ev_join2);
  if (h->side) (void)hipStreamDestroy(h->side);
  if (h->gemm2) (void)hipStreamDestroy(h->gemm2);
  delete h;
  return TPF_OK;
}

size_t tpf_workspace_size(int op, int p, int64_t M, int64_t N, int64_t K, int n_chunks, int sched) {
  const bool div = op == TPF_OP_MATMUL_REDUCESCATTER || op == TPF_OP_ALLGATHER_MATMUL || op == TPF_OP_MLP_SP;
  std::string saved = g_last_error;
  int st = check_common(p, M, N, K, n_chunks, TPF_BF16, sched, div);
  g_last_error = saved;
  if (st != TPF_OK) return 0;
  switch (op) {
    case TPF_OP_MATMUL_ALLREDUCE:
    case TPF_OP_MATMUL_REDUCESCATTER:
    case TPF_OP_MLP_SP:          // FC2's partials: N = Hd
      return partial_bytes(p, M, N, sched, true);
    case TPF_OP_MATMUL_DX:
      return partial_bytes(p, M, N, sched, false);
    case TPF_OP_ALLGATHER_MATMUL:
      return 0;
    default:
      return 0;
  }
}

int tpf_matmul_allreduce(tpf_handle h, int p, int64_t M, int64_t N, int64_t K_shard, const void* const* X,
                         const void* const* W, void* Y, int y_dtype, int n_chunks, int sched, void* ws,
                         size_t ws_bytes, void* stream) {
  int st = check_common(p, M, N, K_shard, n_chunks, y_dtype, sched, false);
  if (st) return st;
  if ((st = check_ptrs(X, p, "X"))) return st;
  if ((st = check_ptrs(W, p, "W"))) return st;
  if ((st = check_ptr(Y, "Y"))) return st;
  if ((st = check_ws(ws, ws_bytes, partial_bytes(p, M, N, sched, true)))) return st;
  if ((st = check_handle(h))) return st;
  ReduceCall rc{};
  rc.p = p;
  rc.M = (int)M;
  rc.N = (int)N;
  rc.K = (int)K_shard;
  rc.bl = B_KN;
  rc.A = X;
  rc.B = W;
  rc.ro.y[0] = Y;
  rc.ro.scatter = 0;
  rc.ro.rows_per_slice = (int)M;
  rc.ro.dtype = out_kind(y_dtype);
  rc.n_chunks = n_chunks;
  rc.sched = resolve_sched(sched, n_chunks);
  rc.ro.pbf16 = msg_bf16(sched) ? 1 : 0;
  rc.P = ws;
  return run_reduce_call(h, rc, reinterpret_cast<hipStream_t>(stream));
}

int tpf_matmul_allreduce_noalloc(tpf_handle h, int p, int64_t M, int64_t N, int64_t K_shard, const void* const* X,
                                 const void* const* W, void* Y, int y_dtype, int n_chunks, int sched, void* stream) {
  int st = check_common(p, M, N, K_shard, n_chunks, y_dtype, sched, false);
  if (st) return st;
  if ((st = check_ptrs(X, p, "X"))) return st;
  if ((st = check_ptrs(W, p, "W"))) return st;
  if ((st = check_ptr(Y, "Y"))) return st;
  const size_t need = partial_bytes(p, M, N, sched, true);
  if (need > (size_t)TPF_NOALLOC_SCRATCH_BYTES)
    return fail(TPF_ERR_UNSUPPORTED, "the partials need " + std::to_string(need) + " bytes; the no-allocation entry "
                                     "point holds at most " + std::to_string((size_t)TPF_NOALLOC_SCRATCH_BYTES));
  if ((st = check_handle(h))) return st;
  if (!h->scratch) return fail(TPF_ERR_UNSUPPORTED, "no static workspace on this device");
  ReduceCall rc{};
  rc.p = p;
  rc.M = (int)M;
  rc.N = (int)N;
  rc.K = (int)K_shard;
  rc.bl = B_KN;
  rc.A = X;
  rc.B = W;
  rc.ro.y[0] = Y;
  rc.ro.scatter = 0;
  rc.ro.rows_per_slice = (int)M;
  rc.ro.dtype = out_kind(y_dtype);
  rc.n_chunks = n_chunks;
  rc.sched = resolve_sched(sched, n_chunks);
  rc.ro.pbf16 = msg_bf16(sched) ? 1 : 0;
  rc.P = h->scratch;
  return run_reduce_call(h, rc, reinterpret_cast<hipStream_t>(stream));
}

int tpf_matmul_reducescatter(tpf_handle h, int p, int64_t M, int64_t N, int64_t K_shard, const void* const* X,
                             const void* const* W, void* const* Y_slices, int y_dtype, int n_chunks, int sched,
                             void* ws, size_t ws_bytes, void* stream) {
  int st = check_common(p, M, N, K_shard, n_chunks, y_dtype, sched, true);
  if (st) return st;
  if ((st = check_ptrs(X, p, "X"))) return st;
  if ((st = check_ptrs(W, p, "W"))) return st;
  if ((st = check_ptrs(Y_slices, p, "Y_slices"))) return st;
  if ((st = check_ws(ws, ws_bytes, partial_bytes(p, M, N, sched, true)))) return st;
  if ((st = check_handle(h))) return st;
  ReduceCall rc{};
  rc.p = p;
  rc.M = (int)M;
  rc.N = (int)N;
  rc.K = (int)K_shard;
  rc.bl = B_KN;
  rc.A = X;
  rc.B = W;
  for (int r = 0; r < p; ++r) rc.ro.y[r] = Y_slices[r];
  rc.ro.scatter = 1;
  rc.ro.rows_per_slice = (int)(M / p);
  rc.ro.dtype = out_kind(y_dtype);
  rc.n_chunks = n_chunks;
  rc.sched = resolve_sched(sched, n_chunks);
  rc.ro.pbf16 = msg_bf16(sched) ? 1 : 0;
  rc.P = ws;
  return run_reduce_call(h, rc, reinterpret_cast<hipStream_t>(stream));
}

int tpf_matmul_dx(tpf_handle h, int sem, int p, int64_t M, int64_t K_in, int64_t N_shard, const void* const* dY,
                  const void* const* W, void* const* dX, int dx_dtype, int n_chunks, int sched, void* ws,
                  size_t ws_bytes, void* stream) {
  if (sem != TPF_ALLREDUCE && sem != TPF_REDUCESCATTER) return fail(TPF_ERR_INVALID_ARG, "unknown semantic");
  const bool rs = sem == TPF_REDUCESCATTER;
  int st = check_common(p, M, K_in, N_shard, n_chunks, dx_dtype, sched, rs);
  if (st) return st;
  if ((st = check_ptrs(dY, p, "dY"))) return st;
  if ((st = check_ptrs(W, p, "W"))) return st;
  if ((st = check_ptrs(dX, rs ? p : 1, "dX"))) return st;
  if ((st = check_ws(ws, ws_bytes, partial_bytes(p, M, K_in, sched)))) return st;
  if ((st = check_handle(h))) return st;
  ReduceCall rc{};
  rc.p = p;
  rc.M = (int)M;
  rc.N = (int)K_in;        // output width
  rc.K = (int)N_shard;     // reduction length per shard
  rc.bl = B_NK;
  rc.A = dY;
  rc.B = W;
  for (int r = 0; r < (rs ? p : 1); ++r) rc.ro.y[r] = dX[r];
  rc.ro.scatter = rs ? 1 : 0;
  rc.ro.rows_per_slice = rs ? (int)(M / p) : (int)M;
  rc.ro.dtype = out_kind(dx_dtype);
  rc.n_chunks = n_chunks;
  rc.sched = resolve_sched(sched, n_chunks);
  rc.ro.pbf16 = msg_bf16(sched) ? 1 : 0;
  rc.P = ws;
  return run_reduce_call(h, rc, reinterpret_cast<hipStream_t>(stream));
}

int tpf_allgather_matmul(tpf_handle h, int p, int64_t M, int64_t N_shard, int64_t K, const void* const* X_slices,
                         const void* W, void* X_gathered, void* Y, int y_dtype, int n_chunks, int sched, void* ws,
                         size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int st = check_common(p, M, N_shard, K, n_chunks, y_dtype, sched, true);
  if (st) return st;
  if ((st = check_ptrs(X_slices, p, "X_slices"))) return st;
  if ((st = check_ptr(W, "W"))) return st;
  if ((st = check_ptr(X_gathered, "X_gathered"))) return st;
  if ((st = check_ptr(Y, "Y"))) return st;
  if ((st = check_handle(h))) return st;
  if ((st = set_device(h))) return st;
  hipStream_t stream_ = reinterpret_cast<hipStream_t>(stream);
  const int Mi = (int)M, Ni = (int)N_shard, Ki = (int)K;
  const int cfg = pick_cfg(M);
  GemmOperands g{};
  g.A[0] = reinterpret_cast<const __bf16*>(X_gathered);
  g.B[0] = reinterpret_cast<const __bf16*>(W);
  g.lda = Ki;
  g.a_rows = Mi;
  g.ldb = Ni;
  g.dst = Y;
  g.dst_shard_stride = 0;
  g.ldd = Ni;
  g.dst_dtype = out_kind(y_dtype);
  g.M = Mi;
  g.N = Ni;
  g.K = Ki;
  g.b_rows = Ki;
  g.nshard = 1;
  g.delay = h->delay;
  const int slice_rows = Mi / p;
  const int64_t slice_bytes = (int64_t)slice_rows * Ki * 2;
  char* xg = reinterpret_cast<char*>(X_gathered);
  ChunkGeom ch{n_chunks, Mi / n_chunks, Mi};
  int s = resolve_sched(sched, n_chunks);
  if (s == TPF_SCHED_TILE) s = TPF_SCHED_PERSISTENT;   // no reduction to fold into the tiles
  if (s == TPF_SCHED_FOLD || s == TPF_SCHED_STATIONARY || s == TPF_SCHED_AUTO) s = TPF_SCHED_UNFUSED;
  h->last_sched = s;
  switch (s) {
    case TPF_SCHED_GEMM_ONLY:
      TPF_TIMED(h, stream_, launch_gemm_rows(cfg, B_KN, g, 0, Mi, stream_));
      return TPF_OK;
    case TPF_SCHED_REDUCE_ONLY:
      TPF_HIP(launch_gather(X_slices, p, xg, slice_bytes, h->num_cus, stream_));
      return TPF_OK;
    case TPF_SCHED_UNFUSED:
      TPF_HIP(launch_gather(X_slices, p, xg, slice_bytes, h->num_cus, stream_));
      TPF_TIMED(h, stream_, launch_gemm_rows(cfg, B_KN, g, 0, Mi, stream_));
      return TPF_OK;
    case TPF_SCHED_TWO_STREAM: {
      // Slices are copied on the side stream in rank order; chunk c's GEMM
      // waits for the last slice under its rows, alternating between the
      // caller's stream and the handle's second GEMM stream as above.
      TPF_HIP(hipEventRecord(h->ev_fork, stream_));
      TPF_HIP(hipStreamWaitEvent(h->side, h->ev_fork, 0));
      TPF_HIP(hipStreamWaitEvent(h->gemm2, h->ev_fork, 0));
      for (int r = 0; r < p; ++r) {
        TPF_HIP(launch_copy(reinterpret_cast<const char*>(X_slices[r]), xg + r * slice_bytes, slice_bytes, h->num_cus,
                            h->side));
        TPF_HIP(hipEventRecord(h->ev_slice[r], h->side));
      }
      for (int c = 0; c < ch.n; ++c) {
        hipStream_t gs = (c & 1) ? h->gemm2 : stream_;
        TPF_HIP(hipStreamWaitEvent(gs, h->ev_slice[(ch.row1(c) - 1) / slice_rows], 0));
        TPF_HIP(launch_gemm_rows(cfg, B_KN, g, ch.row0(c), ch.row1(c), gs));
      }
      TPF_HIP(hipEventRecord(h->ev_join, h->side));
      TPF_HIP(hipEventRecord(h->ev_join2, h->gemm2));
      TPF_HIP(hipStreamWaitEvent(stream_, h->ev_join, 0));
      TPF_HIP(hipStreamWaitEvent(stream_, h->ev_join2, 0));
      return TPF_OK;
    }
    case TPF_SCHED_PERSISTENT: {
      FusedArgs a{};
      a.g = g;
      a.p = 1;
      a.gather = 1;
      for (int r = 0; r < p; ++r) a.src[r] = reinterpret_cast<const char*>(X_slices[r]);
      a.gathered = xg;
      a.slice_bytes = slice_bytes;
      a.slice_rows = slice_rows;
      // Copy tasks of 256 KiB (rounded to 16 bytes).
      const int64_t seg = std::min<int64_t>(slice_bytes, (int64_t)256 * 1024);
      a.copy_seg_bytes = (seg + 15) / 16 * 16;
      a.copy_segs = (int)((slice_bytes + a.copy_seg_bytes - 1) / a.copy_seg_bytes);
      a.ch = ch;
      a.ctrl = h->ctrl;
      a.spin_limit = h->spin_limit > 0 ? h->spin_limit : kDefaultSpinLimit;
      a.unreachable = h->unreachable;
      a.timeline = h->timeline;
      a.timeline_cap = h->timeline_cap;
      const int bm = cfg_bm(cfg), bn = cfg_bn(cfg);
      const int tiles_n = (Ni + bn - 1) / bn;
      int nseg = 0, t = 0;
      auto add_seg = [&](int kind, int idx, int count) {
        a.seg_start[nseg] = t;
        a.seg_info[nseg] = kind | (idx << 4);
        t += count;
        ++nseg;
      };
      // Copies of the slices under chunk c+1 are queued before chunk c's
      // GEMM tiles, so the next transfer overlaps the current GEMM.
      int copied = -1;
      auto copy_upto = [&](int slice) {
        while (copied < slice) {
          ++copied;
          add_seg(TK_COPY, copied, a.copy_segs);
        }
      };
      copy_upto((ch.row1(0) - 1) / slice_rows);
      for (int c = 0; c < ch.n; ++c) {
        if (c + 1 < ch.n) copy_upto((ch.row1(c + 1) - 1) / slice_rows);
        const int cnt = ((ch.row1(c) - ch.row0(c) + bm - 1) / bm) * tiles_n;
        a.gemm_tasks[c] = cnt;
        add_seg(TK_GEMM, c, cnt);
      }
      copy_upto(p - 1);
      a.nseg = nseg;
      a.seg_start[nseg] = t;
      const int grid = std::min(t, h->num_cus * fused_occupancy(cfg, B_KN));
      TPF_TIMED(h, stream_, launch_fused(cfg, B_KN, a, grid, stream_));
      return TPF_OK;
    }
  }
  return fail(TPF_ERR_INVALID_ARG, "unknown scheduler");
}

int tpf_weight_grad(tpf_handle h, int p, int64_t M, int64_t R, int64_t C, const void* const* A,
                    const void* const* B, void* const* dW, int dw_dtype, void* stream) {
  if (p < 1 || p > kMaxShards) return fail(TPF_ERR_SHAPE, "p must be in [1, " + std::to_string(kMaxShards) + "]");
  if (M <= 0 || R <= 0 || C <= 0) return fail(TPF_ERR_SHAPE, "M, R and C must be positive");
  if (M > INT32_MAX || R > INT32_MAX || C > INT32_MAX) return fail(TPF_ERR_SHAPE, "M, R and C must fit in 31 bits");
  if (R % 8 != 0 || C % 8 != 0) return fail(TPF_ERR_ALIGNMENT, "R and C must be multiples of 8");
  const int64_t lim = ((int64_t)1 << 31) - 1;
  if (M * R * 2 > lim || M * C * 2 > lim || R * C * 4 > lim)
    return fail(TPF_ERR_UNSUPPORTED, "each operand and each output must be smaller than 2 GiB");
  if (!valid_dtype(dw_dtype)) return fail(TPF_ERR_INVALID_ARG, "unknown output dtype");
  int st;
  if ((st = check_ptrs(A, p, "A"))) return st;
  if ((st = check_ptrs(B, p, "B"))) return st;
  if ((st = check_ptrs(const_cast<const void* const*>(dW), p, "dW"))) return st;
  if ((st = check_handle(h))) return st;
  if ((st = set_device(h))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // dW[k] [R, C] = A[k]^T B[k]: output rows index A's columns, the contraction
  // runs over the M rows of both operands (A stored [M][R]: transposed-A
  // tiles; B stored [M][C]: KN tiles).
  GemmOperands g{};
  for (int k = 0; k < p; ++k) {
    g.A[k] = reinterpret_cast<const __bf16*>(A[k]);
    g.B[k] = reinterpret_cast<const __bf16*>(B[k]);
    g.dstv[k] = dW[k];
  }
  g.lda = R;
  g.a_rows = (int)M;
  g.ldb = C;
  g.b_rows = (int)M;
  g.ldd = C;
  g.dst_dtype = out_kind(dw_dtype);
  g.M = (int)R;
  g.N = (int)C;
  g.K = (int)M;
  g.nshard = p;
  TPF_TIMED(h, s, launch_gemm_rows(CFG_LARGE, A_KM | B_KN, g, 0, (int)R, s));
  return TPF_OK;
}

int tpf_rowpar_dx(tpf_handle h, int p, int64_t M, int64_t K_shard, int64_t N, const void* dY,
                  const void* const* W, void* const* dX, int dx_dtype, void* stream) {
  if (p < 1 || p > kMaxShards) return fail(TPF_ERR_SHAPE, "p must be in [1, " + std::to_string(kMaxShards) + "]");
  if (M <= 0 || K_shard <= 0 || N <= 0) return fail(TPF_ERR_SHAPE, "M, K_shard and N must be positive");
  if (M > INT32_MAX || K_shard > INT32_MAX || N > INT32_MAX)
    return fail(TPF_ERR_SHAPE, "M, K_shard and N must fit in 31 bits");
  if (K_shard % 8 != 0 || N % 8 != 0) return fail(TPF_ERR_ALIGNMENT, "K_shard and N must be multiples of 8");
  const int64_t lim = ((int64_t)1 << 31) - 1;
  if (M * N * 2 > lim || K_shard * N * 2 > lim || M * K_shard * 4 > lim)
    return fail(TPF_ERR_UNSUPPORTED, "each operand and each output must be smaller than 2 GiB");
  if (!valid_dtype(dx_dtype)) return fail(TPF_ERR_INVALID_ARG, "unknown output dtype");
  int st;
  if ((st = check_ptr(dY, "dY"))) return st;
  if ((st = check_ptrs(W, p, "W"))) return st;
  if ((st = check_ptrs(const_cast<const void* const*>(dX), p, "dX"))) return st;
  if ((st = check_handle(h))) return st;
  if ((st = set_device(h))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // dX[k] [M, K_shard] = dY W[k]^T: every shard reads the same dY [M][N]; the
  // weights stay in their forward layout [K_shard][N] and are used
  // transposed (NK tiles, as in the column-parallel dX).
  GemmOperands g{};
  for (int k = 0; k < p; ++k) {
    g.A[k] = reinterpret_cast<const __bf16*>(dY);
    g.B[k] = reinterpret_cast<const __bf16*>(W[k]);
    g.dstv[k] = dX[k];
  }
  g.lda = N;
  g.a_rows = (int)M;
  g.ldb = N;
  g.b_rows = (int)K_shard;
  g.ldd = K_shard;
  g.dst_dtype = out_kind(dx_dtype);
  g.M = (int)M;
  g.N = (int)K_shard;
  g.K = (int)N;
  g.nshard = p;
  TPF_TIMED(h, s, launch_gemm_rows(pick_cfg(M), B_NK, g, 0, (int)M, s));
  return TPF_OK;
}

int tpf_mlp_sp(tpf_handle h, int p, int64_t S, int64_t Hd, int64_t F, const void* const* X_slices,
               const void* const* W1, const void* const* W2, void* X_gathered, void* const* H,
               void* const* Y_slices, int y_dtype, int n_chunks, int sched, void* ws, size_t ws_bytes,
               void* stream) {
  // FC1's shapes ([S, Hd] x [Hd, F]) and FC2's ([S, F] x [F, Hd]) share the checks.
  int st = check_common(p, S, F, Hd, n_chunks, y_dtype, sched, true);
  if (st) return st;
  if ((st = check_common(p, S, Hd, F, n_chunks, y_dtype, sched, true))) return st;
  if ((st = check_ptrs(X_slices, p, "X_slices"))) return st;
  if ((st = check_ptrs(W1, p, "W1"))) return st;
  if ((st = check_ptrs(W2, p, "W2"))) return st;
  if ((st = check_ptr(X_gathered, "X_gathered"))) return st;
  if ((st = check_ptrs(const_cast<const void* const*>(H), p, "H"))) return st;
  if ((st = check_ptrs(const_cast<const void* const*>(Y_slices), p, "Y_slices"))) return st;
  if ((st = check_ws(ws, ws_bytes, partial_bytes(p, S, Hd, sched, true)))) return st;
  if ((st = check_handle(h))) return st;
  if ((st = set_device(h))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int Si = (int)S, Hi = (int)Hd, Fi = (int)F;
  // AllGather of the sequence slices in rank order.
  const int64_t slice_bytes = (int64_t)(Si / p) * Hi * 2;
  char* xg = reinterpret_cast<char*>(X_gathered);
  TPF_HIP(launch_gather(X_slices, p, xg, slice_bytes, h->num_cus, s));
  // FC1 on the column shards, GeLU in the epilogue, bf16 activations.
  GemmOperands g{};
  for (int k = 0; k < p; ++k) {
    g.A[k] = reinterpret_cast<const __bf16*>(X_gathered);
    g.B[k] = reinterpret_cast<const __bf16*>(W1[k]);
    g.dstv[k] = H[k];
  }
  g.lda = Hi;
  g.a_rows = Si;
  g.ldb = Fi;
  g.b_rows = Hi;
  g.ldd = Fi;
  g.dst_dtype = OUT_BF16;
  g.act = 1;
  g.M = Si;
  g.N = Fi;
  g.K = Hi;
  g.nshard = p;
  TPF_HIP(launch_gemm_rows(pick_cfg(S), B_KN, g, 0, Si, s));
  // FC2 on the row shards and the ReduceScatter of the partial sums.
  ReduceCall rc{};
  rc.p = p;
  rc.M = Si;
  rc.N = Hi;
  rc.K = Fi;
  rc.bl = B_KN;
  rc.A = const_cast<const void* const*>(H);
  rc.B = W2;
  for (int r = 0; r < p; ++r) rc.ro.y[r] = Y_slices[r];
  rc.ro.scatter = 1;
  rc.ro.rows_per_slice = Si / p;
  rc.ro.dtype = out_kind(y_dtype);
  rc.ro.pbf16 = msg_bf16(sched) ? 1 : 0;
  rc.n_chunks = n_chunks;
  rc.sched = resolve_sched(sched, n_chunks);
  rc.P = ws;
  return run_reduce_call(h, rc, s);
}

int tpf_sync_status(tpf_handle h, void* stream) {
  int st = check_handle(h);
  if (st) return st;
  if ((st = set_device(h))) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int status = 0;
  TPF_HIP(hipStreamSynchronize(s));
  TPF_HIP(hipMemcpy(&status, &h->ctrl->status, sizeof(int), hipMemcpyDeviceToHost));
  if (status) {
    TPF_HIP(launch_clear_status(h->ctrl, s));
    TPF_HIP(hipStreamSynchronize(s));
    return fail(TPF_ERR_TIMEOUT, "a bounded wait in the persistent kernel gave up");
  }
  return TPF_OK;
}

int tpf_debug_set_timeline(tpf_handle h, void* events, int max_events) {
  int st = check_handle(h);
  if (st) return st;
  if (max_events < 0 || (max_events > 0 && !events)) return fail(TPF_ERR_INVALID_ARG, "bad timeline buffer");
  if (events && !aligned16(events)) return fail(TPF_ERR_ALIGNMENT, "timeline buffer is not 16-byte aligned");
  h->timeline = max_events > 0 ? reinterpret_cast<TimelineEvent*>(events) : nullptr;
  h->timeline_cap = max_events;
  return TPF_OK;
}

int tpf_debug_set_kernel_timing(tpf_handle h, int enable) {
  int st = check_handle(h);
  if (st) return st;
  if ((st = set_device(h))) return st;
  if (enable && !h->kt0[0]) {
    // Timing-only events: without the system-scope fence (a cache write-back
    // and invalidation when the event is reached) that a default event
    // performs, which would otherwise lengthen every timed launch by a few
    // microseconds.  They are only read for their timestamps.
    for (int i = 0; i < kKernelTimes; ++i) {
      TPF_HIP(hipEventCreateWithFlags(&h->kt0[i], hipEventDisableSystemFence));
      TPF_HIP(hipEventCreateWithFlags(&h->kt1[i], hipEventDisableSystemFence));
    }
  }
  h->ktime = enable != 0;
  h->kt_next = 0;
  h->kt_count = 0;
  return TPF_OK;
}

int tpf_debug_kernel_times(tpf_handle h, float* ms, int max) {
  int st = check_handle(h);
  if (st) return st;
  if (max < 0 || (max > 0 && !ms)) return fail(TPF_ERR_INVALID_ARG, "bad output array");
  if ((st = set_device(h))) return st;
  const int n = std::min(max, h->kt_count);
  const int first = (h->kt_next - h->kt_count + kKernelTimes) % kKernelTimes;
  for (int i = 0; i < n; ++i) {
    const int j = (first + i) % kKernelTimes;
    TPF_HIP(hipEventSynchronize(h->kt1[j]));
    TPF_HIP(hipEventElapsedTime(&ms[i], h->kt0[j], h->kt1[j]));
  }
  h->kt_next = 0;
  h->kt_count = 0;
  return n;
}

int tpf_debug_last_sched(tpf_handle h) {
  int st = check_handle(h);
  if (st) return st;
  return h->last_sched;
}

int tpf_debug_set_delay(tpf_handle h, uint32_t seed, int period, int sleeps) {
  if (period < 0 || sleeps < 0 || sleeps > 1024)
    return fail(TPF_ERR_INVALID_ARG, "period must be >= 0 and sleeps in [0, 1024]");
  int st = check_handle(h);
  if (st) return st;
  h->delay.seed = seed;
  h->delay.period = sleeps > 0 ? period : 0;
  h->delay.sleeps = sleeps;
  return TPF_OK;
}

int tpf_debug_set_wait(tpf_handle h, int64_t spins, int unreachable) {
  int st = check_handle(h);
  if (st) return st;
  if (spins < 0) return fail(TPF_ERR_INVALID_ARG, "spins must be >= 0");
  h->spin_limit = spins;
  h->unreachable = unreachable ? 1 : 0;
  return TPF_OK;
}

}  // extern "C"
