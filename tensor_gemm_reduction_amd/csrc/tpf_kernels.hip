// Kernels of the fused tensor-parallel Linear and their launchers.
//
//  tile_kernel       one workgroup per shard GEMM tile of a row range: the
//                    shard GEMMs of one chunk (two-stream scheduler) or of all
//                    rows (unfused baseline); with RED = 1 also the tile
//                    scheduler, whose last workgroup to finish an output tile
//                    sums it over the shards.
//  reduce_rows_kernel the fixed-order sum over shards of a row range, written
//                    in AllReduce or ReduceScatter layout.
//  fused_kernel      the persistent scheduler: every workgroup pulls tickets
//                    from one queue whose order interleaves the GEMM tiles of
//                    chunk c+1 with the reduction tasks of chunk c; a reduce
//                    task waits on chunk c's ready counter, which each GEMM
//                    tile of chunk c bumps after its partial is visible.  For
//                    AllGather->MatMul the queue holds gather-copy tasks
//                    instead, and a GEMM tile waits until the slices under its
//                    rows have landed.
//
// Deadlock freedom of fused_kernel: a task only ever waits for tasks with
// smaller tickets, and a ticket is handed out only to a workgroup that is
// already running, so every awaited task is owned by a running workgroup
// that does not itself wait on anything later.  This holds however many
// workgroups are resident.
#include <algorithm>

#include "tpf_internal.hpp"
#include "tpf_stationary.hpp"

// The launchers are split into parts so that the build can compile them as
// separate translation units in parallel (-DTPF_PART=n, n = 0..8); without
// TPF_PART every part is compiled.
//   0: reductions, copies, status, dispatch      1: persistent kernel, large tiles
//   2: large tiles (plain, tile scheduler)        3: fold epilogue, fp32 messages
//   4: decode-shaped (small and mid) tiles        5: persistent kernel, small and mid tiles
//   6: fold epilogue, bf16 messages               7: output-stationary single launch (decode)
//   8: output-stationary single launch (large tiles)
#ifdef TPF_PART
#define TPF_IN_PART(n) (TPF_PART == (n))
#else
#define TPF_IN_PART(n) 1
#endif

namespace tpf {

// Kernel arguments are read in place from the kernarg segment.  Indexing a
// by-value struct argument with a run-time index (a shard's pointer, a
// segment boundary) would otherwise make the compiler copy the whole struct
// into per-lane scratch memory.  Each kernel below takes exactly one
// argument, which therefore sits at offset 0 of the segment.
template <class T>
__device__ __forceinline__ const T& kernarg() {
  return *(const T*)__builtin_amdgcn_kernarg_segment_ptr();
}

#if TPF_IN_PART(0)
int cfg_bm(int cfg) { return cfg == CFG_SMALL ? CfgSmall::BM : cfg == CFG_MID ? CfgMid::BM : CfgLarge::BM; }
int cfg_bn(int cfg) { return cfg == CFG_SMALL ? CfgSmall::BN : cfg == CFG_MID ? CfgMid::BN : CfgLarge::BN; }
#endif

template <class Cfg>
__device__ __forceinline__ void store_any(const Frag<Cfg>& f, const TileJob& j, const GemmOperands& g, int shard) {
  if (g.act) {   // activation of the MLP block's FC1: GeLU, then bf16
    uint16_t* d = g.dstv[0] ? reinterpret_cast<uint16_t*>(g.dstv[shard])
                            : reinterpret_cast<uint16_t*>(g.dst) + (int64_t)shard * g.dst_shard_stride;
    store_tile<Cfg, OUT_BF16, 1>(f, j, d, g.ldd);
    return;
  }
  if (g.dst_dtype == OUT_F32) {
    float* d = g.dstv[0] ? reinterpret_cast<float*>(g.dstv[shard])
                         : reinterpret_cast<float*>(g.dst) + (int64_t)shard * g.dst_shard_stride;
    store_tile<Cfg, OUT_F32>(f, j, d, g.ldd);
  } else {
    uint16_t* d = g.dstv[0] ? reinterpret_cast<uint16_t*>(g.dstv[shard])
                            : reinterpret_cast<uint16_t*>(g.dst) + (int64_t)shard * g.dst_shard_stride;
    store_tile<Cfg, OUT_BF16>(f, j, d, g.ldd);
  }
}

template <class Cfg>
__device__ __forceinline__ TileJob make_job(const GemmOperands& g, int shard, int row0, int row1, int tm, int tn) {
  TileJob j;
  j.A = g.A[shard];
  j.B = g.B[shard];
  j.lda = g.lda;
  j.ldb = g.ldb;
  j.a_rows = g.a_rows;
  j.b_rows = g.b_rows;
  j.m0 = row0 + tm * Cfg::BM;
  j.rows = min(Cfg::BM, row1 - j.m0);
  j.n0 = tn * Cfg::BN;
  j.N = g.N;
  j.K = g.K;
  return j;
}

// Tile u of a row range (shard-major) -> (shard, tm, tn).  Within a shard the
// tiles go in groups of kGroupM tile-rows, column by column, so that tiles
// running at the same time share A and B panels (the 32 tiles an XCD runs
// at once cover 8 row panels x 4 column panels; measured about 1 % faster
// than groups of 4 rows, groups of 2 or 16 slower).
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_coords(int u, int tiles_m, int tiles_n, int& shard, int& tm, int& tn) {
  const int per_shard = tiles_m * tiles_n;
  shard = u / per_shard;
  const int t = u - shard * per_shard;
  const int group = t / (kGroupM * tiles_n);
  const int first = group * kGroupM;
  const int gsize = min(kGroupM, tiles_m - first);
  const int w = t - first * tiles_n;
  tm = first + w % gsize;
  tn = w / gsize;
}

template <int OUT, int PB>
__device__ __forceinline__ void reduce_dispatch_p(const void* P, int64_t stride, int p, int64_t e0, int64_t e1,
                                                  int N, const ReduceOut& o, int64_t t, int64_t nthr) {
  if constexpr (PB) {   // bf16 partials: 16-byte loads of eight elements
    switch (p) {
      case 2: reduce_range_b16<2, OUT>(P, stride, p, e0, e1, N, o, t, nthr); break;
      case 4: reduce_range_b16<4, OUT>(P, stride, p, e0, e1, N, o, t, nthr); break;
      case 8: reduce_range_b16<8, OUT>(P, stride, p, e0, e1, N, o, t, nthr); break;
      default: reduce_range_b16<0, OUT>(P, stride, p, e0, e1, N, o, t, nthr); break;
    }
  } else {
    switch (p) {
      case 2: reduce_range<2, OUT, 0>(P, stride, p, e0, e1, N, o, t, nthr); break;
      case 4: reduce_range<4, OUT, 0>(P, stride, p, e0, e1, N, o, t, nthr); break;
      case 8: reduce_range<8, OUT, 0>(P, stride, p, e0, e1, N, o, t, nthr); break;
      default: reduce_range<0, OUT, 0>(P, stride, p, e0, e1, N, o, t, nthr); break;
    }
  }
}

__device__ __forceinline__ void reduce_any(const void* P, int64_t stride, int p, int64_t e0, int64_t e1, int N,
                                           const ReduceOut& o, int64_t t, int64_t nthr) {
  if (o.pbf16) {
    if (o.dtype == OUT_F32)
      reduce_dispatch_p<OUT_F32, 1>(P, stride, p, e0, e1, N, o, t, nthr);
    else
      reduce_dispatch_p<OUT_BF16, 1>(P, stride, p, e0, e1, N, o, t, nthr);
  } else {
    if (o.dtype == OUT_F32)
      reduce_dispatch_p<OUT_F32, 0>(P, stride, p, e0, e1, N, o, t, nthr);
    else
      reduce_dispatch_p<OUT_BF16, 0>(P, stride, p, e0, e1, N, o, t, nthr);
  }
}

#if TPF_IN_PART(0)
__global__ __launch_bounds__(256) void reduce_rows_kernel(const void* P, int64_t stride, int p, int64_t e0,
                                                          int64_t e1, int N, ReduceOut o) {
  reduce_any(P, stride, p, e0, e1, N, o, (int64_t)blockIdx.x * 256 + threadIdx.x, (int64_t)gridDim.x * 256);
}

__global__ __launch_bounds__(256) void copy_kernel(const char* src, char* dst, int64_t bytes) {
  copy_range(src, dst, 0, bytes, (int64_t)blockIdx.x * 256 + threadIdx.x, (int64_t)gridDim.x * 256);
}

// One launch for the whole AllGather: block row y copies slice y.
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs args) {
  (void)args;
  const GatherArgs& a = kernarg<GatherArgs>();
  const int r = blockIdx.y;
  copy_range(a.src[r], a.dst + (int64_t)r * a.slice_bytes, 0, a.slice_bytes,
             (int64_t)blockIdx.x * 256 + threadIdx.x, (int64_t)gridDim.x * 256);
}

__global__ void clear_status_kernel(Ctrl* c) {
  if (threadIdx.x == 0) atomic_store_relaxed(&c->status, 0);
}
#endif

// The XCD (accelerator die) this wave runs on, from the hardware register
// XCC_ID.  Used only as a locality hint.
__device__ __forceinline__ int xcd_id() {
  return (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & (kXcds - 1));
}

// Claim one of the G GEMM tiles of chunk c for a workgroup on XCD x.  The
// tiles of a chunk are split into kXcds contiguous shares; a workgroup takes
// the next tile of its own XCD's share, or, once that share is used up, of
// the next XCD's.  The global ticket already guarantees that exactly G
// claims are made for chunk c, so every claim finds a free tile.
__device__ __forceinline__ int claim_tile(Ctrl* ctl, int c, int G, int x) {
  const int q = G / kXcds, r = G % kXcds;
  for (int d = 0; d < kXcds; ++d) {
    const int y = (x + d) & (kXcds - 1);
    const int size = q + (y < r ? 1 : 0);
    if (size == 0) continue;
    const int s = __hip_atomic_fetch_add(&ctl->sub[c][y], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (s < size) return y * q + min(y, r) + s;
  }
  return -1;   // unreachable: G claims are made for G tiles
}

// Debug timing perturbation: task `task` of a launch sleeps a bounded time
// before it stores or publishes its results when the seeded hash selects it
// (the same decision for every thread of the workgroup).
__device__ __forceinline__ void debug_delay(const DelayArgs& d, uint32_t task) {
  if (d.period <= 0) return;
  uint32_t x = d.seed ^ (task * 0x9E3779B9u);
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  if (x % (uint32_t)d.period != 0) return;
  for (int i = 0; i < d.sleeps; ++i) __builtin_amdgcn_s_sleep(127);
}

// Thread 0 polls *ctr with relaxed loads (no cache maintenance per poll),
// backing off exponentially so that many waiting workgroups do not hammer one
// memory channel, until it reaches target or the bound runs out; then one
// agent-scope acquire.  The caller's following barrier orders the other
// threads' loads after that acquire.
__device__ __forceinline__ void wait_at_least(const int* ctr, int target, const FusedArgs& a) {
  if (a.unreachable) target = target + 1 + (1 << 30);
  int64_t polls = 0;
  int nap = 1;
  while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    if (++polls > a.spin_limit) {
      __hip_atomic_fetch_or(&a.ctrl->status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    for (int i = 0; i < nap; ++i) __builtin_amdgcn_s_sleep(8);   // ~512 clocks each
    nap = nap < 8 ? nap * 2 : 8;
  }
  fence_acquire_agent();
}

// Publish this workgroup's global writes: every thread's writes are ordered
// before the barrier (workgroup-scope release), and thread 0's agent-scope
// release increment makes them visible to any workgroup on any XCD that
// acquires the counter.
__device__ __forceinline__ void publish(int* ctr) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) atomic_add_release(ctr, 1);
}

template <class Cfg, int BL>
__global__ __launch_bounds__(Cfg::THREADS) void fused_kernel(FusedArgs args) {
  (void)args;
  const FusedArgs& a = kernarg<FusedArgs>();
  // The ticket is broadcast through the first word of LDS stage 0, which is
  // idle between tasks (gemm_tile ends with every load consumed and a
  // barrier) and keeps the LDS footprint at exactly STAGES stages.
  int& s_ticket = *reinterpret_cast<int*>(stage_ptr<Cfg, 0>());
  const int tid = threadIdx.x;
  Ctrl* ctl = a.ctrl;
  const int total = a.seg_start[a.nseg];
  const int tiles_n = (a.g.N + Cfg::BN - 1) / Cfg::BN;
  int seg = 0;
  const int xcd = xcd_id();
  for (;;) {
    if (tid == 0) {
      const int tk = __hip_atomic_fetch_add(&ctl->ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int val = tk;
      if (tk < total) {
        int sg = seg;
        while (a.seg_start[sg + 1] <= tk) ++sg;
        // A GEMM ticket names the chunk; the tile comes from this XCD's share.
        if ((a.seg_info[sg] & 0xF) == TK_GEMM) {
          const int c = a.seg_info[sg] >> 4;
          val = a.seg_start[sg] + claim_tile(ctl, c, a.seg_start[sg + 1] - a.seg_start[sg], xcd);
        }
      }
      s_ticket = val;
    }
    __syncthreads();
    // The ticket is the same for the whole workgroup; saying so keeps every
    // value derived from it (shard, operand pointers, buffer resources) in
    // scalar registers instead of per-lane "waterfall" loops.
    const int t = __builtin_amdgcn_readfirstlane(s_ticket);
    __syncthreads();
    if (t >= total) break;
    const uint64_t t_start = a.timeline ? __builtin_amdgcn_s_memrealtime() : 0;
    uint64_t t_mid = 0;
    while (a.seg_start[seg + 1] <= t) ++seg;   // this workgroup's tickets only increase
    const int u = t - a.seg_start[seg];
    const int kind = a.seg_info[seg] & 0xF;
    const int idx = a.seg_info[seg] >> 4;

    if (kind == TK_GEMM) {
      const int c = idx;
      const int row0 = a.ch.row0(c), row1 = a.ch.row1(c);
      const int tiles_m = (row1 - row0 + Cfg::BM - 1) / Cfg::BM;
      int shard, tm, tn;
      tile_coords(u, tiles_m, tiles_n, shard, tm, tn);
      const TileJob j = make_job<Cfg>(a.g, shard, row0, row1, tm, tn);
      if (a.gather) {
        // The rows of this tile must have landed in the gathered buffer.
        if (tid == 0) {
          const int s0 = j.m0 / a.slice_rows, s1 = (j.m0 + j.rows - 1) / a.slice_rows;
          for (int s = s0; s <= s1; ++s) wait_at_least(&ctl->landed[s], a.copy_segs, a);
        }
        __syncthreads();
      }
      Frag<Cfg> f;
      gemm_tile<Cfg, BL>(f, j);
      store_any<Cfg>(f, j, a.g, shard);
      debug_delay(a.g.delay, (uint32_t)t);
      if (!a.gather) {
        publish(&ctl->ready[c]);
        if (a.piggyback && c > 0) {
          // Slice u of chunk c-1's reduction.  Every tile of chunk c-1 holds a
          // smaller ticket than this one, so the wait ends; usually at once.
          t_mid = a.timeline ? __builtin_amdgcn_s_memrealtime() : 0;
          const int G = a.gemm_tasks[c];
          const int64_t cb = (int64_t)a.ch.row0(c - 1) * a.g.N, ce = (int64_t)a.ch.row1(c - 1) * a.g.N;
          const int64_t per = ((ce - cb + G - 1) / G + 7) / 8 * 8;   // whole 8-element groups
          const int64_t e0 = cb + (int64_t)u * per, e1 = min(e0 + per, ce);
          if (e0 < e1) {
            if (tid == 0) wait_at_least(&ctl->ready[c - 1], a.gemm_tasks[c - 1], a);
            __syncthreads();
            reduce_any(a.P, a.p_stride, a.p, e0, e1, a.g.N, a.ro, tid, Cfg::THREADS);
          }
        }
      }
    } else if (kind == TK_REDUCE) {
      const int c = idx;
      if (tid == 0) wait_at_least(&ctl->ready[c], a.gemm_tasks[c], a);
      __syncthreads();
      const int64_t e0 = (int64_t)a.ch.row0(c) * a.g.N + (int64_t)u * a.reduce_elems;
      const int64_t e1 = min(e0 + a.reduce_elems, (int64_t)a.ch.row1(c) * a.g.N);
      reduce_any(a.P, a.p_stride, a.p, e0, e1, a.g.N, a.ro, tid, Cfg::THREADS);
    } else {  // TK_COPY
      const int r = idx;
      const int64_t b0 = (int64_t)u * a.copy_seg_bytes;
      const int64_t b1 = min(b0 + a.copy_seg_bytes, a.slice_bytes);
      copy_range(a.src[r], a.gathered + (int64_t)r * a.slice_bytes, b0, b1, tid, Cfg::THREADS);
      debug_delay(a.g.delay, (uint32_t)t);
      publish(&ctl->landed[r]);
    }
    if (a.timeline && tid == 0 && t < a.timeline_cap) {
      TimelineEvent ev;
      ev.ticket = (uint32_t)t;
      ev.kind = (uint16_t)kind;
      ev.chunk = (uint16_t)idx;
      ev.block = (uint16_t)blockIdx.x;
      ev.xcd = (uint16_t)xcd;
      ev.mid = t_mid ? (uint32_t)(t_mid - t_start) : 0u;
      ev.t_start = t_start;
      ev.t_end = __builtin_amdgcn_s_memrealtime();
      a.timeline[t] = ev;
    }
  }
  // The last workgroup out clears the counters for the next call.
  if (tid == 0) {
    const int d = atomic_add_acq_rel(&ctl->done, 1);
    if (d == (int)gridDim.x - 1) {
      for (int c = 0; c < a.ch.n; ++c) {
        atomic_store_relaxed(&ctl->ready[c], 0);
        for (int x = 0; x < kXcds; ++x) atomic_store_relaxed(&ctl->sub[c][x], 0);
      }
      for (int s = 0; s < kMaxShards; ++s) atomic_store_relaxed(&ctl->landed[s], 0);
      atomic_store_relaxed(&ctl->ticket, 0);
      atomic_store_relaxed(&ctl->done, 0);
    }
  }
}

// Block b of a grid of `total` blocks -> task index.  Blocks are dealt to the
// XCDs round-robin (block b runs on XCD b % 8), so the tasks are split into
// kXcds contiguous shares and block b takes task b / 8 of share b % 8: each
// XCD's L2 then sees a contiguous run of tiles.
__device__ __forceinline__ int xcd_task(int b, int total) {
  const int x = b & (kXcds - 1), i = b / kXcds;
  return x * (total / kXcds) + min(x, total % kXcds) + i;
}

// Sum output tile (m0, rows, n0, ncols) over the p shards' partials.
template <int OUT, int PB>
__device__ __forceinline__ void reduce_tile_p(const TileArgs& a, int m0, int rows, int n0, int ncols, int tid,
                                              int nthr) {
  const int N = a.g.N;
  if constexpr (PB) {
    switch (a.p) {
      case 2: reduce_tile_b16<2, OUT>(a.P, a.p_stride, 2, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
      case 4: reduce_tile_b16<4, OUT>(a.P, a.p_stride, 4, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
      case 8: reduce_tile_b16<8, OUT>(a.P, a.p_stride, 8, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
      default: reduce_tile_b16<0, OUT>(a.P, a.p_stride, a.p, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
    }
  } else {
    switch (a.p) {
      case 2: reduce_tile<2, OUT, 0>(a.P, a.p_stride, 2, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
      case 4: reduce_tile<4, OUT, 0>(a.P, a.p_stride, 4, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
      case 8: reduce_tile<8, OUT, 0>(a.P, a.p_stride, 8, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
      default: reduce_tile<0, OUT, 0>(a.P, a.p_stride, a.p, m0, rows, n0, ncols, N, a.ro, tid, nthr); break;
    }
  }
}

__device__ __forceinline__ void reduce_tile_any(const TileArgs& a, int m0, int rows, int n0, int ncols, int tid,
                                                int nthr) {
  if (a.ro.pbf16) {
    if (a.ro.dtype == OUT_F32) reduce_tile_p<OUT_F32, 1>(a, m0, rows, n0, ncols, tid, nthr);
    else reduce_tile_p<OUT_BF16, 1>(a, m0, rows, n0, ncols, tid, nthr);
  } else {
    if (a.ro.dtype == OUT_F32) reduce_tile_p<OUT_F32, 0>(a, m0, rows, n0, ncols, tid, nthr);
    else reduce_tile_p<OUT_BF16, 0>(a, m0, rows, n0, ncols, tid, nthr);
  }
}

// Epilogue of the fold scheduler, run by the tiles of the last shard after
// the partials of shards 0..p-2 are complete (an earlier launch wrote them).
// For each element: s = P_0 + P_1 + ... + P_{p-2} left to right in fp32, then
// s + (this tile's fp32 accumulator, rounded to bf16 first for 2-byte
// messages, exactly the message this shard would have stored), rounded once
// into the AllReduce or ReduceScatter destination.  These are the reduction
// kernel's additions in its order, so the bits are the same.  The partials of
// up to four shards for 8 of the 16 elements a lane holds of one 32x32 block
// are requested together before they are added.
template <int PB>
__device__ __forceinline__ float message_value(float acc) {
  if constexpr (PB) return __uint_as_float(f32_to_bf16_bits(acc) << 16);
  else return acc;
}

// The fold epilogue streams the partials with 16-byte loads: the tile's
// accumulators are staged through idle LDS slots in bands of
// FoldBand::ROWS rows, then every thread takes groups of four consecutive
// columns of a band row, loads the p-1 partials of those elements, adds them
// in shard order and then its own value, and stores the four results.
template <class Cfg>
struct FoldBand {
  // A band of 64 rows spans the first two A slots when one holds fewer rows
  // (rows [0, SLOT_ROWS) in slot 0, the rest in slot 1).
  static constexpr int SLOT_ROWS = Cfg::LDS_A / (Cfg::BN * 4);
  static constexpr int ROWS = 64;
  static_assert(SLOT_ROWS >= 64 || (SLOT_ROWS == 32 && Cfg::STAGES_A >= 2), "a band fits two idle LDS slots");
  static_assert(Cfg::BM % ROWS == 0 && Cfg::WM % 32 == 0, "bands of whole 32-row blocks");
  __device__ __forceinline__ static float* row_ptr(int row) {
    if constexpr (SLOT_ROWS >= ROWS) {
      return reinterpret_cast<float*>(stage_ptr<Cfg, 0>()) + row * Cfg::BN;
    } else {
      return row < SLOT_ROWS ? reinterpret_cast<float*>(stage_ptr<Cfg, 0>()) + row * Cfg::BN
                             : reinterpret_cast<float*>(stage_ptr<Cfg, 1>()) + (row - SLOT_ROWS) * Cfg::BN;
    }
  }
};

// Sum of the partials of shards 0 .. np-1 at elements e .. e+3, left to right
// (PP > 0: np == PP at compile time, all loads issued first).
template <int PP, int PB>
__device__ __forceinline__ f32x4_t fold_partials4(const void* P, int64_t stride, int np, int64_t e) {
  if constexpr (PP > 0) {
    f32x4_t v[PP];
#pragma unroll
    for (int k = 0; k < PP; ++k) v[k] = load_partial4<PB>(P, (int64_t)k * stride + e);
    f32x4_t s = v[0];
#pragma unroll
    for (int k = 1; k < PP; ++k) s = s + v[k];
    return s;
  } else {
    f32x4_t s = load_partial4<PB>(P, e);
    for (int k = 1; k < np; ++k) s = s + load_partial4<PB>(P, (int64_t)k * stride + e);
    return s;
  }
}

template <class Cfg, int OUT, int PB, int PP>
__device__ __forceinline__ void fold_store_pp(const Frag<Cfg>& f, const TileJob& j, const TileArgs& a) {
  constexpr int BR = FoldBand<Cfg>::ROWS;
  constexpr int GROUPS = BR * Cfg::BN / 4;                 // four-column groups per band
  constexpr int PER = GROUPS / Cfg::THREADS;
  static_assert(GROUPS % Cfg::THREADS == 0, "whole groups per thread");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int r32 = lane & 31, half = lane >> 5;
  const int np = a.p - 1;
  const int N = j.N;
  const int ncols = min(Cfg::BN, N - j.n0);                // a multiple of 8
#pragma unroll
  for (int b0 = 0; b0 < Cfg::BM; b0 += BR) {
    if (b0 >= j.rows) break;                               // the same for the whole workgroup
    // This band's 32-row blocks go to LDS.
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int r0 = wm * Cfg::WM + i * 32;
      if (r0 >= b0 && r0 < b0 + BR) {
#pragma unroll
        for (int jn = 0; jn < Cfg::TN; ++jn) {
          const int col = wn * Cfg::WN + jn * 32 + r32;
          float* blk = FoldBand<Cfg>::row_ptr(r0 - b0);   // a 32-row block lies in one slot
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = 8 * (v >> 2) + 4 * half + (v & 3);
            blk[row * Cfg::BN + col] = f.acc[i][jn][v];
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int g = q * Cfg::THREADS + threadIdx.x;
      const int row = g / (Cfg::BN / 4), c = (g % (Cfg::BN / 4)) * 4;
      if (b0 + row < j.rows && c < ncols) {
        const int64_t e = (int64_t)(j.m0 + b0 + row) * N + j.n0 + c;
        // This shard's own values as the message it would have stored
        // (rounded to bf16 first for 2-byte messages).
        f32x4_t own = *reinterpret_cast<const f32x4_t*>(FoldBand<Cfg>::row_ptr(row) + c);
#pragma unroll
        for (int t = 0; t < 4; ++t) own[t] = message_value<PB>(own[t]);
        const f32x4_t s = np > 0 ? fold_partials4<PP, PB>(a.P, a.p_stride, np, e) + own : own;
        reduce_store4<OUT>(a.ro, e, N, s);
      }
    }
    __syncthreads();                                       // the band is free again
  }
}

template <class Cfg, int OUT, int PB>
__device__ __forceinline__ void fold_store(const Frag<Cfg>& f, const TileJob& j, const TileArgs& a) {
  switch (a.p) {   // the partials of the other shards: p - 1 of them
    case 2: fold_store_pp<Cfg, OUT, PB, 1>(f, j, a); break;
    case 4: fold_store_pp<Cfg, OUT, PB, 3>(f, j, a); break;
    case 8: fold_store_pp<Cfg, OUT, PB, 7>(f, j, a); break;
    default: fold_store_pp<Cfg, OUT, PB, 0>(f, j, a); break;
  }
}

// The fold variants of tile_kernel: RED = 2 + (fp32 output) + 2 * (bf16 messages).
constexpr int fold_red(int out, int pbf16) { return 2 + (out == OUT_F32 ? 1 : 0) + 2 * pbf16; }

// One workgroup per GEMM tile, used for plain shard GEMMs (RED = 0), for the
// tile scheduler (RED = 1) and for the last shard of the fold scheduler
// (RED = 2..5, see fold_red: a.g holds that one shard's operands).  The nshard * tiles_m * tiles_n tiles of
// rows [row0, row1) are taken in the order of tile_coords (shard-major,
// grouped tile rows) through xcd_task, so each XCD works through the operand
// panels of one shard, and the XCDs of different shards advance through the
// same output tiles at the same time.
//
// RED = 1: after storing its partial, a workgroup bumps the output
// tile's counter (release); the one that brings it to p acquires and sums
// the tile in shard order.  No workgroup ever waits for another.
template <class Cfg, int BL, int RED>
__global__ __launch_bounds__(Cfg::THREADS) void tile_kernel(TileArgs args) {
  (void)args;
  const TileArgs& a = kernarg<TileArgs>();
  const int tid = threadIdx.x;
  const int u = xcd_task(blockIdx.x, a.tasks);
  int shard, tm, tn;
  tile_coords(u, a.tiles_m, a.tiles_n, shard, tm, tn);
  const TileJob j = make_job<Cfg>(a.g, shard, a.row0, a.row1, tm, tn);
  Frag<Cfg> f;
  if constexpr (RED == 0) {
    gemm_tile<Cfg, BL>(f, j);
    debug_delay(a.g.delay, (uint32_t)u);
    store_any<Cfg>(f, j, a.g, shard);
  } else if constexpr (RED >= 2) {
    gemm_tile<Cfg, BL>(f, j);
    constexpr int FOLD_OUT = ((RED - 2) & 1) ? OUT_F32 : OUT_BF16;
    constexpr int FOLD_PB = (RED - 2) / 2;
    fold_store<Cfg, FOLD_OUT, FOLD_PB>(f, j, a);
  } else {
    int& s_word = *reinterpret_cast<int*>(stage_ptr<Cfg, 0>());   // idle once gemm_tile returns
    const uint64_t t_start = a.timeline ? __builtin_amdgcn_s_memrealtime() : 0;
    uint64_t t_mid = 0;
    gemm_tile<Cfg, BL>(f, j);
    store_any<Cfg>(f, j, a.g, shard);   // fp32 partial, or bf16 for the 2-byte message
    debug_delay(a.g.delay, (uint32_t)u);
    const int T = tm * a.tiles_n + tn;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (tid == 0) {
      const int prev = atomic_add_release(&a.cnt[T], 1);
      const int last = prev == a.p - 1;
      if (last) {
        fence_acquire_agent();
        atomic_store_relaxed(&a.cnt[T], 0);   // every shard of tile T is counted: ready for the next call
      }
      s_word = last;
    }
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_word)) {
      t_mid = a.timeline ? __builtin_amdgcn_s_memrealtime() : 0;
      reduce_tile_any(a, j.m0, j.rows, j.n0, min(Cfg::BN, j.N - j.n0), tid, Cfg::THREADS);
    }
    if (a.timeline && tid == 0 && u < a.timeline_cap) {
      TimelineEvent ev;
      ev.ticket = (uint32_t)u;
      ev.kind = (uint16_t)TK_GEMM;
      ev.chunk = (uint16_t)T;
      ev.block = (uint16_t)blockIdx.x;
      ev.xcd = (uint16_t)xcd_id();
      ev.mid = t_mid ? (uint32_t)(t_mid - t_start) : 0u;
      ev.t_start = t_start;
      ev.t_end = __builtin_amdgcn_s_memrealtime();
      a.timeline[u] = ev;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

// Per-part launchers (defined in parts 1 to 6, dispatched in part 0).
void launch_tiles_large(int bl, int red, const TileArgs& a, int grid, hipStream_t s);
void launch_tiles_fold_f32msg(int bl, int out, const TileArgs& a, int grid, hipStream_t s);
void launch_tiles_fold_bf16msg(int bl, int out, const TileArgs& a, int grid, hipStream_t s);
int fused_occupancy_large(int bl);
int fused_occupancy_small(int cfg, int bl);
void launch_fused_large(int bl, const FusedArgs& a, int grid, hipStream_t s);
void launch_fused_small(int cfg, int bl, const FusedArgs& a, int grid, hipStream_t s);
void launch_tiles_small(int cfg, int bl, int red, const TileArgs& a, int grid, hipStream_t s);

template <class Cfg, int RED>
static void launch_tile_cfg(int bl, const TileArgs& a, int grid, hipStream_t s) {
  if constexpr (Cfg::KM_OK && RED == 0) {
    if (bl == (A_KM | B_KN)) {
      hipLaunchKernelGGL((tile_kernel<Cfg, A_KM | B_KN, 0>), dim3(grid), dim3(Cfg::THREADS), 0, s, a);
      return;
    }
  }
  if (bl == B_KN)
    hipLaunchKernelGGL((tile_kernel<Cfg, B_KN, RED>), dim3(grid), dim3(Cfg::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((tile_kernel<Cfg, B_NK, RED>), dim3(grid), dim3(Cfg::THREADS), 0, s, a);
}

template <class Cfg>
static void launch_tile_red(int bl, int red, const TileArgs& a, int grid, hipStream_t s) {
  if (red == 1) launch_tile_cfg<Cfg, 1>(bl, a, grid, s);
  else launch_tile_cfg<Cfg, 0>(bl, a, grid, s);
}

#if TPF_IN_PART(0)
hipError_t launch_reduce_rows(const void* P, int64_t stride, int p, int row0, int row1, int N,
                              const ReduceOut& o, int num_cus, hipStream_t s) {
  const int64_t e0 = (int64_t)row0 * N, e1 = (int64_t)row1 * N;
  const int64_t groups = (e1 - e0) / 4;
  if (groups <= 0) return hipSuccess;
  int64_t grid = (groups + 256 * 2 - 1) / (256 * 2);
  // A small reduction (decode shapes: a few MB of partials) is bound by the
  // latency of its loads, not by bandwidth: spread it over every CU, down to
  // a quarter of a 256-thread block's groups per workgroup.
  const int64_t spread = std::min<int64_t>((groups + 63) / 64, num_cus);
  if (grid < spread) grid = spread;
  const int64_t cap = (int64_t)num_cus * 8;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(reduce_rows_kernel, dim3((unsigned)grid), dim3(256), 0, s, P, stride, p, e0, e1, N, o);
  return hipGetLastError();
}

hipError_t launch_copy(const char* src, char* dst, int64_t bytes, int num_cus, hipStream_t s) {
  const int64_t chunks = bytes / 16;
  if (chunks <= 0) return hipSuccess;
  int64_t grid = (chunks + 256 * 4 - 1) / (256 * 4);
  const int64_t cap = (int64_t)num_cus * 8;
  if (grid > cap) grid = cap;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)grid), dim3(256), 0, s, src, dst, bytes);
  return hipGetLastError();
}

hipError_t launch_gather(const void* const* src, int p, char* dst, int64_t slice_bytes, int num_cus, hipStream_t s) {
  const int64_t chunks = slice_bytes / 16;
  if (chunks <= 0 || p <= 0) return hipSuccess;
  if (p > kMaxShards) return hipErrorInvalidValue;
  GatherArgs a{};
  for (int r = 0; r < p; ++r) a.src[r] = reinterpret_cast<const char*>(src[r]);
  a.dst = dst;
  a.slice_bytes = slice_bytes;
  int64_t gx = (chunks + 256 * 4 - 1) / (256 * 4);
  int64_t cap = (int64_t)num_cus * 8 / p;
  if (cap < 1) cap = 1;
  if (gx > cap) gx = cap;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)gx, (unsigned)p), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_tiles(int cfg, int bl, int red, const TileArgs& a, hipStream_t s) {
  if (a.tasks <= 0) return hipSuccess;
  const int grid = a.tasks;
  if (red >= 2) {   // fold epilogue: large tiles only
    if (cfg != CFG_LARGE || red > 5) return hipErrorInvalidValue;
    const int out = ((red - 2) & 1) ? OUT_F32 : OUT_BF16;
    if ((red - 2) >> 1) launch_tiles_fold_bf16msg(bl, out, a, grid, s);
    else launch_tiles_fold_f32msg(bl, out, a, grid, s);
    return hipGetLastError();
  }
  if (cfg == CFG_SMALL || cfg == CFG_MID) launch_tiles_small(cfg, bl, red, a, grid, s);
  else launch_tiles_large(bl, red, a, grid, s);
  return hipGetLastError();
}

hipError_t launch_gemm_rows(int cfg, int bl, const GemmOperands& g, int row0, int row1, hipStream_t s) {
  TileArgs a{};
  a.g = g;
  a.row0 = row0;
  a.row1 = row1;
  a.tiles_m = (row1 - row0 + cfg_bm(cfg) - 1) / cfg_bm(cfg);
  a.tiles_n = (g.N + cfg_bn(cfg) - 1) / cfg_bn(cfg);
  a.tasks = g.nshard * a.tiles_m * a.tiles_n;
  return launch_tiles(cfg, bl, 0, a, s);
}

hipError_t launch_clear_status(Ctrl* c, hipStream_t s) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, s, c);
  return hipGetLastError();
}

int fused_occupancy(int cfg, int bl) {
  return cfg == CFG_LARGE ? fused_occupancy_large(bl) : fused_occupancy_small(cfg, bl);
}

hipError_t launch_fused(int cfg, int bl, const FusedArgs& a, int grid, hipStream_t s) {
  if (cfg == CFG_LARGE) launch_fused_large(bl, a, grid, s);
  else launch_fused_small(cfg, bl, a, grid, s);
  return hipGetLastError();
}
#endif

template <class Cfg, int BL>
static int fused_blocks_per_cu() {
  static int cached = 0;
  if (!cached) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fused_kernel<Cfg, BL>, Cfg::THREADS, 0) != hipSuccess ||
        n < 1)
      n = 1;
    cached = n;
  }
  return cached;
}

template <class Cfg>
static void launch_fused_cfg(int bl, const FusedArgs& a, int grid, hipStream_t s) {
  if (bl == B_KN)
    hipLaunchKernelGGL((fused_kernel<Cfg, B_KN>), dim3(grid), dim3(Cfg::THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((fused_kernel<Cfg, B_NK>), dim3(grid), dim3(Cfg::THREADS), 0, s, a);
}

#if TPF_IN_PART(1)
int fused_occupancy_large(int bl) {
  return bl == B_KN ? fused_blocks_per_cu<CfgLargeFused, B_KN>() : fused_blocks_per_cu<CfgLargeFused, B_NK>();
}
void launch_fused_large(int bl, const FusedArgs& a, int grid, hipStream_t s) {
  launch_fused_cfg<CfgLargeFused>(bl, a, grid, s);
}
#endif

#if TPF_IN_PART(5)
int fused_occupancy_small(int cfg, int bl) {
  if (cfg == CFG_SMALL) return bl == B_KN ? fused_blocks_per_cu<CfgSmall, B_KN>() : fused_blocks_per_cu<CfgSmall, B_NK>();
  return bl == B_KN ? fused_blocks_per_cu<CfgMid, B_KN>() : fused_blocks_per_cu<CfgMid, B_NK>();
}
void launch_fused_small(int cfg, int bl, const FusedArgs& a, int grid, hipStream_t s) {
  if (cfg == CFG_SMALL) launch_fused_cfg<CfgSmall>(bl, a, grid, s);
  else launch_fused_cfg<CfgMid>(bl, a, grid, s);
}
#endif

#if TPF_IN_PART(2)
void launch_tiles_large(int bl, int red, const TileArgs& a, int grid, hipStream_t s) {
  launch_tile_red<CfgLarge>(bl, red, a, grid, s);
}
#endif

#if TPF_IN_PART(3)
void launch_tiles_fold_f32msg(int bl, int out, const TileArgs& a, int grid, hipStream_t s) {
  if (out == OUT_BF16) launch_tile_cfg<CfgLarge, fold_red(OUT_BF16, 0)>(bl, a, grid, s);
  else launch_tile_cfg<CfgLarge, fold_red(OUT_F32, 0)>(bl, a, grid, s);
}
#endif

#if TPF_IN_PART(6)
void launch_tiles_fold_bf16msg(int bl, int out, const TileArgs& a, int grid, hipStream_t s) {
  if (out == OUT_BF16) launch_tile_cfg<CfgLarge, fold_red(OUT_BF16, 1)>(bl, a, grid, s);
  else launch_tile_cfg<CfgLarge, fold_red(OUT_F32, 1)>(bl, a, grid, s);
}
#endif

#if TPF_IN_PART(4)
void launch_tiles_small(int cfg, int bl, int red, const TileArgs& a, int grid, hipStream_t s) {
  if (cfg == CFG_SMALL) launch_tile_red<CfgSmall>(bl, red, a, grid, s);
  else launch_tile_red<CfgMid>(bl, red, a, grid, s);
}
#endif

// The output-stationary single launch (tpf_stationary.hpp): one workgroup of
// eight waves per output tile of 32 columns and 32 (M <= 32) or 64 rows.  The
// LDS holds the eight waves' weight rings during the K loops and the p
// partials of the tile (at most 16 x 64 x 32 fp32 = 128 KiB) for the fold
// after them.  Measured on the decode shapes (p = 8, K = 1024, N = 8192):
// 2, 3 and 4 ring slots within 3 %; 64-column tiles (half the workgroups,
// 128-byte weight rows) 8-15 % slower; tiles dealt round-robin over the XCDs
// instead of in contiguous shares 17 % slower.
#ifndef TPF_ST_SMALL
#define TPF_ST_SMALL StCfg<1, 1, 64, 2>
#endif
#ifndef TPF_ST_MID
#define TPF_ST_MID StCfg<2, 1, 64, 2>
#endif
using StSmall = TPF_ST_SMALL;
using StMid = TPF_ST_MID;
using StSmallAnyP = StCfg<1, 1, 64, 2>;
using StMidAnyP = StCfg<2, 1, 64, 2>;
static_assert(st_max_shards<StSmallAnyP>() >= kMaxShards && st_max_shards<StMidAnyP>() >= kMaxShards,
              "the fallback shapes hold every shard's partials");

template <class C, int PB, int OUT>
__global__ __launch_bounds__(kStWaves * 64) void stationary_kernel(StationaryArgs args) {
  (void)args;
  const StationaryArgs& a = kernarg<StationaryArgs>();
  __shared__ __attribute__((aligned(1024))) char lds[kStLdsBytes];
  stationary_tile<C, PB, OUT>(a, lds, xcd_task(blockIdx.x, a.tiles_m * a.tiles_n));
}

#if TPF_IN_PART(7)
template <class C>
static hipError_t launch_st_cfg(StationaryArgs a, int pbf16, int out, hipStream_t s) {
  a.tiles_m = (a.M + C::BM - 1) / C::BM;
  a.tiles_n = (a.N + C::BN - 1) / C::BN;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  if (grid <= 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  const dim3 g((unsigned)grid), b(kStWaves * 64);
  if (pbf16) {
    if (out == OUT_F32) hipLaunchKernelGGL((stationary_kernel<C, 1, OUT_F32>), g, b, 0, s, a);
    else hipLaunchKernelGGL((stationary_kernel<C, 1, OUT_BF16>), g, b, 0, s, a);
  } else {
    if (out == OUT_F32) hipLaunchKernelGGL((stationary_kernel<C, 0, OUT_F32>), g, b, 0, s, a);
    else hipLaunchKernelGGL((stationary_kernel<C, 0, OUT_BF16>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_stationary(const StationaryArgs& a, int pbf16, int out, hipStream_t s) {
  if (a.p < 1 || a.p > kMaxShards || a.M <= 0 || a.N <= 0) return hipErrorInvalidValue;
  if (a.M <= 32)
    return a.p <= st_max_shards<StSmall>() ? launch_st_cfg<StSmall>(a, pbf16, out, s)
                                           : launch_st_cfg<StSmallAnyP>(a, pbf16, out, s);
  return a.p <= st_max_shards<StMid>() ? launch_st_cfg<StMid>(a, pbf16, out, s)
                                       : launch_st_cfg<StMidAnyP>(a, pbf16, out, s);
}
#endif

// ---------------------------------------------------------------------------
// Output-stationary single launch, large tiles (part 8)
// ---------------------------------------------------------------------------
// One workgroup per 128 x 256 output tile, in the shard GEMMs' grouped,
// XCD-aware tile order.  For k = 0 .. p-1 it runs shard k's K loop (the same
// MFMA chain from a zero accumulator as every other path, so the result is
// the partial shard k would send, rounded to bf16 first for 2-byte messages)
// and folds it into a running sum kept in registers: S = P_0, then
// S = S + P_k in shard order -- the reduction kernel's additions in its
// order.  The sum is rounded once and stored to the AllReduce or
// ReduceScatter destination.  No partial goes to memory and no second
// launch follows; the price is a smaller tile (128 x 256 instead of
// 256 x 256: half the MFMAs per loaded byte), which the two accumulator sets
// need to fit the register file.
#if TPF_IN_PART(8)
template <class Cfg, int OUT>
__device__ __forceinline__ void store_sum(const Frag<Cfg>& s, const TileJob& j, const ReduceOut& ro) {
  if (!ro.scatter) {
    store_tile<Cfg, OUT>(s, j, ro.y[0], j.N);
    return;
  }
  const int rps = ro.rows_per_slice;
  const int sl = j.m0 / rps;
  if ((j.m0 + j.rows - 1) / rps == sl) {   // the tile lies in one slice (uniform)
    TileJob js = j;
    js.m0 = j.m0 - sl * rps;
    store_tile<Cfg, OUT>(s, js, ro.y[sl], j.N);
    return;
  }
  // a tile that straddles two slices: element by element
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn) {
      const int col = j.n0 + wn * Cfg::WN + jn * 32 + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * Cfg::WM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (row < j.rows && col < j.N) {
          const int gr = j.m0 + row, r_sl = gr / rps;
          const int64_t off = (int64_t)(gr - r_sl * rps) * j.N + col;
          if constexpr (OUT == OUT_F32)
            reinterpret_cast<float*>(ro.y[r_sl])[off] = s.acc[i][jn][v];
          else
            reinterpret_cast<uint16_t*>(ro.y[r_sl])[off] = (uint16_t)f32_to_bf16_bits(s.acc[i][jn][v]);
        }
      }
    }
}

template <class Cfg, int BL, int PB, int OUT>
__global__ __launch_bounds__(Cfg::THREADS) void stationary_large_kernel(StatLargeArgs args) {
  (void)args;
  const StatLargeArgs& a = kernarg<StatLargeArgs>();
  const int u = xcd_task(blockIdx.x, a.tiles_m * a.tiles_n);
  int shard, tm, tn;
  tile_coords(u, a.tiles_m, a.tiles_n, shard, tm, tn);   // shard = 0: one grid of output tiles
  // The running sum starts at -0, the identity of fp32 addition for every
  // value (also -0 itself), so after shard 0 it holds P_0 bit for bit.
  Frag<Cfg> s;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) s.acc[i][jn][v] = -0.0f;
  const TileJob j0 = make_job<Cfg>(a.g, 0, 0, a.g.M, tm, tn);
  for (int k = 0; k < a.g.nshard; ++k) {
    TileJob j = j0;
    j.A = a.g.A[k];
    j.B = a.g.B[k];
    Frag<Cfg> f;
    gemm_tile<Cfg, BL>(f, j);
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int jn = 0; jn < Cfg::TN; ++jn)
#pragma unroll
        for (int v = 0; v < 16; ++v) s.acc[i][jn][v] += message_value<PB>(f.acc[i][jn][v]);
  }
  store_sum<Cfg, OUT>(s, j0, a.ro);
}

template <class Cfg, int BL>
static void launch_stl(const StatLargeArgs& a, int grid, hipStream_t s) {
  const dim3 g((unsigned)grid), b(Cfg::THREADS);
  if (a.ro.pbf16) {
    if (a.ro.dtype == OUT_F32) hipLaunchKernelGGL((stationary_large_kernel<Cfg, BL, 1, OUT_F32>), g, b, 0, s, a);
    else hipLaunchKernelGGL((stationary_large_kernel<Cfg, BL, 1, OUT_BF16>), g, b, 0, s, a);
  } else {
    if (a.ro.dtype == OUT_F32) hipLaunchKernelGGL((stationary_large_kernel<Cfg, BL, 0, OUT_F32>), g, b, 0, s, a);
    else hipLaunchKernelGGL((stationary_large_kernel<Cfg, BL, 0, OUT_BF16>), g, b, 0, s, a);
  }
}

hipError_t launch_stationary_large(int bl, const StatLargeArgs& a0, hipStream_t s) {
  StatLargeArgs a = a0;
  if (a.g.nshard < 1 || a.g.nshard > kMaxShards || a.g.M <= 0 || a.g.N <= 0) return hipErrorInvalidValue;
  a.tiles_m = (a.g.M + CfgStatLarge::BM - 1) / CfgStatLarge::BM;
  a.tiles_n = (a.g.N + CfgStatLarge::BN - 1) / CfgStatLarge::BN;
  const int64_t grid = (int64_t)a.tiles_m * a.tiles_n;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (bl == B_KN) launch_stl<CfgStatLarge, B_KN>(a, (int)grid, s);
  else if (bl == B_NK) launch_stl<CfgStatLarge, B_NK>(a, (int)grid, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}
#endif

}  // namespace tpf
