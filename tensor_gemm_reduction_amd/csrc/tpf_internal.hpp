// Host/device shared descriptions of a launch.  Plain structs passed by value
// as kernel arguments (all well under the 4 KiB kernel-argument limit).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpf_gemm.hpp"

namespace tpf {

constexpr int kMaxShards = 16;
constexpr int kXcds = 8;      // accelerator dies (XCDs) of an MI355X, each with its own L2
constexpr int kMaxChunks = 64;
// GEMM and reduce segments per chunk, plus one copy segment per slice.
constexpr int kMaxSegs = 2 * kMaxChunks + kMaxShards + 2;

// Device control block owned by a handle.  All counters are zero between
// calls: the last workgroup of the persistent kernel to finish clears them.
struct Ctrl {
  int ticket;                 // next task of the work queue
  int done;                   // workgroups that have left the queue
  int status;                 // sticky: bit 0 = a bounded wait gave up
  int pad;
  int ready[kMaxChunks];      // completed GEMM tiles per chunk
  int landed[kMaxShards];     // copied segments per gathered slice
  int sub[kMaxChunks][kXcds]; // claimed tiles of each XCD's share of a chunk
};

// Per-output-tile counters of the tile scheduler (shards finished).  A handle
// owns this many; every count is back at zero when a call ends.
constexpr int kTileCounters = 1 << 17;

enum TaskKind : int { TK_GEMM = 0, TK_REDUCE = 1, TK_COPY = 2 };

// Debug timing perturbation (tpf_debug_set_delay): a producer task with
// index i for which mix(seed, i) % period == 0 executes s_sleep 127 `sleeps`
// times (bounded; about 1 us each) before it publishes or stores its results.
// period == 0 turns it off.
struct DelayArgs {
  uint32_t seed;
  int period;
  int sleeps;
};

// The shard GEMMs of one call.  Tile (shard k, rows, cols) reads A[k] and
// B[k] and writes dst + k * dst_shard_stride.
struct GemmOperands {
  const __bf16* A[kMaxShards];
  const __bf16* B[kMaxShards];
  int64_t lda, ldb;
  int a_rows;                 // rows of each A operand as stored (M, or K for A stored [K][M])
  void* dst;                  // fp32 partials (reducing ops) or the output (AllGather->MatMul)
  void* dstv[kMaxShards];     // if dstv[0] is set: shard k's output at dstv[k] (weight gradients)
  int64_t dst_shard_stride;   // elements
  int64_t ldd;
  int dst_dtype;              // OUT_F32 or OUT_BF16
  int act;                    // 1: GeLU applied to the fp32 result before it is stored
  int M, N, K;                // rows, output width, reduction length per shard
  int b_rows;                 // rows of each B operand (K for KN weights, N for NK)
  int nshard;                 // shard GEMMs (p, or 1 for AllGather->MatMul)
  DelayArgs delay;            // debug: timing perturbation of the producers
};

// Sources of a one-launch AllGather (read in place from the kernarg segment).
struct GatherArgs {
  const char* src[kMaxShards];
  char* dst;
  int64_t slice_bytes;
};

struct ChunkGeom {
  int n;       // number of chunks
  int base;    // rows of every chunk but the last (floor(M / n))
  int M;
  __host__ __device__ int row0(int c) const { return c * base; }
  __host__ __device__ int row1(int c) const { return c == n - 1 ? M : (c + 1) * base; }
};

struct FusedArgs {
  GemmOperands g;
  ReduceOut ro;
  const void* P;              // partials (reducing ops): fp32, or bf16 when ro.pbf16
  int64_t p_stride;           // elements between shards' partials (M * N)
  int p;                      // shards summed by the reduction
  int64_t reduce_elems;      // output elements per separate reduce task (multiple of 4)
  int piggyback;             // 1: each GEMM tile of chunk c > 0 also reduces one slice of chunk c-1
  // AllGather: slice r (slice_bytes) is copied to gathered + r * slice_bytes
  const char* src[kMaxShards];
  char* gathered;
  int64_t slice_bytes;
  int64_t copy_seg_bytes;
  int copy_segs;              // copy tasks per slice
  int slice_rows;             // M / p
  int gather;                 // 1 for AllGather->MatMul
  ChunkGeom ch;
  int nseg;
  int seg_start[kMaxSegs + 1];   // first ticket of each segment; seg_start[nseg] = total tasks
  int seg_info[kMaxSegs];        // kind | (chunk or slice) << 4
  int gemm_tasks[kMaxChunks];    // GEMM tiles of each chunk (the ready target)
  Ctrl* ctrl;
  int64_t spin_limit;
  int unreachable;               // debug: waits target an unreachable count
  // Optional task timeline: one TimelineEvent per ticket (NULL = off).
  struct TimelineEvent* timeline;
  int timeline_cap;
};

// The nshard * tiles_m * tiles_n GEMM tiles of a row range, one workgroup
// each.  Plain shard GEMMs use only g, the rows and the tile grid.  The tile
// scheduler adds the reduction: each output tile has its own counter, and
// the workgroup that completes the last shard of an output tile sums that
// tile.  Nothing waits.
struct TileArgs {
  GemmOperands g;
  int row0, row1;             // output rows covered (the tile grid starts at row0)
  ReduceOut ro;
  const void* P;              // partials (fp32, or bf16 when ro.pbf16), shard k at element k * p_stride
  int64_t p_stride;
  int p;
  int tiles_m, tiles_n;       // output tile grid
  int tasks;                  // p * tiles_m * tiles_n
  int* cnt;                   // kTileCounters per-output-tile counters
  struct TimelineEvent* timeline;
  int timeline_cap;
};

// One persistent-kernel task, stamped with the GPU's constant 100 MHz clock
// (s_memrealtime), so events of different workgroups share one time base.
struct TimelineEvent {
  uint32_t ticket;     // global ticket (queue position)
  uint16_t kind;       // TK_GEMM / TK_REDUCE / TK_COPY
  uint16_t chunk;      // chunk (GEMM, reduce) or slice (copy)
  uint16_t block;      // workgroup id
  uint16_t xcd;        // XCD the workgroup ran on
  uint32_t mid;        // GEMM tasks with a reduce slice: clock ticks from t_start to the end of the GEMM part
  uint64_t t_start;    // after the task was claimed
  uint64_t t_end;      // after the task's results were published
};
static_assert(sizeof(TimelineEvent) == 32, "timeline event layout");

// Tile configurations (chosen from the op's shape only, never from the chunk
// count, so every chunking runs the same per-element arithmetic).
enum CfgId : int { CFG_LARGE = 0, CFG_SMALL = 1, CFG_MID = 2 };
#ifndef TPF_LARGE_STAGES
#define TPF_LARGE_STAGES 2
#endif
#ifndef TPF_LARGE_BK
#define TPF_LARGE_BK 64
#endif
#ifndef TPF_LARGE_WN
#define TPF_LARGE_WN 4
#endif
#ifndef TPF_LARGE_WM
#define TPF_LARGE_WM 2
#endif
#ifndef TPF_LARGE_BM
#define TPF_LARGE_BM 256
#endif
#ifndef TPF_LARGE_BN
#define TPF_LARGE_BN 256
#endif
// The large tiles (one per workgroup, and the persistent kernel's) give A
// one more LDS slot than B (3 x 32 KiB + 2 x 32 KiB = the whole 160 KiB):
// each step's A loads then go out during the MFMAs before the barrier
// (measured 3-7 % faster than two slots each, and the persistent kernel
// 5-14 % faster than with two slots and an L2 line touch of a later step,
// which cost one extra load instruction per step: 8-12 % slower with the
// interleaved loads).
#ifndef TPF_LARGE_STAGES_A
#define TPF_LARGE_STAGES_A 3
#endif
#ifndef TPF_LARGE_STAGES_B
#define TPF_LARGE_STAGES_B 0
#endif
using CfgLarge = TileCfg<TPF_LARGE_BM, TPF_LARGE_BN, TPF_LARGE_WM, TPF_LARGE_WN, TPF_LARGE_STAGES, TPF_LARGE_BK, 2,
                         TPF_LARGE_STAGES_A, TPF_LARGE_STAGES_B>;
#ifndef TPF_FUSED_STAGES
#define TPF_FUSED_STAGES 2
#endif
#ifndef TPF_FUSED_BK
#define TPF_FUSED_BK 64
#endif
#ifndef TPF_FUSED_STAGES_A
#define TPF_FUSED_STAGES_A 3
#endif
// Output-stationary large tiles: 128 x 256 (wave tiles of 64 x 64), so that
// the running sum over the shards and the current shard's accumulators both
// stay in registers; A has the third LDS slot (3 x 16 + 2 x 32 KiB).
#ifndef TPF_STL_CFG
#define TPF_STL_CFG TileCfg<128, 256, 2, 4, 2, 64, 2, 3>
#endif
using CfgStatLarge = TPF_STL_CFG;
using CfgLargeFused = TileCfg<TPF_LARGE_BM, TPF_LARGE_BN, TPF_LARGE_WM, TPF_LARGE_WN, TPF_FUSED_STAGES,
                              TPF_FUSED_BK, 2, TPF_FUSED_STAGES_A>;
#ifndef TPF_SMALL_BM
#define TPF_SMALL_BM 32
#endif
#ifndef TPF_SMALL_BN
#define TPF_SMALL_BN 128
#endif
#ifndef TPF_SMALL_STAGES
#define TPF_SMALL_STAGES 2
#endif
// Decode-shaped row counts (measured on 134 MB of weights, p = 8):
//   M <= 32:  32 x 128 tiles, 2 stages of 20 KiB (measured 4-6 % faster
//             than 3 or 4 stages; 5 or 6 leave room for one workgroup per CU
//             and were 25 % slower);
//   M <= 64:  64 x 256 tiles, 3 stages of 40 KiB: each weight tile is read by
//             one workgroup instead of two (47 % -> 61 % of HBM bandwidth at M = 64).
using CfgSmall = TileCfg<TPF_SMALL_BM, TPF_SMALL_BN, 1, 4, TPF_SMALL_STAGES, 64>;
#ifndef TPF_MID_STAGES
#define TPF_MID_STAGES 3
#endif
using CfgMid = TileCfg<64, 256, 1, 4, TPF_MID_STAGES, 64>;

int cfg_bm(int cfg);
int cfg_bn(int cfg);

// Shard GEMM tiles of rows [row0, row1) into g.dst (no reduction).  bl may
// include A_KM (transposed A) for the large tile configuration only.
hipError_t launch_gemm_rows(int cfg, int bl, const GemmOperands& g, int row0, int row1, hipStream_t s);
hipError_t launch_reduce_rows(const void* P, int64_t stride, int p, int row0, int row1, int N,
                              const ReduceOut& o, int num_cus, hipStream_t s);
hipError_t launch_fused(int cfg, int bl, const FusedArgs& a, int grid, hipStream_t s);
int fused_occupancy(int cfg, int bl);   // resident fused workgroups per CU
// One workgroup per tile; red = 1 for the tile scheduler (partials,
// per-output-tile counters, last arriver sums); red = 2 for the last shard of
// the fold scheduler (a.g holds that shard alone; its epilogue adds the
// partials of the p - 1 shards before it, already in a.P): red = 2 + (fp32
// output) + 2 * (bf16 messages), CFG_LARGE only.
hipError_t launch_tiles(int cfg, int bl, int red, const TileArgs& a, hipStream_t s);
hipError_t launch_copy(const char* src, char* dst, int64_t bytes, int num_cus, hipStream_t s);
// AllGather in one launch: slice r (slice_bytes, a multiple of 16) is copied
// from src[r] to dst + r * slice_bytes, r = 0 .. p-1.
hipError_t launch_gather(const void* const* src, int p, char* dst, int64_t slice_bytes, int num_cus, hipStream_t s);
hipError_t launch_clear_status(Ctrl* c, hipStream_t s);
// Output-stationary single launch of a reducing call with B stored [K][N]
// (the launcher sets the tile grid from the tile shape it picks for M and p).
struct StationaryArgs;
hipError_t launch_stationary(const StationaryArgs& a, int pbf16, int out, hipStream_t s);
// Output-stationary single launch with large tiles (more than 64 rows): one
// workgroup per 128 x 256 output tile runs every shard's K loop and keeps the
// running sum over the shards in registers (g: the p shards' operands, N the
// output width; ro: the AllReduce or ReduceScatter destination).
struct StatLargeArgs {
  GemmOperands g;
  ReduceOut ro;
  int tiles_m, tiles_n;
};
hipError_t launch_stationary_large(int bl, const StatLargeArgs& a, hipStream_t s);

}  // namespace tpf
