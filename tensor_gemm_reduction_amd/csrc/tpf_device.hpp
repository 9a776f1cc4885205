// Device building blocks for gfx950: the bf16 matrix-core GEMM tile, the
// fixed-order cross-shard reduction, the gather copy and the small
// synchronisation helpers used by the persistent scheduler.
//
// GEMM tile.  A workgroup of 256 threads (four wave64s arranged WAVES_M x
// WAVES_N) computes a BM x BN block of C = A B with A row-major [M][K] and B
// either row-major [K][N] ("KN", the forward weight W_k) or row-major [N][K]
// ("NK", a weight used transposed as in dX = dY W^T).  K advances in steps of
// BK through two LDS stages: the next step's global loads are issued before
// the current step's MFMAs and written to the other stage afterwards, so one
// barrier per step suffices.  In LDS both operands are stored K-contiguous
// ([row][k], 16-byte chunks XOR-swizzled by row) because every lane of
// v_mfma_f32_32x32x16_bf16 consumes eight consecutive k of one row (A) or
// one column (B).  A "KN" B tile is transposed on its way to LDS: each thread
// loads an 8(k) x 8(n) block with eight 16-byte loads and writes eight
// 16-byte k-runs.
//
// Every output element is accumulated by the same sequence of MFMAs in
// increasing k, whatever the tile shape, the tile origin or the number of
// valid rows, so the result does not depend on how the rows are chunked.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

enum BLayout : int { B_KN = 0, B_NK = 1 };
enum OutKind : int { OUT_F32 = 1, OUT_BF16 = 0 };

// Round-to-nearest-even binary32 -> bfloat16 (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile of 32x32 MFMA blocks");
  static constexpr int KCH = BK / 8;                  // 16-byte chunks per LDS row
  static_assert(BK % 64 == 0, "swizzle needs >= 8 chunks per row");
  static constexpr int A_LOADS = BM * KCH / kThreads; // 16-byte loads per thread for A (and NK B)
  static_assert((BM * KCH) % kThreads == 0, "A tile must split evenly");
  static constexpr int BN_LOADS_NK = BN * KCH / kThreads;
  static_assert((BN * KCH) % kThreads == 0, "B tile must split evenly");
  static constexpr int B_BLOCKS_KN = (BK / 8) * (BN / 8);       // 8x8 blocks of a KN tile
  static constexpr int B_ITERS_KN = (B_BLOCKS_KN + kThreads - 1) / kThreads;
  static constexpr int LDS_A = BM * BK * 2;
  static constexpr int LDS_B = BN * BK * 2;
  static constexpr int LDS_STAGE = LDS_A + LDS_B;
  static constexpr int LDS_BYTES = 2 * LDS_STAGE;
};

__device__ __forceinline__ int swz(int row, int kc) { return kc ^ (row & 7); }

// Operand description of one tile job.
struct TileJob {
  const __bf16* A;   // row m0 of this tile's A panel is A + m0 * lda
  const __bf16* B;
  int64_t lda, ldb;
  int m0;            // first row (absolute)
  int rows;          // valid rows from m0 (<= BM)
  int n0;            // first column
  int N, K;          // output width and reduction length
};

template <class Cfg>
struct Frag {
  f32x16_t acc[Cfg::TM][Cfg::TN];
};

template <class Cfg, int BL>
struct Loader {
  u32x4_t a[Cfg::A_LOADS];
  u32x4_t b[BL == B_KN ? Cfg::B_ITERS_KN * 8 : Cfg::BN_LOADS_NK];

  __device__ __forceinline__ void load(const TileJob& j, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) {
      const int q = tid + i * kThreads;
      const int m = q / Cfg::KCH, kc = q % Cfg::KCH;
      const int gk = k0 + kc * 8;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (m < j.rows && gk < j.K)
        v = *reinterpret_cast<const u32x4_t*>(j.A + (int64_t)(j.m0 + m) * j.lda + gk);
      a[i] = v;
    }
    if constexpr (BL == B_NK) {
#pragma unroll
      for (int i = 0; i < Cfg::BN_LOADS_NK; ++i) {
        const int q = tid + i * kThreads;
        const int n = q / Cfg::KCH, kc = q % Cfg::KCH;
        const int gk = k0 + kc * 8;
        const int gn = j.n0 + n;
        u32x4_t v = {0u, 0u, 0u, 0u};
        if (gn < j.N && gk < j.K)
          v = *reinterpret_cast<const u32x4_t*>(j.B + (int64_t)gn * j.ldb + gk);
        b[i] = v;
      }
    } else {
#pragma unroll
      for (int it = 0; it < Cfg::B_ITERS_KN; ++it) {
        const int blk = tid + it * kThreads;
        const int kb = blk % (Cfg::BK / 8), nb = blk / (Cfg::BK / 8);
        const int gn = j.n0 + nb * 8;
        const bool colok = (blk < Cfg::B_BLOCKS_KN) && (gn < j.N);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int gk = k0 + kb * 8 + r;
          u32x4_t v = {0u, 0u, 0u, 0u};
          if (colok && gk < j.K)
            v = *reinterpret_cast<const u32x4_t*>(j.B + (int64_t)gk * j.ldb + gn);
          b[it * 8 + r] = v;
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* stage, int tid) const {
    char* la = stage;
    char* lb = stage + Cfg::LDS_A;
#pragma unroll
    for (int i = 0; i < Cfg::A_LOADS; ++i) {
      const int q = tid + i * kThreads;
      const int m = q / Cfg::KCH, kc = q % Cfg::KCH;
      *reinterpret_cast<u32x4_t*>(la + (m * Cfg::KCH + swz(m, kc)) * 16) = a[i];
    }
    if constexpr (BL == B_NK) {
#pragma unroll
      for (int i = 0; i < Cfg::BN_LOADS_NK; ++i) {
        const int q = tid + i * kThreads;
        const int n = q / Cfg::KCH, kc = q % Cfg::KCH;
        *reinterpret_cast<u32x4_t*>(lb + (n * Cfg::KCH + swz(n, kc)) * 16) = b[i];
      }
    } else {
#pragma unroll
      for (int it = 0; it < Cfg::B_ITERS_KN; ++it) {
        const int blk = tid + it * kThreads;
        if (blk < Cfg::B_BLOCKS_KN) {
          const int kb = blk % (Cfg::BK / 8), nb = blk / (Cfg::BK / 8);
          const u32x4_t* r = &b[it * 8];
          // Transpose the 8(k) x 8(n) block of 16-bit values: column j of the
          // block becomes one 16-byte run of eight consecutive k.
#pragma unroll
          for (int jn = 0; jn < 8; ++jn) {
            const int w = jn >> 1;
            u32x4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t lo = r[2 * q][w], hi = r[2 * q + 1][w];
              o[q] = (jn & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
            }
            const int n = nb * 8 + jn;
            *reinterpret_cast<u32x4_t*>(lb + (n * Cfg::KCH + swz(n, kb)) * 16) = o;
          }
        }
      }
    }
  }
};

template <class Cfg>
__device__ __forceinline__ void mma_stage(Frag<Cfg>& f, const char* stage, int wm, int wn, int lane) {
  const char* la = stage;
  const char* lb = stage + Cfg::LDS_A;
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int s = 0; s < Cfg::BK / 16; ++s) {
    const int kc = s * 2 + half;
    bf16x8_t av[Cfg::TM], bv[Cfg::TN];
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = wm * Cfg::WM + i * 32 + r32;
      av[i] = *reinterpret_cast<const bf16x8_t*>(la + (m * Cfg::KCH + swz(m, kc)) * 16);
    }
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn) {
      const int n = wn * Cfg::WN + jn * 32 + r32;
      bv[jn] = *reinterpret_cast<const bf16x8_t*>(lb + (n * Cfg::KCH + swz(n, kc)) * 16);
    }
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
      for (int jn = 0; jn < Cfg::TN; ++jn)
        f.acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[jn], f.acc[i][jn], 0, 0, 0);
    // Keep each k16 step's fragments short-lived: without this fence the
    // scheduler hoists every step's LDS reads ahead and runs out of VGPRs.
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Full K loop of one tile into registers.  `lds` holds two stages.
// Ends with a barrier so the caller may reuse LDS immediately.
template <class Cfg, int BL>
__device__ __forceinline__ void gemm_tile(Frag<Cfg>& f, const TileJob& j, char* lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) f.acc[i][jn][v] = 0.0f;

  const int nk = (j.K + Cfg::BK - 1) / Cfg::BK;
  Loader<Cfg, BL> ld;
  ld.load(j, 0, tid);
  ld.store(lds, tid);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = lds + (kt & 1) * Cfg::LDS_STAGE;
    char* nxt = lds + ((kt + 1) & 1) * Cfg::LDS_STAGE;
    const bool more = kt + 1 < nk;
    if (more) ld.load(j, (kt + 1) * Cfg::BK, tid);
    mma_stage<Cfg>(f, cur, wm, wn, lane);
    if (more) ld.store(nxt, tid);
    __syncthreads();
  }
}

// Write the accumulators of one tile.  Element (row, col) of the 32x32 MFMA
// block held in register v of lane l: col = l % 32,
// row = 8 * (v / 4) + 4 * (l / 32) + v % 4.
template <class Cfg, int OUT>
__device__ __forceinline__ void store_tile(const Frag<Cfg>& f, const TileJob& j, void* out, int64_t ldo) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn) {
      const int col = j.n0 + wn * Cfg::WN + jn * 32 + r32;
      if (col >= j.N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * Cfg::WM + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (row < j.rows) {
          const int64_t off = (int64_t)(j.m0 + row) * ldo + col;
          if constexpr (OUT == OUT_F32)
            reinterpret_cast<float*>(out)[off] = f.acc[i][jn][v];
          else
            reinterpret_cast<uint16_t*>(out)[off] = (uint16_t)f32_to_bf16_bits(f.acc[i][jn][v]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fixed-order cross-shard reduction.
//
// Element e of the output (row-major, rows [row0, row1) of an [M][N] result)
// is ((P_0[e] + P_1[e]) + P_2[e]) + ... + P_{p-1}[e] in fp32, then rounded
// once.  P_k[e] lives at P + k * shard_stride + e.
// ---------------------------------------------------------------------------
struct ReduceOut {
  void* y[16];          // AllReduce: y[0] is the full [M][N]; ReduceScatter: p slices
  int scatter;          // 0: AllReduce layout, 1: ReduceScatter layout
  int rows_per_slice;   // M / p for ReduceScatter
  int dtype;            // OUT_F32 or OUT_BF16
};

template <int OUT>
__device__ __forceinline__ void reduce_store4(const ReduceOut& o, int64_t e, int N, f32x4_t s) {
  void* base;
  int64_t off;
  if (o.scatter) {
    const int64_t row = e / N;
    const int sl = (int)(row / o.rows_per_slice);
    base = o.y[sl];
    off = e - (int64_t)sl * o.rows_per_slice * N;
  } else {
    base = o.y[0];
    off = e;
  }
  if constexpr (OUT == OUT_F32) {
    *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + off) = s;
  } else {
    u32x2_t w;
    w[0] = f32_to_bf16_bits(s[0]) | (f32_to_bf16_bits(s[1]) << 16);
    w[1] = f32_to_bf16_bits(s[2]) | (f32_to_bf16_bits(s[3]) << 16);
    *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(base) + off) = w;
  }
}

// Reduce elements [e0, e1) (multiples of 4) with `nthr` cooperating threads
// numbered `t`.  P is compile-time when PP > 0 (loads of all shards are then
// issued together), run-time otherwise.
template <int PP, int OUT>
__device__ __forceinline__ void reduce_range(const float* __restrict__ P, int64_t shard_stride, int p,
                                             int64_t e0, int64_t e1, int N, const ReduceOut& o,
                                             int64_t t, int64_t nthr) {
  constexpr int U = 2;   // float4 groups per thread per iteration
  const int np = PP > 0 ? PP : p;
  for (int64_t g = e0 + t * 4; g < e1; g += nthr * 4 * U) {
    f32x4_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = g + (int64_t)u * nthr * 4;
      if (e < e1) s[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(P + e));
    }
    if constexpr (PP > 0) {
      f32x4_t v[PP > 1 ? PP - 1 : 1][U];
#pragma unroll
      for (int k = 1; k < PP; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t e = g + (int64_t)u * nthr * 4;
          if (e < e1)
            v[k - 1][u] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4_t*>(P + (int64_t)k * shard_stride + e));
        }
#pragma unroll
      for (int k = 1; k < PP; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] = s[u] + v[k - 1][u];
    } else {
      for (int k = 1; k < np; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t e = g + (int64_t)u * nthr * 4;
          if (e < e1)
            s[u] = s[u] + __builtin_nontemporal_load(
                              reinterpret_cast<const f32x4_t*>(P + (int64_t)k * shard_stride + e));
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = g + (int64_t)u * nthr * 4;
      if (e < e1) reduce_store4<OUT>(o, e, N, s[u]);
    }
  }
}

// Copy bytes [b0, b1) (multiples of 16) from src to dst with nthr threads.
__device__ __forceinline__ void copy_range(const char* __restrict__ src, char* __restrict__ dst,
                                           int64_t b0, int64_t b1, int64_t t, int64_t nthr) {
  constexpr int U = 4;
  for (int64_t g = b0 + t * 16; g < b1; g += nthr * 16 * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = g + (int64_t)u * nthr * 16;
      if (b < b1) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + b));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t b = g + (int64_t)u * nthr * 16;
      if (b < b1) *reinterpret_cast<u32x4_t*>(dst + b) = v[u];
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-workgroup signalling (agent scope: visible across all XCDs' L2s).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int atomic_load_acquire(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_add_release(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_add_acq_rel(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void atomic_store_relaxed(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void fence_release_agent() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire_agent() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }

}  // namespace tpf
