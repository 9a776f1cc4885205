// Device building blocks shared by the kernels: vector types, bf16 rounding,
// the fixed-order cross-shard reduction, the gather copy and the
// cross-workgroup signalling helpers.  The GEMM tile lives in tpf_gemm.hpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpf {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Operand layouts of a GEMM tile, as one template parameter: bit 0 is the B
// layout (B_KN: B stored [K][N]; B_NK: [N][K]); bit 1 (A_KM) stores A as
// [K][M] (the contraction index runs down the rows) instead of [M][K].
enum BLayout : int { B_KN = 0, B_NK = 1, A_KM = 2 };
constexpr int b_layout(int L) { return L & 1; }
constexpr bool a_trans(int L) { return (L & A_KM) != 0; }
enum OutKind : int { OUT_F32 = 1, OUT_BF16 = 0 };

// Round-to-nearest-even binary32 -> bfloat16 (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---------------------------------------------------------------------------
// Fixed-order cross-shard reduction.
//
// Element e of the output (row-major, rows [row0, row1) of an [M][N] result)
// is ((P_0[e] + P_1[e]) + P_2[e]) + ... + P_{p-1}[e] in fp32, then rounded
// once.  P_k[e] is element k * shard_stride + e of the partials, which are
// fp32, or bf16 for the 2-byte message variant (widened exactly to fp32).
// ---------------------------------------------------------------------------
struct ReduceOut {
  void* y[16];          // AllReduce: y[0] is the full [M][N]; ReduceScatter: p slices
  int scatter;          // 0: AllReduce layout, 1: ReduceScatter layout
  int rows_per_slice;   // M / p for ReduceScatter
  int dtype;            // OUT_F32 or OUT_BF16
  int pbf16;            // partials ("messages") stored as bf16 instead of fp32
};

// Four consecutive partials starting at element e, widened to fp32.  PB = 1:
// the partials are bf16 (8 bytes), PB = 0: fp32 (16 bytes).
template <int PB>
__device__ __forceinline__ f32x4_t load_partial4(const void* P, int64_t e) {
  if constexpr (PB) {
    const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(
        reinterpret_cast<const uint16_t*>(P) + e));
    f32x4_t v;
    v[0] = __uint_as_float(w[0] << 16);
    v[1] = __uint_as_float(w[0] & 0xffff0000u);
    v[2] = __uint_as_float(w[1] << 16);
    v[3] = __uint_as_float(w[1] & 0xffff0000u);
    return v;
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(P) + e));
  }
}

template <int OUT>
__device__ __forceinline__ void reduce_store4(const ReduceOut& o, int64_t e, int N, f32x4_t s) {
  void* base;
  int64_t off;
  if (o.scatter) {
    // Outputs hold fewer than 2^29 elements (each fp32 partial is below
    // 2 GiB), so one 32-bit division finds the slice.
    const uint32_t slice = (uint32_t)o.rows_per_slice * (uint32_t)N;
    const uint32_t sl = (uint32_t)e / slice;
    base = o.y[sl];
    off = (int64_t)((uint32_t)e - sl * slice);
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
template <int PP, int OUT, int PB>
__device__ __forceinline__ void reduce_range(const void* __restrict__ P, int64_t shard_stride, int p,
                                             int64_t e0, int64_t e1, int N, const ReduceOut& o,
                                             int64_t t, int64_t nthr) {
  // About sixteen 16-byte loads in flight per thread.
  constexpr int U = PP >= 8 ? 2 : (PP >= 4 ? 4 : (PP >= 2 ? 8 : 4));
  const int np = PP > 0 ? PP : p;
  for (int64_t g = e0 + t * 4; g < e1; g += nthr * 4 * U) {
    f32x4_t s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = g + (int64_t)u * nthr * 4;
      if (e < e1) s[u] = load_partial4<PB>(P, e);
    }
    if constexpr (PP > 0) {
      f32x4_t v[PP > 1 ? PP - 1 : 1][U];
#pragma unroll
      for (int k = 1; k < PP; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t e = g + (int64_t)u * nthr * 4;
          if (e < e1) v[k - 1][u] = load_partial4<PB>(P, (int64_t)k * shard_stride + e);
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
          if (e < e1) s[u] = s[u] + load_partial4<PB>(P, (int64_t)k * shard_stride + e);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = g + (int64_t)u * nthr * 4;
      if (e < e1) reduce_store4<OUT>(o, e, N, s[u]);
    }
  }
}

// The same fixed-order sum over one rectangular output tile: rows
// [m0, m0 + rows) and columns [n0, n0 + ncols) (ncols a multiple of 4) of the
// [M][N] result, with `nthr` threads numbered `t`.  Per element it performs
// exactly the additions of reduce_range, so both give identical bits.
template <int PP, int OUT, int PB>
__device__ __forceinline__ void reduce_tile(const void* __restrict__ P, int64_t shard_stride, int p, int m0,
                                            int rows, int n0, int ncols, int N, const ReduceOut& o, int t, int nthr) {
  constexpr int U = PP >= 8 ? 2 : (PP >= 4 ? 4 : (PP >= 2 ? 8 : 4));
  const int np = PP > 0 ? PP : p;
  const int gpr = ncols / 4;               // 4-element groups per tile row
  const int total = rows * gpr;
  for (int g = t; g < total; g += nthr * U) {
    f32x4_t s[U];
    int64_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = g + u * nthr;
      const int r = i / gpr;
      e[u] = (int64_t)(m0 + r) * N + n0 + 4 * (i - r * gpr);
      if (i < total) s[u] = load_partial4<PB>(P, e[u]);
    }
    if constexpr (PP > 0) {
      f32x4_t v[PP > 1 ? PP - 1 : 1][U];
#pragma unroll
      for (int k = 1; k < PP; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (g + u * nthr < total) v[k - 1][u] = load_partial4<PB>(P, (int64_t)k * shard_stride + e[u]);
#pragma unroll
      for (int k = 1; k < PP; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) s[u] = s[u] + v[k - 1][u];
    } else {
      for (int k = 1; k < np; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (g + u * nthr < total) s[u] = s[u] + load_partial4<PB>(P, (int64_t)k * shard_stride + e[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (g + u * nthr < total) reduce_store4<OUT>(o, e[u], N, s[u]);
  }
}

// Eight consecutive bf16 partials (16 bytes) at element e, widened to fp32.
__device__ __forceinline__ void load_partial8_bf16(const void* P, int64_t e, f32x4_t& lo, f32x4_t& hi) {
  const u32x4_t w =
      __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(P) + e));
  lo[0] = __uint_as_float(w[0] << 16);
  lo[1] = __uint_as_float(w[0] & 0xffff0000u);
  lo[2] = __uint_as_float(w[1] << 16);
  lo[3] = __uint_as_float(w[1] & 0xffff0000u);
  hi[0] = __uint_as_float(w[2] << 16);
  hi[1] = __uint_as_float(w[2] & 0xffff0000u);
  hi[2] = __uint_as_float(w[3] << 16);
  hi[3] = __uint_as_float(w[3] & 0xffff0000u);
}

// reduce_range for bf16 partials, eight elements (one 16-byte load per shard)
// per thread and step; [e0, e1) are multiples of 8.  The same additions in
// the same order as reduce_range, so the same bits.
template <int PP, int OUT>
__device__ __forceinline__ void reduce_range_b16(const void* __restrict__ P, int64_t shard_stride, int p,
                                                 int64_t e0, int64_t e1, int N, const ReduceOut& o, int64_t t,
                                                 int64_t nthr) {
  constexpr int U = PP >= 8 ? 1 : (PP >= 4 ? 2 : (PP >= 2 ? 4 : 2));
  const int np = PP > 0 ? PP : p;
  for (int64_t g = e0 + t * 8; g < e1; g += nthr * 8 * U) {
    f32x4_t lo[U], hi[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = g + (int64_t)u * nthr * 8;
      if (e < e1) load_partial8_bf16(P, e, lo[u], hi[u]);
    }
    if constexpr (PP > 0) {
      f32x4_t vl[PP > 1 ? PP - 1 : 1][U], vh[PP > 1 ? PP - 1 : 1][U];
#pragma unroll
      for (int k = 1; k < PP; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t e = g + (int64_t)u * nthr * 8;
          if (e < e1) load_partial8_bf16(P, (int64_t)k * shard_stride + e, vl[k - 1][u], vh[k - 1][u]);
        }
#pragma unroll
      for (int k = 1; k < PP; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          lo[u] = lo[u] + vl[k - 1][u];
          hi[u] = hi[u] + vh[k - 1][u];
        }
    } else {
      for (int k = 1; k < np; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t e = g + (int64_t)u * nthr * 8;
          if (e < e1) {
            f32x4_t a, b;
            load_partial8_bf16(P, (int64_t)k * shard_stride + e, a, b);
            lo[u] = lo[u] + a;
            hi[u] = hi[u] + b;
          }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = g + (int64_t)u * nthr * 8;
      if (e < e1) {
        reduce_store4<OUT>(o, e, N, lo[u]);
        reduce_store4<OUT>(o, e + 4, N, hi[u]);
      }
    }
  }
}

// reduce_tile for bf16 partials, eight elements per thread and step (ncols is
// a multiple of 8).
template <int PP, int OUT>
__device__ __forceinline__ void reduce_tile_b16(const void* __restrict__ P, int64_t shard_stride, int p, int m0,
                                                int rows, int n0, int ncols, int N, const ReduceOut& o, int t,
                                                int nthr) {
  constexpr int U = PP >= 8 ? 1 : (PP >= 4 ? 2 : (PP >= 2 ? 4 : 2));
  const int np = PP > 0 ? PP : p;
  const int gpr = ncols / 8;
  const int total = rows * gpr;
  for (int g = t; g < total; g += nthr * U) {
    f32x4_t lo[U], hi[U];
    int64_t e[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = g + u * nthr;
      const int r = i / gpr;
      e[u] = (int64_t)(m0 + r) * N + n0 + 8 * (i - r * gpr);
      if (i < total) load_partial8_bf16(P, e[u], lo[u], hi[u]);
    }
    for (int k = 1; k < np; ++k)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (g + u * nthr < total) {
          f32x4_t a, b;
          load_partial8_bf16(P, (int64_t)k * shard_stride + e[u], a, b);
          lo[u] = lo[u] + a;
          hi[u] = hi[u] + b;
        }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (g + u * nthr < total) {
        reduce_store4<OUT>(o, e[u], N, lo[u]);
        reduce_store4<OUT>(o, e[u] + 4, N, hi[u]);
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
