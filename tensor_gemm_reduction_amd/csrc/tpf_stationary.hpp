// Output-stationary single-launch path for reducing calls with few rows
// (decode-shaped M): one workgroup per output tile of BM = 32 * RB rows and
// BN = 32 * CB columns computes every shard's partial of that tile and folds
// them on chip, so no partial ever goes to memory and there is no second
// launch.
//
//  * Eight waves per workgroup; wave w computes the partials of shards
//    w, w + 8 (p <= 16), each as the same MFMA chain as every other path:
//    v_mfma_f32_32x32x16_bf16 over k = 0, 16, 32, ... from a zero
//    accumulator, so each shard's partial has the same bits as the partial
//    the shard-GEMM kernels store.
//  * The weight tile of a shard (BK k x BN n per step, row-major [K][N]) is
//    streamed by its wave alone through a private ring of STAGES LDS buffers
//    (buffer_load_dwordx4 ... lds) and read with the gfx950 transpose read;
//    no barrier is needed inside the K loop because no other wave touches the
//    ring.  Rows of BN bf16 are stored with their 32-byte blocks XOR-swizzled
//    by (k mod 4) when a row holds more than two blocks, so the four rows a
//    16-lane group reads with one transpose read sit in distinct banks.
//  * The activation rows (A operand: lane l holds row l % 32, eight
//    consecutive k) are loaded straight into registers, 16 bytes per lane and
//    k slice, STAGES - 1 steps ahead; rows past M and k past K read as zero.
//  * After every wave's K loops, the partials go to LDS (the rings are free
//    by then) as P[k][BM][BN] fp32 (rounded to bf16 first for 2-byte
//    messages: the message that shard would have sent), and the workgroup
//    sums them element by element in shard order k = 0..p-1 in fp32 -- the
//    additions of the reduction kernel, in its order -- rounds once and
//    stores to the AllReduce or ReduceScatter destination.
#pragma once

#include "tpf_gemm.hpp"

namespace tpf {

constexpr int kStWaves = 8;                 // waves per workgroup
constexpr int kStMaxShardsPerWave = 2;      // p <= 16
constexpr int kStLdsBytes = 128 * 1024;     // weight rings during the K loops, partials after them

struct StationaryArgs {
  const __bf16* A[kMaxShards];   // X_k [M][K]
  const __bf16* B[kMaxShards];   // W_k [K][N]
  int M, N, K, p;
  int tiles_m, tiles_n;
  ReduceOut ro;
};

// s_waitcnt vmcnt(steps * PER) for steps in 0..3 (PER * 3 <= 63).
template <int PER>
__device__ __forceinline__ void st_wait_steps(int steps) {
#define TPF_STVM(N) __builtin_amdgcn_s_waitcnt((((N) & 15) | 0x70 | 0xF00 | (((N) >> 4) << 14)))
  static_assert(3 * PER <= 63, "vmcnt range");
  switch (steps) {
    case 0: TPF_STVM(0); break;
    case 1: TPF_STVM(PER); break;
    case 2: TPF_STVM(2 * PER); break;
    default: TPF_STVM(3 * PER); break;
  }
#undef TPF_STVM
  asm volatile("" ::: "memory");   // no LDS read may be moved above the wait
}

// Tile and pipeline shape: RB row blocks and CB column blocks of 32, K steps
// of BK, STAGES ring slots, cache-policy bits WAUX on the weight loads.
template <int RB_, int CB_, int BK_, int STAGES_, int WAUX_ = 0>
struct StCfg {
  static constexpr int RB = RB_, CB = CB_, BK = BK_, STAGES = STAGES_, WAUX = WAUX_;
  static constexpr int BM = 32 * RB, BN = 32 * CB;
  static constexpr int SUB = BK / 16;                   // 16-wide k slices per step
  static constexpr int ROW_BYTES = BN * 2;              // one k row of the weight tile
  static constexpr int STAGE_BYTES = BK * ROW_BYTES;
  static constexpr int W_LOADS = STAGE_BYTES / 1024;    // 1 KiB per buffer_load ... lds
  static constexpr int LANES_PER_ROW = ROW_BYTES / 16;
  static constexpr int ROWS_PER_LOAD = 64 / LANES_PER_ROW;
  static constexpr bool SWZ = CB >= 2;                  // rows of 4+ blocks of 32 bytes
  static constexpr int PER = SUB * RB + W_LOADS;        // vector-memory loads per step
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  static_assert(CB == 1 || CB == 2 || CB == 4, "32, 64 or 128 columns");
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 steps in flight");
  static_assert(kStWaves * STAGES * STAGE_BYTES <= kStLdsBytes, "weight rings fit the LDS");
  static_assert(STAGE_BYTES % 1024 == 0, "whole 1 KiB loads");
};

// Physical byte offset of logical 16-byte chunk c (8 columns) of weight-tile
// row k.
template <class C>
__device__ __forceinline__ int st_chunk_off(int k, int c) {
  if constexpr (C::SWZ) {
    const int blk = (c >> 1) ^ (k & 3);
    return k * C::ROW_BYTES + (blk * 2 + (c & 1)) * 16;
  } else {
    return k * C::ROW_BYTES + c * 16;
  }
}

template <class C>
struct StPipe {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t a_off[C::RB];         // byte offset of this lane's A chunk at k = 0 (kOOB: row past M)
  uint32_t b_off[C::W_LOADS];    // byte offset of this lane's weight chunk at k = 0 (kOOB: column past N)
  int K;
  uint32_t ldb_bytes;
  char* ring;                    // this wave's STAGES x STAGE_BYTES
  bf16x8_t a[C::STAGES][C::SUB][C::RB];

  // Issue the loads of step t into ring slot (and A register set) st.
  __device__ __forceinline__ void issue(int st, int t) {
    const int lane = threadIdx.x & 63;
    const int k0 = t * C::BK;
    // A: SUB 16-wide k slices, RB row blocks each; a_off already holds this
    // lane's row and its eight-element k chunk, the slice adds k0 + 16 s.
#pragma unroll
    for (int s = 0; s < C::SUB; ++s) {
      const int kb = k0 + s * 16;
      const bool k_ok = kb + 8 * (lane >> 5) < K;       // K is a multiple of 8: whole chunks
#pragma unroll
      for (int i = 0; i < C::RB; ++i) {
        const uint32_t off = (a_off[i] != kOOB && k_ok) ? a_off[i] + (uint32_t)kb * 2u : kOOB;
        a[st][s][i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
      }
    }
    // weights: W_LOADS loads of 1 KiB into this wave's ring slot; rows past K
    // fall outside the resource and read as zeros
    char* dst = ring + st * C::STAGE_BYTES;
#pragma unroll
    for (int q = 0; q < C::W_LOADS; ++q) {
      const uint32_t off = b_off[q] != kOOB ? b_off[q] + (uint32_t)k0 * ldb_bytes : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(dst + q * 1024), 16, (int)off, 0, C::WAUX, 0);
    }
  }
};

// One step: the MFMAs of step t from ring slot ST (loads of steps up to
// t + STAGES - 1 issued on entry to the step).
template <class C, int ST>
__device__ __forceinline__ void st_step(f32x16_t (&acc)[C::RB][C::CB], StPipe<C>& P, int t, int nk) {
  if (t + C::STAGES - 1 < nk) P.issue((ST + C::STAGES - 1) % C::STAGES, t + C::STAGES - 1);
  st_wait_steps<C::PER>(min(C::STAGES - 1, nk - 1 - t));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, jl = lane & 15;
  const int r = jl >> 2, q = jl & 3;
  const char* slot = P.ring + ST * C::STAGE_BYTES;
#pragma unroll
  for (int s = 0; s < C::SUB; ++s) {
    const int k = s * 16 + (g >> 1) * 8 + r;          // this lane's row for the first read; +4 for the second
    bf16x8_t b[C::CB];
#pragma unroll
    for (int jn = 0; jn < C::CB; ++jn) {
      const int c = jn * 4 + (g & 1) * 2 + (q >> 1);   // 16-byte chunk holding columns n .. n+3
      const int off = st_chunk_off<C>(k, c) + (q & 1) * 8;   // (k + 4) & 3 == k & 3: same swizzle
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)((lds_void_t*)(slot + off)));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4_t*)((lds_void_t*)(slot + off + 4 * C::ROW_BYTES)));
      b[jn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
#pragma unroll
    for (int i = 0; i < C::RB; ++i)
#pragma unroll
      for (int jn = 0; jn < C::CB; ++jn)
        acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(P.a[ST][s][i], b[jn], acc[i][jn], 0, 0, 0);
  }
}

template <class C, int ST>
__device__ __forceinline__ void st_steps(f32x16_t (&acc)[C::RB][C::CB], StPipe<C>& P, int t, int nk) {
  if constexpr (ST < C::STAGES) {
    if (t + ST < nk) {
      st_step<C, ST>(acc, P, t + ST, nk);
      st_steps<C, ST + 1>(acc, P, t, nk);
    }
  }
}

template <class C, int S>
__device__ __forceinline__ void st_prologue(StPipe<C>& P, int nk) {
  if constexpr (S < C::STAGES - 1) {
    if (S < nk) P.issue(S, S);
    st_prologue<C, S + 1>(P, nk);
  }
}

// Shard k's partial of the tile (m0, n0): the full K loop into acc.
template <class C>
__device__ __forceinline__ void st_shard(f32x16_t (&acc)[C::RB][C::CB], const StationaryArgs& a, int k, int m0,
                                         int n0, char* ring) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
#pragma unroll
    for (int jn = 0; jn < C::CB; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jn][v] = 0.0f;
  StPipe<C> P;
  P.K = a.K;
  P.ldb_bytes = (uint32_t)a.N * 2u;
  P.ra = make_rsrc(a.A[k], (int64_t)a.M * a.K * 2);
  P.rb = make_rsrc(a.B[k], (int64_t)a.K * a.N * 2);
  P.ring = ring;
#pragma unroll
  for (int i = 0; i < C::RB; ++i) {
    const int m = m0 + i * 32 + (lane & 31);
    P.a_off[i] = m < a.M ? (uint32_t)(((int64_t)m * a.K + 8 * (lane >> 5)) * 2) : kOOB;
  }
  // Weight load q, lane l lands at byte q * 1024 + 16 l of the ring slot:
  // tile row k = q * ROWS_PER_LOAD + l / LANES_PER_ROW, physical chunk
  // l % LANES_PER_ROW, which holds logical chunk (8 columns) c.
#pragma unroll
  for (int q = 0; q < C::W_LOADS; ++q) {
    const int row = q * C::ROWS_PER_LOAD + lane / C::LANES_PER_ROW;
    const int pc = lane % C::LANES_PER_ROW;
    int c = pc;
    if constexpr (C::SWZ) c = (((pc >> 1) ^ (row & 3)) << 1) | (pc & 1);
    const int col = n0 + 8 * c;
    P.b_off[q] = col < a.N ? (uint32_t)(((int64_t)row * a.N + col) * 2) : kOOB;
  }
  const int nk = (a.K + C::BK - 1) / C::BK;
  st_prologue<C, 0>(P, nk);
  for (int t = 0; t < nk; t += C::STAGES) st_steps<C, 0>(acc, P, t, nk);
}

template <int PB>
__device__ __forceinline__ float st_message(float acc) {
  if constexpr (PB) return __uint_as_float(f32_to_bf16_bits(acc) << 16);
  else return acc;
}

// Largest p whose partials of one tile fit the LDS at once.
template <class C>
constexpr int st_max_shards() {
  return kStLdsBytes / (C::BM * C::BN * 4) < kMaxShards ? kStLdsBytes / (C::BM * C::BN * 4) : kMaxShards;
}

template <class C, int PB, int OUT>
__device__ __forceinline__ void stationary_tile(const StationaryArgs& a, char* lds, int tile) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  char* ring = lds + wv * (C::STAGES * C::STAGE_BYTES);
  f32x16_t acc[kStMaxShardsPerWave][C::RB][C::CB];
#pragma unroll
  for (int j = 0; j < kStMaxShardsPerWave; ++j)
    if (wv + j * kStWaves < a.p) st_shard<C>(acc[j], a, wv + j * kStWaves, m0, n0, ring);
  __syncthreads();                                  // every ring is idle: the LDS holds the partials now
  float* part = reinterpret_cast<float*>(lds);      // [p][BM][BN]
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int j = 0; j < kStMaxShardsPerWave; ++j) {
    const int k = wv + j * kStWaves;
    if (k < a.p) {
      float* pk = part + (int64_t)k * C::BM * C::BN;
#pragma unroll
      for (int i = 0; i < C::RB; ++i)
#pragma unroll
        for (int jn = 0; jn < C::CB; ++jn)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
            pk[row * C::BN + jn * 32 + r32] = st_message<PB>(acc[j][i][jn][v]);
          }
    }
  }
  __syncthreads();
  // the fold: four consecutive columns per thread and pass, shards in order
  constexpr int GROUPS = C::BM * C::BN / 4;
  for (int t = threadIdx.x; t < GROUPS; t += kStWaves * 64) {
    const int row = t / (C::BN / 4), c = (t % (C::BN / 4)) * 4;
    if (m0 + row < a.M && n0 + c < a.N) {
      f32x4_t s = *reinterpret_cast<const f32x4_t*>(part + row * C::BN + c);
      for (int k = 1; k < a.p; ++k)
        s = s + *reinterpret_cast<const f32x4_t*>(part + ((int64_t)k * C::BM + row) * C::BN + c);
      reduce_store4<OUT>(a.ro, (int64_t)(m0 + row) * a.N + n0 + c, a.N, s);
    }
  }
}

}  // namespace tpf
