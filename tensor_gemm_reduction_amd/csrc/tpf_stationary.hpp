// Output-stationary single-launch path for reducing calls with few rows
// (decode-shaped M): one workgroup per output tile of BM = 32 * RB rows and
// 32 columns computes every shard's partial of that tile and folds them on
// chip, so no partial ever goes to memory and there is no second launch.
//
//  * Eight waves per workgroup; wave w computes the partials of shards
//    w, w + 8 (p <= 16), each as the same MFMA chain as every other path:
//    v_mfma_f32_32x32x16_bf16 over k = 0, 16, 32, ... from a zero
//    accumulator, so each shard's partial has the same bits as the partial
//    the shard-GEMM kernels store.
//  * The weight tile of a shard (64 k x 32 n per step, row-major [K][N]) is
//    streamed by its wave alone through a private ring of STAGES LDS buffers
//    (buffer_load_dwordx4 ... lds, 4 KiB per step) and read with the gfx950
//    transpose read; no barrier is needed inside the K loop because no other
//    wave touches the ring.  Rows of 32 bf16 (64 bytes) need no swizzle: the
//    four rows a 16-lane group reads with one transpose read sit in four
//    different 16-bank groups, and the two halves of the wave read disjoint
//    bank halves.
//  * The activation rows (A operand: lane l holds row l % 32, eight
//    consecutive k) are loaded straight into registers, 16 bytes per lane and
//    k slice, STAGES - 1 steps ahead; rows past M and k past K read as zero.
//  * After every wave's K loops, the partials go to LDS (the rings are free
//    by then) as P[k][BM][32] fp32 (rounded to bf16 first for 2-byte
//    messages: the message that shard would have sent), and the workgroup
//    sums them element by element in shard order k = 0..p-1 in fp32 -- the
//    additions of the reduction kernel, in its order -- rounds once and
//    stores to the AllReduce or ReduceScatter destination.
#pragma once

#include "tpf_gemm.hpp"

namespace tpf {

constexpr int kStWaves = 8;                               // waves per workgroup
constexpr int kStBN = 32;                                 // output columns per workgroup
constexpr int kStBK = 64;                                 // k per pipeline step
constexpr int kStStageBytes = kStBK * kStBN * 2;          // 4 KiB: one step of one shard's weights
constexpr int kStMaxShardsPerWave = 2;                    // p <= 16

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

template <int RB, int STAGES>
struct StPipe {
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 steps in flight");
  static constexpr int PER = 4 * RB + 4;      // loads per step: 4 slices x RB A rows, 4 weight loads
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t a_off[RB];      // byte offset of this lane's A chunk at k = 0 (kOOB: row past M)
  uint32_t b_off[4];       // byte offset of this lane's weight chunk at k = 0 (kOOB: column past N)
  int K;
  uint32_t ldb_bytes;
  char* ring;              // this wave's STAGES x 4 KiB
  bf16x8_t a[STAGES][4][RB];

  // Issue the loads of step t into ring slot (and A register set) st.
  __device__ __forceinline__ void issue(int st, int t) {
    const int lane = threadIdx.x & 63;
    const int k0 = t * kStBK;
    // A: four 16-wide k slices, RB row blocks each; a_off already holds this
    // lane's row and its eight-element k chunk, the slice adds k0 + 16 s.
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int kb = k0 + s * 16;
      const bool k_ok = kb + 8 * (lane >> 5) < K;       // K is a multiple of 8: whole chunks
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const uint32_t off = (a_off[i] != kOOB && k_ok) ? a_off[i] + (uint32_t)kb * 2u : kOOB;
        a[st][s][i] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
      }
    }
    // weights: 4 loads of 16 rows x 64 bytes into this wave's ring slot; rows
    // past K fall outside the resource and read as zeros
    char* dst = ring + st * kStStageBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t off = b_off[q] != kOOB ? b_off[q] + (uint32_t)k0 * ldb_bytes : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(dst + q * 1024), 16, (int)off, 0, 0, 0);
    }
  }
};

// One step: the MFMAs of step t from ring slot ST (loads of steps up to
// t + STAGES - 1 issued on entry to the step).
template <int RB, int STAGES, int ST>
__device__ __forceinline__ void st_step(f32x16_t (&acc)[RB], StPipe<RB, STAGES>& P, int t, int nk) {
  if (t + STAGES - 1 < nk) P.issue((ST + STAGES - 1) % STAGES, t + STAGES - 1);
  st_wait_steps<StPipe<RB, STAGES>::PER>(min(STAGES - 1, nk - 1 - t));
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, jl = lane & 15;
  const int r = jl >> 2, q = jl & 3;
  const char* slot = P.ring + ST * kStStageBytes;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int k = s * 16 + (g >> 1) * 8 + r;          // this lane's row for the first read; +4 for the second
    const int off = k * (kStBN * 2) + ((g & 1) * 16 + q * 4) * 2;
    const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t*)((lds_void_t*)(slot + off)));
    const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4_t*)((lds_void_t*)(slot + off + 4 * kStBN * 2)));
    const bf16x8_t b = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(P.a[ST][s][i], b, acc[i], 0, 0, 0);
  }
}

template <int RB, int STAGES, int ST>
__device__ __forceinline__ void st_steps(f32x16_t (&acc)[RB], StPipe<RB, STAGES>& P, int t, int nk) {
  if constexpr (ST < STAGES) {
    if (t + ST < nk) {
      st_step<RB, STAGES, ST>(acc, P, t + ST, nk);
      st_steps<RB, STAGES, ST + 1>(acc, P, t, nk);
    }
  }
}

template <int RB, int STAGES, int S>
__device__ __forceinline__ void st_prologue(StPipe<RB, STAGES>& P, int nk) {
  if constexpr (S < STAGES - 1) {
    if (S < nk) P.issue(S, S);
    st_prologue<RB, STAGES, S + 1>(P, nk);
  }
}

// Shard k's partial of the tile (m0, n0): the full K loop into acc.
template <int RB, int STAGES>
__device__ __forceinline__ void st_shard(f32x16_t (&acc)[RB], const StationaryArgs& a, int k, int m0, int n0,
                                         char* ring) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.0f;
  StPipe<RB, STAGES> P;
  P.K = a.K;
  P.ldb_bytes = (uint32_t)a.N * 2u;
  P.ra = make_rsrc(a.A[k], (int64_t)a.M * a.K * 2);
  P.rb = make_rsrc(a.B[k], (int64_t)a.K * a.N * 2);
  P.ring = ring;
#pragma unroll
  for (int i = 0; i < RB; ++i) {
    const int m = m0 + i * 32 + (lane & 31);
    P.a_off[i] = m < a.M ? (uint32_t)(((int64_t)m * a.K + 8 * (lane >> 5)) * 2) : kOOB;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = q * 16 + (lane >> 2);               // k row within the step
    const int col = n0 + 8 * (lane & 3);
    P.b_off[q] = col < a.N ? (uint32_t)(((int64_t)row * a.N + col) * 2) : kOOB;
  }
  const int nk = (a.K + kStBK - 1) / kStBK;
  st_prologue<RB, STAGES, 0>(P, nk);
  for (int t = 0; t < nk; t += STAGES) st_steps<RB, STAGES, 0>(acc, P, t, nk);
}

template <int PB>
__device__ __forceinline__ float st_message(float acc) {
  if constexpr (PB) return __uint_as_float(f32_to_bf16_bits(acc) << 16);
  else return acc;
}

template <int RB, int STAGES, int PB, int OUT>
__device__ __forceinline__ void stationary_tile(const StationaryArgs& a, char* lds, int tile) {
  constexpr int BM = 32 * RB;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tm = tile / a.tiles_n, tn = tile - tm * a.tiles_n;
  const int m0 = tm * BM, n0 = tn * kStBN;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  char* ring = lds + wv * (STAGES * kStStageBytes);
  f32x16_t acc[kStMaxShardsPerWave][RB];
#pragma unroll
  for (int j = 0; j < kStMaxShardsPerWave; ++j)
    if (wv + j * kStWaves < a.p) st_shard<RB, STAGES>(acc[j], a, wv + j * kStWaves, m0, n0, ring);
  __syncthreads();                                  // every ring is idle: the LDS holds the partials now
  float* part = reinterpret_cast<float*>(lds);      // [p][BM][32]
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int j = 0; j < kStMaxShardsPerWave; ++j) {
    const int k = wv + j * kStWaves;
    if (k < a.p) {
      float* pk = part + (int64_t)k * BM * kStBN;
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          pk[row * kStBN + r32] = st_message<PB>(acc[j][i][v]);
        }
    }
  }
  __syncthreads();
  // the fold: four consecutive columns per thread, shards in order
  const int t = threadIdx.x;
  if (t < BM * (kStBN / 4)) {
    const int row = t / (kStBN / 4), c = (t % (kStBN / 4)) * 4;
    if (m0 + row < a.M && n0 + c < a.N) {
      f32x4_t s = *reinterpret_cast<const f32x4_t*>(part + row * kStBN + c);
      for (int k = 1; k < a.p; ++k) s = s + *reinterpret_cast<const f32x4_t*>(part + ((int64_t)k * BM + row) * kStBN + c);
      reduce_store4<OUT>(a.ro, (int64_t)(m0 + row) * a.N + n0 + c, a.N, s);
    }
  }
}

}  // namespace tpf
