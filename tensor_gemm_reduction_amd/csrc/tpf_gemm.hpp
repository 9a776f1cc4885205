// bf16 matrix-core GEMM tile for gfx950.
//
// A workgroup of NW wave64s (arranged WAVES_M x WAVES_N) computes a BM x BN
// block of C = A B in fp32, with A row-major [M][K] (or [K][M], "KM": an
// activation used transposed, as in dW = X^T dY) and B either row-major
// [K][N] ("KN": a forward weight W_k) or row-major [N][K] ("NK": a weight
// used transposed, as in dX = dY W^T).
//
// Data path:
//  * global -> LDS without registers: buffer_load_dwordx4 ... lds.  One such
//    instruction moves 64 lanes x 16 bytes into 1 KiB of contiguous LDS, lane
//    l landing at byte 16*l.  Loads are addressed through buffer resources
//    whose size is the whole operand, so rows past the end of an operand and
//    K (or N) tails read as zeros.
//  * K advances in steps of BK (32 or 64) through STAGES LDS buffers: the loads of step
//    kt+STAGES-1 are issued right after the barrier of step kt, so they
//    overlap STAGES-1 steps of MFMAs.  One barrier per step.  With two
//    stages and K a multiple of BK, each wave's loads are issued between the
//    MFMAs of the slice that follows the barrier rather than in one burst.
//  * A tiles are stored [m][BK k]; each lane of
//    v_mfma_f32_32x32x16_bf16 reads its eight consecutive k with one
//    ds_read_b128.  16-byte chunks are XOR-swizzled by row so that the 16
//    lanes of one LDS pass (same k, consecutive rows) hit all 64 banks once.
//  * KN B tiles stay row-major [BK k][BN n] as they come from memory.  The
//    gfx950 transpose read ds_read_b64_tr_b16 hands lane i of each 16-lane
//    group element i of the four 16-element rows supplied by lanes 4r..4r+3,
//    so lanes 4r+q pointing at B[k0+r][n0+4q] deliver to lane i the four
//    values B[k0..k0+3][n0+i]: two such reads give the eight consecutive k of
//    one column that the MFMA B operand needs.  32-byte blocks are
//    XOR-swizzled by k so that the four rows of a read land in distinct banks.
//  * NK B tiles are stored like A.  KM A tiles are stored and read like KN B
//    tiles (the A and B operands of the MFMA have the same lane layout).
//
// Every output element is accumulated by the same sequence of MFMAs in
// increasing k whatever the tile shape, origin or number of valid rows, so the
// result does not depend on how the rows are chunked or which tile
// configuration computed it.
#pragma once

#include "tpf_device.hpp"

namespace tpf {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset that is always out of range (operands < 2 GiB)

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int BK_ = 64, int SWB_ = 2, int STAGES_A_ = 0,
          int STAGES_B_ = 0>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_;
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  static constexpr int KCH = BK / 8;              // 16-byte chunks per A row
  static constexpr int RB = BK * 2;               // bytes per A row
  static constexpr int ROWS_PER_PERIOD = 256 / RB;  // A rows per 256-byte span of the 64 LDS banks
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NW = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * NW;
  static constexpr int STAGES = STAGES_;
  // A tiles may have one more LDS slot than B tiles (STAGES_A = STAGES + 1):
  // then each step's A loads go out during the MFMAs before the barrier, one
  // step earlier, and only the B loads follow the barrier.
  static constexpr int STAGES_A = STAGES_A_ ? STAGES_A_ : STAGES_;
  static constexpr int STAGES_B = STAGES_B_ ? STAGES_B_ : STAGES_;   // or B has the extra slot
  static_assert(STAGES_A == STAGES || STAGES_A == STAGES + 1, "A slots: STAGES or STAGES + 1");
  static_assert(STAGES_B == STAGES || STAGES_B == STAGES + 1, "B slots: STAGES or STAGES + 1");
  static_assert(STAGES_A == STAGES || STAGES_B == STAGES, "one operand with an extra slot");
  static constexpr int SWB = SWB_;    // KN-B 32-byte block swizzle: block ^ (SWB * (k & 3))
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static_assert(TM >= 1 && TN >= 1 && WM % 32 == 0 && WN % 32 == 0, "wave tile of 32x32 MFMA blocks");
  static constexpr int LDS_A = BM * BK * 2;
  static constexpr int LDS_B = BN * BK * 2;
  static constexpr int LDS_BYTES = STAGES_A * LDS_A + STAGES_B * LDS_B;
  static constexpr int A_INSTR = LDS_A / 1024;   // 1 KiB load instructions per A tile
  static constexpr int B_INSTR = LDS_B / 1024;
  static_assert(A_INSTR % NW == 0 && B_INSTR % NW == 0, "loads must split evenly over waves");
  static constexpr int A_PER_WAVE = A_INSTR / NW;
  static constexpr int B_PER_WAVE = B_INSTR / NW;
  static constexpr int LOADS_PER_WAVE = A_PER_WAVE + B_PER_WAVE;
  static_assert(BN >= 128 && 1024 % (BN * 2 > 1024 ? 1024 : BN * 2) == 0 && (BN * 2) % 256 == 0,
                "KN rows hold >= 8 swizzled 32-byte blocks and tile 1 KiB");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert((STAGES - 2) * LOADS_PER_WAVE <= 63, "vmcnt range");
  // A stored [K][M] (transposed A) uses the KN-style layout: rows of BM
  // elements that tile 1 KiB.
  static constexpr bool KM_OK = BM >= 128 && (BM * 2) % 256 == 0 && 1024 % (BM * 2 > 1024 ? 1024 : BM * 2) == 0;
};

// The LDS slots of one K step: its A tile and its B tile.
struct Stage {
  char* a;
  char* b;
};

// Operand description of one tile job.
struct TileJob {
  const __bf16* A;   // operand base (row 0)
  const __bf16* B;
  int64_t lda, ldb;  // elements
  int a_rows;        // rows of the A operand (its size bound)
  int b_rows;        // rows of the B operand (K for KN, N for NK)
  int m0;            // first row of the tile (absolute)
  int rows;          // valid rows from m0 (<= BM)
  int n0;            // first column
  int N, K;          // output width and reduction length
};

template <class Cfg>
struct Frag {
  f32x16_t acc[Cfg::TM][Cfg::TN];
};

// A buffer resource lives in scalar registers.  Its base and size are the
// same for every lane of the workgroup; readfirstlane states that, so the
// compiler never falls back to per-lane "waterfall" loops around the loads
// when it cannot prove the uniformity itself (e.g. when the operand was
// chosen from a ticket read back from LDS).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* ub = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000);
}

// A (and NK-B) rows: 16 consecutive rows read the same logical chunk in one
// pass of 16 lanes x 16 bytes = 256 bytes = all 64 banks.  Rows in the same
// 256-byte span already use different banks; rows ROWS_PER_PERIOD apart would
// collide, so the chunk is XORed with (row / ROWS_PER_PERIOD) mod KCH.
template <class Cfg>
__device__ __forceinline__ int swz_row(int row) { return (row / Cfg::ROWS_PER_PERIOD) & (Cfg::KCH - 1); }

// Workgroup barrier for the K loop that orders LDS only: this wave's LDS
// reads have returned (the slot they read may be refilled once every wave
// has passed), and the compiler keeps memory accesses on their side of it.
// __syncthreads() would also wait for every outstanding global load
// (vmcnt(0)), including loads issued for later steps; the loads a step needs
// are waited for explicitly instead (wait_vmcnt).
#ifndef TPF_LDS_BARRIER
#define TPF_LDS_BARRIER 1
#endif
__device__ __forceinline__ void lds_barrier() {
#if TPF_LDS_BARRIER
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#else
  __syncthreads();
#endif
}

// s_waitcnt vmcnt(n) for a small compile-time bound on outstanding loads.
__device__ __forceinline__ void wait_vmcnt(int n) {
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] in [15:14]
#define TPF_VM(N) __builtin_amdgcn_s_waitcnt((((N) & 15) | 0x70 | 0xF00 | (((N) >> 4) << 14)))
  switch (n) {
    case 0: TPF_VM(0); break;
    case 1: TPF_VM(1); break;
    case 2: TPF_VM(2); break;
    case 3: TPF_VM(3); break;
    case 4: TPF_VM(4); break;
    case 5: TPF_VM(5); break;
    case 6: TPF_VM(6); break;
    case 7: TPF_VM(7); break;
    case 8: TPF_VM(8); break;
    case 10: TPF_VM(10); break;
    case 12: TPF_VM(12); break;
    case 14: TPF_VM(14); break;
    case 16: TPF_VM(16); break;
    case 20: TPF_VM(20); break;
    case 24: TPF_VM(24); break;
    case 28: TPF_VM(28); break;
    case 32: TPF_VM(32); break;
    case 40: TPF_VM(40); break;
    case 48: TPF_VM(48); break;
    default: TPF_VM(0); break;
  }
#undef TPF_VM
}

template <class Cfg, int BL>
struct TileLoader {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t a_off[Cfg::A_PER_WAVE];   // byte offsets at k0 = 0 (kOOB when out of range)
  uint32_t b_off[Cfg::B_PER_WAVE];
  int K;
  uint32_t ldb_bytes;
  uint32_t lda_bytes;

  __device__ __forceinline__ void init(const TileJob& j) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    K = j.K;
    ldb_bytes = (uint32_t)(j.ldb * 2);
    lda_bytes = (uint32_t)(j.lda * 2);
    ra = make_rsrc(j.A, (int64_t)j.a_rows * j.lda * 2);
    rb = make_rsrc(j.B, (int64_t)j.b_rows * j.ldb * 2);
    if constexpr (a_trans(BL)) {
      // A stored [K][M]: the tile is 64 rows of k, each BM elements of m.
      static_assert(Cfg::KM_OK, "transposed A needs BM-wide rows tiling 1 KiB");
      constexpr int ROW_BYTES = Cfg::BM * 2;
#pragma unroll
      for (int i = 0; i < Cfg::A_PER_WAVE; ++i) {
        const int byte = (wave * Cfg::A_PER_WAVE + i) * 1024 + lane * 16;
        const int k = byte / ROW_BYTES;
        const int pchunk = (byte % ROW_BYTES) / 16;
        const int cblk = (pchunk >> 1) ^ (Cfg::SWB * (k & 3));
        const int c = cblk * 2 + (pchunk & 1);           // logical 16-byte chunk: m = 8c
        const int gm = j.m0 + c * 8;
        a_off[i] = c * 8 < j.rows ? (uint32_t)(((int64_t)k * j.lda + gm) * 2) : kOOB;
      }
    } else {
#pragma unroll
      for (int i = 0; i < Cfg::A_PER_WAVE; ++i) {
        const int row = (wave * Cfg::A_PER_WAVE + i) * (1024 / Cfg::RB) + lane / Cfg::KCH;
        const int kc = (lane % Cfg::KCH) ^ swz_row<Cfg>(row);
        const int gm = j.m0 + row;
        a_off[i] = gm < j.a_rows ? (uint32_t)(((int64_t)gm * j.lda + kc * 8) * 2) : kOOB;
      }
    }
    if constexpr (b_layout(BL) == B_NK) {
#pragma unroll
      for (int i = 0; i < Cfg::B_PER_WAVE; ++i) {
        const int row = (wave * Cfg::B_PER_WAVE + i) * (1024 / Cfg::RB) + lane / Cfg::KCH;
        const int kc = (lane % Cfg::KCH) ^ swz_row<Cfg>(row);
        const int gn = j.n0 + row;
        b_off[i] = gn < j.b_rows ? (uint32_t)(((int64_t)gn * j.ldb + kc * 8) * 2) : kOOB;
      }
    } else {
      constexpr int ROW_BYTES = Cfg::BN * 2;
#pragma unroll
      for (int i = 0; i < Cfg::B_PER_WAVE; ++i) {
        const int byte = (wave * Cfg::B_PER_WAVE + i) * 1024 + lane * 16;
        const int k = byte / ROW_BYTES;                  // row of the 64 x BN tile
        const int pchunk = (byte % ROW_BYTES) / 16;
        const int cblk = (pchunk >> 1) ^ (Cfg::SWB * (k & 3));
        const int c = cblk * 2 + (pchunk & 1);           // logical 16-byte chunk: n = 8c
        const int gn = j.n0 + c * 8;
        b_off[i] = gn < j.N ? (uint32_t)(((int64_t)k * j.ldb + gn) * 2) : kOOB;
      }
    }
  }


  // Logical k chunk (A, NK B) of this lane's i-th A or B load, or (KN B) its
  // k row within the step.  Only the K tail step needs them, so they are
  // recomputed there instead of being kept in registers.
  __device__ __forceinline__ static int a_kpos(int wave, int lane, int i) {
    if constexpr (a_trans(BL)) {
      return ((wave * Cfg::A_PER_WAVE + i) * 1024 + lane * 16) / (Cfg::BM * 2);
    } else {
      const int row = (wave * Cfg::A_PER_WAVE + i) * (1024 / Cfg::RB) + lane / Cfg::KCH;
      return ((lane % Cfg::KCH) ^ swz_row<Cfg>(row)) * 8;
    }
  }
  __device__ __forceinline__ static int b_kpos(int wave, int lane, int i) {
    if constexpr (b_layout(BL) == B_NK) {
      const int row = (wave * Cfg::B_PER_WAVE + i) * (1024 / Cfg::RB) + lane / Cfg::KCH;
      return ((lane % Cfg::KCH) ^ swz_row<Cfg>(row)) * 8;
    } else {
      return ((wave * Cfg::B_PER_WAVE + i) * 1024 + lane * 16) / (Cfg::BN * 2);
    }
  }

  __device__ __forceinline__ void issue(Stage st, int k0) const {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    char* la = st.a;
    char* lb = st.b;
    const bool tail = k0 + Cfg::BK > K;   // the same for the whole workgroup
    if (b_layout(BL) == B_KN && !tail) {
      // Every load of a whole K step is in range along k: the step's offset
      // goes into the scalar offset, the per-lane offsets stay as they were
      // computed for k0 = 0 (kOOB for rows or columns outside the operand,
      // which stays out of range with any scalar offset below 2^31), and the
      // LDS destinations are scalar: no vector arithmetic per load (measured
      // 5-6 % faster on the forward shapes; the weight-transposed (NK)
      // layout measured 4 % slower this way and keeps the path below).
      const int wv = __builtin_amdgcn_readfirstlane(wave);
      const int ka = __builtin_amdgcn_readfirstlane(k0 * (int)(a_trans(BL) ? lda_bytes : 2u));
      const int kb = __builtin_amdgcn_readfirstlane(k0 * (int)(b_layout(BL) == B_NK ? 2u : ldb_bytes));
#pragma unroll
      for (int i = 0; i < Cfg::A_PER_WAVE; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(la + (wv * Cfg::A_PER_WAVE + i) * 1024), 16,
                                                 (int)a_off[i], ka, 0, 0);
#pragma unroll
      for (int i = 0; i < Cfg::B_PER_WAVE; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(lb + (wv * Cfg::B_PER_WAVE + i) * 1024), 16,
                                                 (int)b_off[i], kb, 0, 0);
      return;
    }
    // In the tail step the lane index is passed through an empty asm
    // statement, which the compiler cannot move: the tail-only index
    // arithmetic then stays inside the branch instead of being hoisted out of
    // the K loop into registers that every step would keep live.
    int tl = lane;
    if (tail) asm volatile("" : "+v"(tl));
#pragma unroll
    for (int i = 0; i < Cfg::A_PER_WAVE; ++i) {
      // MK: k runs along the row; KM: the tile's row k is operand row k0 + k
      uint32_t off = a_off[i] != kOOB ? a_off[i] + (uint32_t)k0 * (a_trans(BL) ? lda_bytes : 2u) : kOOB;
      if (tail && k0 + a_kpos(wave, tl, i) >= K) off = kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(la + (wave * Cfg::A_PER_WAVE + i) * 1024), 16,
                                               off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < Cfg::B_PER_WAVE; ++i) {
      // NK: k runs along the row; KN: the tile's row k is operand row k0 + k
      uint32_t off = b_off[i] != kOOB ? b_off[i] + (uint32_t)k0 * (b_layout(BL) == B_NK ? 2u : ldb_bytes) : kOOB;
      if (tail && k0 + b_kpos(wave, tl, i) >= K) off = kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(lb + (wave * Cfg::B_PER_WAVE + i) * 1024), 16,
                                               off, 0, 0, 0);
    }
  }
};

// MFMA operand fragments of one 16-wide k step.
template <class Cfg>
struct Operands {
  bf16x8_t a[Cfg::TM];
  bf16x8_t b[Cfg::TN];
};

template <class Cfg, int BL>
__device__ __forceinline__ void read_a(Operands<Cfg>& o, const char* la, int s, int wm, int wn, int lane) {
  const int r32 = lane & 31, half = lane >> 5;
  const int kc = s * 2 + half;
  if constexpr (a_trans(BL)) {
    // [64 k][BM m] tile, read with transposes exactly like a KN B tile
    constexpr int ROW_BYTES = Cfg::BM * 2;
    const int g = lane >> 4, jl = lane & 15;
    const int r = jl >> 2, q = jl & 3;
    const int k = s * 16 + (g >> 1) * 8 + r;
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = wm * Cfg::WM + i * 32 + (g & 1) * 16 + q * 4;
      const int c = m >> 3;
      const int pblk = (c >> 1) ^ (Cfg::SWB * (k & 3));
      const int off = (pblk * 2 + (c & 1)) * 16 + (q & 1) * 8;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(
          (lds_void_t*)(la + k * ROW_BYTES + off)));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(
          (lds_void_t*)(la + (k + 4) * ROW_BYTES + off)));
      o.a[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  } else {
#pragma unroll
    for (int i = 0; i < Cfg::TM; ++i) {
      const int m = wm * Cfg::WM + i * 32 + r32;
      o.a[i] = *reinterpret_cast<const bf16x8_t*>(la + m * Cfg::RB + ((kc ^ swz_row<Cfg>(m)) * 16));
    }
  }
}

template <class Cfg, int BL>
__device__ __forceinline__ void read_b(Operands<Cfg>& o, const char* lb, int s, int wm, int wn, int lane) {
  const int r32 = lane & 31, half = lane >> 5;
  const int kc = s * 2 + half;
  (void)wm;
  if constexpr (b_layout(BL) == B_NK) {
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn) {
      const int n = wn * Cfg::WN + jn * 32 + r32;
      o.b[jn] = *reinterpret_cast<const bf16x8_t*>(lb + n * Cfg::RB + ((kc ^ swz_row<Cfg>(n)) * 16));
    }
  } else {
    constexpr int ROW_BYTES = Cfg::BN * 2;
    const int g = lane >> 4, jl = lane & 15;
    const int r = jl >> 2, q = jl & 3;
    const int k = s * 16 + (g >> 1) * 8 + r;          // this lane's row for the first read; +4 for the second
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn) {
      const int n = wn * Cfg::WN + jn * 32 + (g & 1) * 16 + q * 4;
      const int c = n >> 3;
      const int pblk = (c >> 1) ^ (Cfg::SWB * (k & 3));   // (k + 4) & 3 == k & 3
      const int off = (pblk * 2 + (c & 1)) * 16 + (q & 1) * 8;
      const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(
          (lds_void_t*)(lb + k * ROW_BYTES + off)));
      const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(
          (lds_void_t*)(lb + (k + 4) * ROW_BYTES + off)));
      o.b[jn] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// The fragments of one 16-wide k slice.
template <class Cfg, int BL>
__device__ __forceinline__ void read_operands(Operands<Cfg>& o, Stage st, int s, int wm, int wn, int lane) {
  read_a<Cfg, BL>(o, st.a, s, wm, wn, lane);
  read_b<Cfg, BL>(o, st.b, s, wm, wn, lane);
}

template <class Cfg>
__device__ __forceinline__ void mfma_step(Frag<Cfg>& f, const Operands<Cfg>& o) {
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn)
      f.acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[i], o.b[jn], f.acc[i][jn], 0, 0, 0);
}

// Each LDS slot (the A tile or the B tile of one stage) is its own __shared__
// object.  The loads of a later step are LDS writes in flight (buffer_load
// ... lds) while the current slots are read; with one object per slot, and
// every access naming its slot at compile time, the compiler can see that
// they do not overlap and does not wait for the in-flight loads before
// reading the current slots.
template <class Cfg, int S>
__device__ __forceinline__ char* a_slot() {
  __shared__ __attribute__((aligned(1024))) char buf[Cfg::LDS_A];
  return buf;
}
template <class Cfg, int S>
__device__ __forceinline__ char* b_slot() {
  __shared__ __attribute__((aligned(1024))) char buf[Cfg::LDS_B];
  return buf;
}
// A slot SA and B slot SB.
template <class Cfg, int SA, int SB = SA>
__device__ __forceinline__ Stage stage() {
  return Stage{a_slot<Cfg, SA>(), b_slot<Cfg, SB>()};
}
// LDS that is idle once gemm_tile has returned (A slot S): LDS_A bytes each.
template <class Cfg, int S>
__device__ __forceinline__ char* stage_ptr() {
  static_assert(S < Cfg::STAGES_A, "an A slot");
  return a_slot<Cfg, S>();
}

// Loads of K step `step` into stage S.  Every wave issues exactly
// LOADS_PER_WAVE vector-memory instructions per call, so vmcnt arithmetic
// stays per-step.
template <class Cfg, int BL, int S>
__device__ __forceinline__ void issue_stage(const TileLoader<Cfg, BL>& ld, int step) {
  ld.issue(stage<Cfg, S>(), step * Cfg::BK);
}

template <class Cfg, int BL, int S>
__device__ __forceinline__ void prefetch(const TileLoader<Cfg, BL>& ld, int nk) {
  if constexpr (S < Cfg::STAGES - 1) {
    if (S < nk) issue_stage<Cfg, BL, S>(ld, S);
    prefetch<Cfg, BL, S + 1>(ld, nk);
  }
}

// Steps 0 .. STAGES-2 into their stages, past the end repeating the last
// step (the interleaved path, K a multiple of BK).
template <class Cfg, int BL, int S>
__device__ __forceinline__ void prefetch_all(const TileLoader<Cfg, BL>& ld, int nk) {
  if constexpr (S < Cfg::STAGES - 1) {
    ld.issue(stage<Cfg, S>(), (S < nk ? S : nk - 1) * Cfg::BK);
    prefetch_all<Cfg, BL, S + 1>(ld, nk);
  }
}

// Wait until this wave's loads of step `t` have landed, given that every
// step up to min(t + STAGES - 2, nk - 1) has been issued.
template <class Cfg>
__device__ __forceinline__ void wait_step(int t, int nk) {
  wait_vmcnt(min(Cfg::STAGES - 2, nk - 1 - t) * Cfg::LOADS_PER_WAVE);
}

// Loads interleaved with the MFMAs: large two-stage tiles, when K is a
// multiple of BK.  (The decode-sized tiles measured 2 % slower with it: one
// MFMA per slice leaves nothing to interleave with.)
#ifndef TPF_ILOAD
#define TPF_ILOAD 1
#endif

template <class Cfg, int BL>
__device__ __forceinline__ constexpr bool iload_ok() {
  return TPF_ILOAD && Cfg::BM >= 128;
}

// Loads of one K step on the interleaved path are numbered q = 0 .. NL-1.

// Scalar offsets of step kn (clamped to the last step) and its load q into
// stage S.
template <class Cfg, int BL>
struct IlOffsets {
  int wv, ka, kb;
  __device__ __forceinline__ IlOffsets(const TileLoader<Cfg, BL>& ld, int kn, int nk) {
    wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int k0 = (kn < nk ? kn : nk - 1) * Cfg::BK;
    ka = __builtin_amdgcn_readfirstlane(k0 * (int)(a_trans(BL) ? ld.lda_bytes : 2u));
    kb = __builtin_amdgcn_readfirstlane(k0 * (int)(b_layout(BL) == B_NK ? 2u : ld.ldb_bytes));
  }
  __device__ __forceinline__ void load(const TileLoader<Cfg, BL>& ld, Stage st, int q) const {
    char* la = st.a;
    char* lb = st.b;
    const bool isa = q < Cfg::A_PER_WAVE;   // A tile's loads first, then B's
    const int i = isa ? q : q - Cfg::A_PER_WAVE;
    if (isa)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld.ra, (lds_void_t*)(la + (wv * Cfg::A_PER_WAVE + i) * 1024), 16,
                                               (int)ld.a_off[i], ka, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ld.rb, (lds_void_t*)(lb + (wv * Cfg::B_PER_WAVE + i) * 1024), 16,
                                               (int)ld.b_off[i], kb, 0, 0);
  }
};

// Loads Q0 .. Q1-1 of step kn into stage S, without MFMAs (prologue).
template <class Cfg, int BL, int SA, int SB, int Q0, int Q1>
__device__ __forceinline__ void il_loads(const TileLoader<Cfg, BL>& ld, int kn, int nk) {
  const IlOffsets<Cfg, BL> x(ld, kn, nk);
#pragma unroll
  for (int q = Q0; q < Q1; ++q) x.load(ld, stage<Cfg, SA, SB>(), q);
}

// One k slice's MFMAs with loads Q0 .. Q1-1 of step kn into stage S issued
// between them.  After a K-step barrier all waves of the workgroup would
// otherwise issue their loads at once; the address unit's queue then fills,
// and a wave stalled on a load cannot issue its MFMAs either (in-order
// issue), so the matrix core idles.  Interleaved, the queue drains while the
// MFMAs run (measured 6-10 % faster on the large shapes).  Only for K a
// multiple of BK (no tail step): the step's offset goes into the scalar
// offset, as in TileLoader::issue.  Past the last step (kn >= nk) the last
// step is loaded again into the free stage, which nothing reads afterwards.
template <class Cfg, int BL, int SA, int SB, int Q0, int Q1>
__device__ __forceinline__ void mfma_step_loads(Frag<Cfg>& f, const Operands<Cfg>& o, const TileLoader<Cfg, BL>& ld,
                                                int kn, int nk) {
  constexpr int NLP = Q1 - Q0;
  constexpr int NM = Cfg::TM * Cfg::TN;
  const IlOffsets<Cfg, BL> x(ld, kn, nk);
#pragma unroll
  for (int q = 0; q < (NM > NLP ? NM : NLP); ++q) {
    if (q < NM) {
      const int i = q / Cfg::TN, jn = q % Cfg::TN;
      f.acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o.a[i], o.b[jn], f.acc[i][jn], 0, 0, 0);
    }
    if (q < NLP) x.load(ld, stage<Cfg, SA, SB>(), Q0 + q);
  }
}

// One K step on stage S, software-pipelined across steps.  On entry the
// fragments of this step's first 16-wide k slice are in o[0].  Each slice's
// MFMAs run while the next slice's fragments are read.  Before the last
// slice's MFMAs, the workgroup waits for the next step's data and passes the
// barrier (every wave has finished reading stage S by then), refills stage S
// with the loads of step kt + STAGES, and starts reading the next step's
// first slice; the last slice's MFMAs then cover that latency.
template <class Cfg, int BL, int S>
__device__ __forceinline__ void kstep(Frag<Cfg>& f, const TileLoader<Cfg, BL>& ld, Operands<Cfg> (&o)[2], int kt,
                                      int nk, int wm, int wn, int lane) {
  constexpr int SUB = Cfg::BK / 16;
  static_assert(SUB % 2 == 0, "even number of k slices per step");
  const Stage cur = stage<Cfg, S>();
#pragma unroll
  for (int s = 0; s < SUB - 1; ++s) {
    read_operands<Cfg, BL>(o[(s + 1) & 1], cur, s + 1, wm, wn, lane);
    mfma_step<Cfg>(f, o[s & 1]);
  }
  if (kt + 1 < nk) {
    wait_step<Cfg>(kt + 1, nk);
    lds_barrier();
    if (kt + Cfg::STAGES < nk) issue_stage<Cfg, BL, S>(ld, kt + Cfg::STAGES);
    read_operands<Cfg, BL>(o[0], stage<Cfg, (S + 1) % Cfg::STAGES>(), 0, wm, wn, lane);
  }
  mfma_step<Cfg>(f, o[1]);
}

// The same K step without branches, for K a multiple of BK: the barrier is
// passed at every step (the last one too), and the loads of step kt + STAGES
// -- past the end, the last step again, into the stage every wave has
// finished reading -- are issued one after each MFMA of the last k slice.
template <class Cfg, int BL, int S>
__device__ __forceinline__ void kstep_il(Frag<Cfg>& f, const TileLoader<Cfg, BL>& ld, Operands<Cfg> (&o)[2], int kt,
                                         int nk, int wm, int wn, int lane) {
  constexpr int SUB = Cfg::BK / 16;
  static_assert(SUB % 2 == 0, "even number of k slices per step");
  constexpr int NL = Cfg::A_PER_WAVE + Cfg::B_PER_WAVE;
  const Stage cur = stage<Cfg, S>();
#pragma unroll
  for (int s = 0; s < SUB - 1; ++s) {
    read_operands<Cfg, BL>(o[(s + 1) & 1], cur, s + 1, wm, wn, lane);
    mfma_step<Cfg>(f, o[s & 1]);
  }
  // Every step issues exactly LOADS_PER_WAVE loads, so the loads of the
  // STAGES - 2 steps after step kt + 1 may stay in flight.
  wait_vmcnt((Cfg::STAGES - 2) * Cfg::LOADS_PER_WAVE);
  lds_barrier();
  read_operands<Cfg, BL>(o[0], stage<Cfg, (S + 1) % Cfg::STAGES>(), 0, wm, wn, lane);
  mfma_step_loads<Cfg, BL, S, S, 0, NL>(f, o[1], ld, kt + Cfg::STAGES, nk);
}

// K step T (mod lcm of the slot counts) with one more LDS slot for one
// operand (the "early" one; A by default): the early operand's loads of step
// kt + 2 go out between the MFMAs of slices 0 .. SUB-2 (their slot held step
// kt - 1, free since the previous barrier), the other operand's loads of step
// kt + 2 between those of the last slice, after the barrier.  The address
// unit then has the whole step for the early loads, and they have almost two
// steps to land.
template <class Cfg, int BL, int T>
__device__ __forceinline__ void kstep_ila(Frag<Cfg>& f, const TileLoader<Cfg, BL>& ld, Operands<Cfg> (&o)[2], int kt,
                                          int nk, int wm, int wn, int lane) {
  constexpr int SUB = Cfg::BK / 16;
  static_assert(SUB % 2 == 0, "even number of k slices per step");
  static_assert(Cfg::STAGES == 2 && Cfg::STAGES_A + Cfg::STAGES_B == 5,
                "two slots for one operand, three for the other");
  constexpr bool EB = Cfg::STAGES_B > Cfg::STAGES;     // B is the early operand
  constexpr int SA = T % Cfg::STAGES_A, SB = T % Cfg::STAGES_B;
  constexpr int SAN = (SA + 2) % Cfg::STAGES_A;        // slots of step kt + 2
  constexpr int SBN = (SB + 2) % Cfg::STAGES_B;
  constexpr int NA = Cfg::A_PER_WAVE, NB = Cfg::B_PER_WAVE;
  constexpr int QE0 = EB ? NA : 0, NE = EB ? NB : NA;  // early loads [QE0, QE0 + NE)
  constexpr int QL0 = EB ? 0 : NA, NLT = EB ? NA : NB; // late loads
  const Stage cur = stage<Cfg, SA, SB>();
#pragma unroll
  for (int s = 0; s < SUB - 1; ++s) {
    read_operands<Cfg, BL>(o[(s + 1) & 1], cur, s + 1, wm, wn, lane);
    // early loads [0, Q1_0) in slice 0, [Q1_0, Q1_1) in slice 1, the rest in
    // slice 2 (front-loaded: the earliest have the longest to land)
    constexpr int Q1_0 = QE0 + (NE + SUB - 2) / (SUB - 1);
    constexpr int Q1_1 = QE0 + (2 * NE + SUB - 2) / (SUB - 1);
    if (s == 0)
      mfma_step_loads<Cfg, BL, SAN, SBN, QE0, Q1_0>(f, o[0], ld, kt + 2, nk);
    else if (s == 1)
      mfma_step_loads<Cfg, BL, SAN, SBN, Q1_0, Q1_1>(f, o[1], ld, kt + 2, nk);
    else if (s == 2)
      mfma_step_loads<Cfg, BL, SAN, SBN, Q1_1, QE0 + NE>(f, o[0], ld, kt + 2, nk);
    else
      mfma_step<Cfg>(f, o[s & 1]);
  }
  // The early loads of step kt + 2 were issued after step kt + 1's.
  wait_vmcnt(NE);
  lds_barrier();
  read_operands<Cfg, BL>(o[0], stage<Cfg, (SA + 1) % Cfg::STAGES_A, (SB + 1) % Cfg::STAGES_B>(), 0, wm, wn, lane);
  mfma_step_loads<Cfg, BL, SAN, SBN, QL0, QL0 + NLT>(f, o[1], ld, kt + 2, nk);
}

template <class Cfg, int BL, int T>
__device__ __forceinline__ void ksteps_ila(Frag<Cfg>& f, const TileLoader<Cfg, BL>& ld, Operands<Cfg> (&o)[2], int kt,
                                           int nk, int wm, int wn, int lane) {
  if constexpr (T < 6) {
    if (kt + T < nk) {
      kstep_ila<Cfg, BL, T>(f, ld, o, kt + T, nk, wm, wn, lane);
      ksteps_ila<Cfg, BL, T + 1>(f, ld, o, kt, nk, wm, wn, lane);
    }
  }
}

template <class Cfg, int BL, int S, bool IL>
__device__ __forceinline__ void ksteps(Frag<Cfg>& f, const TileLoader<Cfg, BL>& ld, Operands<Cfg> (&o)[2], int kt,
                                       int nk, int wm, int wn, int lane) {
  if constexpr (S < Cfg::STAGES) {
    if (kt + S < nk) {
      if constexpr (IL) kstep_il<Cfg, BL, S>(f, ld, o, kt + S, nk, wm, wn, lane);
      else kstep<Cfg, BL, S>(f, ld, o, kt + S, nk, wm, wn, lane);
      ksteps<Cfg, BL, S + 1, IL>(f, ld, o, kt, nk, wm, wn, lane);
    }
  }
}

// Full K loop of one tile into registers.  Ends with a barrier, so the
// caller may reuse the stages (e.g. stage 0's first word) immediately.
template <class Cfg, int BL>
__device__ __forceinline__ void gemm_tile(Frag<Cfg>& f, const TileJob& j) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn)
#pragma unroll
      for (int v = 0; v < 16; ++v) f.acc[i][jn][v] = 0.0f;

  TileLoader<Cfg, BL> ld;
  ld.init(j);
  const int nk = (j.K + Cfg::BK - 1) / Cfg::BK;
  // Steps 0 .. STAGES-2 are loaded up front; step STAGES-1 is issued into
  // the last stage right away (nothing has used it yet).  On the
  // interleaved path every stage is loaded (steps past the end repeat the
  // last step), so that each step has exactly LOADS_PER_WAVE loads behind it.
  const bool il = iload_ok<Cfg, BL>() && j.K % Cfg::BK == 0;   // uniform
  if constexpr (Cfg::STAGES_A > Cfg::STAGES || Cfg::STAGES_B > Cfg::STAGES) {
    if (il) {
      // Steps 0 and 1 into fresh slots, A then B each (the order the steps
      // after them keep); wait for step 0.
      ld.issue(stage<Cfg, 0, 0>(), 0);
      ld.issue(stage<Cfg, 1, 1>(), (1 < nk ? 1 : nk - 1) * Cfg::BK);
      wait_vmcnt(Cfg::LOADS_PER_WAVE);
      __syncthreads();
      Operands<Cfg> o[2];
      read_operands<Cfg, BL>(o[0], stage<Cfg, 0, 0>(), 0, wm, wn, lane);
      for (int kt = 0; kt < nk; kt += 6) ksteps_ila<Cfg, BL, 0>(f, ld, o, kt, nk, wm, wn, lane);
      wait_vmcnt(0);   // the repeated loads past the last step
      __syncthreads();
      return;
    }
  }
  if (il) {
    prefetch_all<Cfg, BL, 0>(ld, nk);
    wait_vmcnt((Cfg::STAGES - 2) * Cfg::LOADS_PER_WAVE);
    __syncthreads();
    il_loads<Cfg, BL, Cfg::STAGES - 1, Cfg::STAGES - 1, 0, Cfg::A_PER_WAVE + Cfg::B_PER_WAVE>(ld, Cfg::STAGES - 1,
                                                                                         nk);
  } else {
    prefetch<Cfg, BL, 0>(ld, nk);
    wait_step<Cfg>(0, nk);
    __syncthreads();
    if (Cfg::STAGES - 1 < nk) issue_stage<Cfg, BL, Cfg::STAGES - 1>(ld, Cfg::STAGES - 1);
  }
  Operands<Cfg> o[2];
  read_operands<Cfg, BL>(o[0], stage<Cfg, 0>(), 0, wm, wn, lane);
  if (il) {
    for (int kt = 0; kt < nk; kt += Cfg::STAGES) ksteps<Cfg, BL, 0, iload_ok<Cfg, BL>()>(f, ld, o, kt, nk, wm, wn, lane);
    wait_vmcnt(0);   // the repeated loads past the last step
  } else {
    for (int kt = 0; kt < nk; kt += Cfg::STAGES) ksteps<Cfg, BL, 0, false>(f, ld, o, kt, nk, wm, wn, lane);
  }
  __syncthreads();
}

// Write the accumulators of one tile.  Element (row, col) of the 32x32 MFMA
// block held in register v of lane l: col = l % 32,
// row = 8 * (v / 4) + 4 * (l / 32) + v % 4.
// GeLU(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) in fp32 (the erf form;
// erff is the device math library's).
__device__ __forceinline__ float gelu_f32(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

template <class Cfg, int OUT, int ACT = 0>
__device__ __forceinline__ void store_tile(const Frag<Cfg>& f, const TileJob& j, void* out, int64_t ldo) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / Cfg::WAVES_N, wn = wave % Cfg::WAVES_N;
  const int r32 = lane & 31, half = lane >> 5;
  constexpr int ES = OUT == OUT_F32 ? 4 : 2;
  // Buffer stores addressed from the tile's first element through a resource
  // that covers only the tile's valid rows; one store per element.  Whole
  // tiles keep one per-lane offset per 32x32 block and put the block-row
  // offsets (8 (v / 4) + v % 4) * ldo in scalar registers.  Edge tiles put
  // the whole offset in the per-lane register (the range check always covers
  // it) and give elements outside the output (row past the valid rows,
  // column past N) an offset beyond any resource, so the hardware drops
  // their stores.  Both cases are straight-line code: the accumulators are
  // only ever indexed by compile-time constants.  Every offset is below
  // 2^31: each output is < 2 GiB.
  // (Uniform values, stated with readfirstlane: a scalar offset the compiler
  // could not prove uniform would cost a per-lane loop around every store.)
  const bool whole = __builtin_amdgcn_readfirstlane(j.rows == Cfg::BM && j.n0 + Cfg::BN <= j.N);
  const int64_t tile0 = (int64_t)j.m0 * ldo + j.n0;
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<char*>(out) + tile0 * ES, (int64_t)j.rows * ldo * ES);
  const int lds = __builtin_amdgcn_readfirstlane((int)ldo * ES);
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
#pragma unroll
    for (int jn = 0; jn < Cfg::TN; ++jn) {
      const int cl = wn * Cfg::WN + jn * 32 + r32;
      const bool col_ok = j.n0 + cl < j.N;
      const int rb = wm * Cfg::WM + i * 32 + 4 * half;
      const int vbase = rb * lds + cl * ES;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ro = 8 * (v >> 2) + (v & 3);
        const int voff = whole ? vbase : (col_ok && rb + ro < j.rows ? vbase + ro * lds : (int)kOOB);
        const int soff = __builtin_amdgcn_readfirstlane(whole ? ro * lds : 0);
        const float x = ACT ? gelu_f32(f.acc[i][jn][v]) : f.acc[i][jn][v];
        if constexpr (OUT == OUT_F32)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, voff, soff, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_bits(x), rs, voff, soff, 0);
      }
    }
  }
}

}  // namespace tpf
