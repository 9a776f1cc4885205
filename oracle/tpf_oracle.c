/*
 * Plain C oracle for the fused tensor-parallel Linear: the definitions of the
 * operations written out as loops, float64 accumulation, OpenMP over output
 * rows.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header or table
 * with the HIP library and includes nothing from it.
 *
 * Inputs are bfloat16 bit patterns (uint16) exactly as the GPU receives them.
 * A bfloat16 value is the top half of an IEEE binary32, so widening it is a
 * shift; the product of two bfloat16 values has at most 16 significant bits
 * and is exact in double, and the sums carry ~2^-53 relative error, far below
 * every tolerance the tests use.
 *
 * Sources (web pages, cited by title and section):
 *  - ai-infra-kb M027 "compute-communication fusion" page, §01: row-parallel
 *    Linear, Y = Y_0 + Y_1 over the ranks' local outputs; AllReduce leaves Y
 *    on every rank, ReduceScatter a row slice on each; AllGather then MatMul.
 *  - cnblogs tensor-parallel tutorial: §2.4 / §四 row shards
 *    (Y = sum_k X_k A_k, A_k the k-th contiguous block of rows); §2.3 / §三
 *    column shards and the backward dX = sum_k dY_k A_k^T (§6.1, §6.4);
 *    §2.5-2.7 AllReduce sums, AllGather concatenates in rank order,
 *    ReduceScatter hands rank r the r-th block of rows.
 *
 * Loop order follows the definition: for each output row i, for each shard k,
 * for each reduction index t, add X_k[i,t] * W_k[t,:] into the row's
 * accumulator (contiguous inner loop).  The column-parallel dX runs dot
 * products over the shard's output columns instead, since its weights are
 * read transposed.  No blocking, no reordering of the sums beyond that.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact value of a bfloat16 bit pattern. */
static double bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int tpfo_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Row index of output row r of the request (all rows when rows == NULL). */
static int64_t row_of(const int64_t* rows, int64_t r) { return rows ? rows[r] : r; }

/*
 * MatMul -> AllReduce (M027 §01; cnblogs §2.4 / §四, §2.5):
 *   Y[r, j] = sum_{k=0}^{p-1} sum_{t=0}^{K-1} X_k[i, t] W_k[t, j],  i = rows[r].
 * X[k]: [M, K], W[k]: [K, N], Y: [nrows, N] float64.  ReduceScatter slice s
 * is rows [s*M/p, (s+1)*M/p) of the same sum (cnblogs §2.7), taken by the
 * caller.  Shard k is the k-th contiguous block of the reduction dimension
 * (cnblogs §2.4); the caller hands the shards in rank order.
 */
void tpfo_matmul_allreduce(int p, int64_t M, int64_t N, int64_t K, const uint16_t* const* X,
                           const uint16_t* const* W, const int64_t* rows, int64_t nrows, double* Y) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = row_of(rows, r);
    double* acc = Y + r * N;
    for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
    for (int k = 0; k < p; ++k) {
      const uint16_t* x = X[k] + i * K;
      for (int64_t t = 0; t < K; ++t) {
        const double a = bf16(x[t]);
        const uint16_t* w = W[k] + t * N;
        for (int64_t j = 0; j < N; ++j) acc[j] += a * bf16(w[j]);
      }
    }
  }
}

/*
 * Column-parallel backward input gradient (cnblogs §三, §6.1, §6.4):
 *   dX[r, j] = sum_{k=0}^{p-1} sum_{t=0}^{Ns-1} dY_k[i, t] W_k[j, t],  i = rows[r].
 * dY[k]: [M, Ns], W[k]: [K_in, Ns] (the forward column shard, read
 * transposed), dX: [nrows, K_in] float64.
 */
void tpfo_matmul_dx(int p, int64_t M, int64_t K_in, int64_t Ns, const uint16_t* const* dY,
                    const uint16_t* const* W, const int64_t* rows, int64_t nrows, double* dX) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = row_of(rows, r);
    double* out = dX + r * K_in;
    for (int64_t j = 0; j < K_in; ++j) out[j] = 0.0;
    for (int k = 0; k < p; ++k) {
      const uint16_t* g = dY[k] + i * Ns;
      for (int64_t j = 0; j < K_in; ++j) {
        const uint16_t* w = W[k] + j * Ns;
        double s = 0.0;
        for (int64_t t = 0; t < Ns; ++t) s += bf16(g[t]) * bf16(w[t]);
        out[j] += s;
      }
    }
  }
}

/*
 * AllGather -> MatMul (M027 §01-§02; cnblogs §2.3, §2.6):
 *   X_gathered = [slice_0; ...; slice_{p-1}] (rank order), Y = X_gathered W.
 * slices[s]: [M/p, K], W: [K, N]; for each requested row i the gathered row
 * (a copy of row i % (M/p) of slice i / (M/p)) goes to Xg[r, :] (bit patterns)
 * and Y[r, :] = that row times W, float64.
 */
void tpfo_allgather_matmul(int p, int64_t M, int64_t N, int64_t K, const uint16_t* const* slices,
                           const uint16_t* W, const int64_t* rows, int64_t nrows, uint16_t* Xg, double* Y) {
  const int64_t per = M / p;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t i = row_of(rows, r);
    const uint16_t* x = slices[i / per] + (i % per) * K;
    memcpy(Xg + r * K, x, (size_t)K * sizeof(uint16_t));
    double* acc = Y + r * N;
    for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
    for (int64_t t = 0; t < K; ++t) {
      const double a = bf16(x[t]);
      const uint16_t* w = W + t * N;
      for (int64_t j = 0; j < N; ++j) acc[j] += a * bf16(w[j]);
    }
  }
}

/*
 * Round float64 values to bfloat16, to nearest with ties to even, in one step
 * (rounding through binary32 first could round twice).  bfloat16 keeps 8
 * significant bits and binary32's exponent range: a finite x with
 * 2^(e-1) <= |x| < 2^e has quantum 2^(e-8), never finer than the subnormal
 * quantum 2^-133.  Scaling by a power of two is exact, nearbyint rounds to
 * nearest even in the default rounding mode, and scaling back is exact; a
 * result at or beyond 2^128 is infinite.  The rounded value is exact in
 * binary32, whose top half is the bfloat16 pattern.  NaN becomes 0x7FC0.
 */
void tpfo_round_bf16(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    const double v = x[i];
    if (isnan(v)) {
      out[i] = 0x7FC0;
      continue;
    }
    double y = v;
    if (isfinite(v) && v != 0.0) {
      int e;
      (void)frexp(v, &e);
      int q = e - 8;
      if (q < -133) q = -133;
      y = ldexp(nearbyint(ldexp(v, -q)), q);
      if (fabs(y) >= ldexp(1.0, 128)) y = copysign(INFINITY, y);
    }
    const float f = (float)y;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    out[i] = (uint16_t)(u >> 16);
  }
}
