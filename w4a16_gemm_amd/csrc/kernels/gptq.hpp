// GPTQ on the device ("AWQ + GPTQ Quantization, in depth", The two algorithms,
// compactly, the GPTQ half): the Hessian H = 2 X X^T of the calibration rows with
// damping, the upper Cholesky factor U of H^-1, and the column-by-column rounding
// with error feedback, all in binary64.
//
// U without forming H^-1: factor H = Ut^T Ut from the bottom-right corner (Ut^T
// upper), then U = (Ut^T)^-1, which is upper with a positive diagonal and satisfies
// U^T U = H^-1, so it is the upper Cholesky factor of H^-1.  Both steps are one
// launch per pivot (a rank-1 update of the rows above it); the matrices stay in HBM.
//
// The rounding runs in blocks of 32 visited columns, four to a batch of 128: a thread
// per output row rounds a block's columns in order with their error fed forward inside
// the block; a rank-32 update carries the block's errors to the batch's later columns,
// and after the batch one rank-128 update carries the batch's errors to every column
// after it (so the weights beyond the batch are read and written once per batch, not
// once per block).  Group starts are block starts (every group size is a multiple of 32,
// and 32, 64 and 128 divide the batch), so a group's grid is taken from columns that
// have received every earlier error, as in the column-by-column order.  The group grid and the rounding are the round-to-nearest quantiser's
// (binary64, round half to even, binary16 scale rounded up).
#pragma once

#include "quantize.hpp"

namespace w4a16 {

constexpr int kGptqBlock = 32;
constexpr int kGptqBatch = 128;

#pragma clang fp contract(off)

// dst[r][i] = binary64(src[r][perm[i]]): rows in the visiting order of the columns.
__global__ __launch_bounds__(256) void gptq_gather_kernel(const uint16_t* __restrict__ src,
                                                          const int32_t* __restrict__ perm, size_t rows, int K,
                                                          double* __restrict__ dst) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= rows * static_cast<size_t>(K)) return;
  const size_t r = i / K;
  const int c = static_cast<int>(i % K);
  dst[i] = half_bits_to_double(src[r * K + perm[c]]);
}

// Lower triangle (j <= i) of H = 2 Xp^T Xp, Xp [T][K]: 64 x 64 tiles, 4 x 4 per thread.
__global__ __launch_bounds__(256) void gptq_gram_kernel(const double* __restrict__ xp, int T, int K,
                                                        double* __restrict__ H) {
  constexpr int TILE = 64, CHUNK = 16;
  const int bi = blockIdx.y, bj = blockIdx.x;
  if (bj > bi) return;
  __shared__ double a[CHUNK][TILE], b[CHUNK][TILE];
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  double acc[4][4];
  for (int r = 0; r < 4; ++r)
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
  for (int t0 = 0; t0 < T; t0 += CHUNK) {
    for (int e = tid; e < CHUNK * TILE; e += 256) {
      const int tt = e / TILE, cc = e % TILE, t = t0 + tt;
      const int ci = bi * TILE + cc, cj = bj * TILE + cc;
      a[tt][cc] = (t < T && ci < K) ? xp[static_cast<size_t>(t) * K + ci] : 0.0;
      b[tt][cc] = (t < T && cj < K) ? xp[static_cast<size_t>(t) * K + cj] : 0.0;
    }
    __syncthreads();
    for (int tt = 0; tt < CHUNK; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(a[tt][tr + 16 * r], b[tt][tc + 16 * c], acc[r][c]);
    __syncthreads();
  }
  for (int r = 0; r < 4; ++r)
    for (int c = 0; c < 4; ++c) {
      const int i = bi * TILE + tr + 16 * r, j = bj * TILE + tc + 16 * c;
      if (i < K && j <= i) H[static_cast<size_t>(i) * K + j] = 2.0 * acc[r][c];
    }
}

// H[i][i] += damp * mean(diag H) (one workgroup).
__global__ __launch_bounds__(256) void gptq_damp_kernel(double* __restrict__ H, int K, double damp) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < K; i += 256) s += H[static_cast<size_t>(i) * K + i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  const double add = damp * (part[0] / K);
  for (int i = threadIdx.x; i < K; i += 256) H[static_cast<size_t>(i) * K + i] += add;
}

// Factorisation from the bottom-right corner, pivot p (grid: p workgroups, one per
// row r < p): H[r][c] -= (H[p][r] / H[p][p]) H[p][c] for c <= r.  Only the lower
// triangle is kept; H[p][r] stands for H[r][p].  A pivot that is not positive is
// caught by the finishing kernel (the updates then carry non-finite values, within
// the same bounds).
__global__ __launch_bounds__(256) void gptq_chol_step_kernel(double* __restrict__ H, int K, int p) {
  const int r = blockIdx.x;
  const double* prow = H + static_cast<size_t>(p) * K;
  const double f = prow[r] / prow[p];
  double* row = H + static_cast<size_t>(r) * K;
  for (int c = threadIdx.x; c <= r; c += 256) row[c] = row[c] - f * prow[c];
}

// Row p of the factor: Ut[p][r] = H[p][r] / sqrt(H[p][p]), r <= p, in place (grid: K).
// flag <- 1 if a pivot is not a positive finite number.
__global__ __launch_bounds__(256) void gptq_chol_finish_kernel(double* __restrict__ H, int K,
                                                               int* __restrict__ flag) {
  const int p = blockIdx.x;
  double* row = H + static_cast<size_t>(p) * K;
  const double d = row[p];
  __syncthreads();   // every thread has read the pivot before it is overwritten
  if (!(d > 0.0) || !isfinite(d)) {
    if (threadIdx.x == 0) *flag = 1;
    return;
  }
  const double s = sqrt(d);
  for (int r = threadIdx.x; r <= p; r += 256) row[r] = row[r] / s;
}

// X = identity [K][K].
__global__ __launch_bounds__(256) void gptq_eye_kernel(double* __restrict__ X, int K) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<size_t>(K) * K) return;
  X[i] = (i / K == i % K) ? 1.0 : 0.0;
}

// Inverse of the upper factor V = Ut^T by row elimination from the bottom, pivot p
// (grid: p workgroups, one per row r < p): X[r][c] -= (Ut[p][r] / Ut[p][p]) X[p][c],
// c >= p.  Row p of X is only read here and rows r < p only written.
__global__ __launch_bounds__(256) void gptq_trinv_step_kernel(const double* __restrict__ Ut,
                                                              double* __restrict__ X, int K, int p) {
  const int r = blockIdx.x;
  const double* urow = Ut + static_cast<size_t>(p) * K;
  const double f = urow[r] / urow[p];
  double* row = X + static_cast<size_t>(r) * K;
  const double* prow = X + static_cast<size_t>(p) * K;
  for (int c = p + static_cast<int>(threadIdx.x); c < K; c += 256) row[c] = row[c] - f * prow[c];
}

// U[p][c] = X[p][c] / Ut[p][p], c >= p (grid: K).
__global__ __launch_bounds__(256) void gptq_trinv_finish_kernel(const double* __restrict__ Ut,
                                                                double* __restrict__ X, int K) {
  const int p = blockIdx.x;
  const double d = Ut[static_cast<size_t>(p) * K + p];
  double* row = X + static_cast<size_t>(p) * K;
  for (int c = p + static_cast<int>(threadIdx.x); c < K; c += 256) row[c] = row[c] / d;
}

// Visited columns [i0, i0 + 32) of every row (thread per row): the group grid at a
// group start (from the row's current values of the group's columns), else the one
// kept in sz; then each column rounded in order, its error e = (w - q^) / U[j][j]
// fed to the block's later columns and kept in err[n * err_stride + c] for the updates.
__global__ __launch_bounds__(128) void gptq_block_kernel(const double* __restrict__ wp,
                                                         const double* __restrict__ U, int N, int K, int i0,
                                                         int group_size, double2* __restrict__ sz,
                                                         double* __restrict__ err, int err_stride,
                                                         uint8_t* __restrict__ codes_p,
                                                         uint16_t* __restrict__ scales,
                                                         uint8_t* __restrict__ zeros) {
  constexpr int B = kGptqBlock;
  __shared__ double u[B][B + 1];
  for (int e = threadIdx.x; e < B * B; e += 128) u[e / B][e % B] = U[static_cast<size_t>(i0 + e / B) * K + i0 + e % B];
  __syncthreads();
  const int n = blockIdx.x * 128 + threadIdx.x;
  if (n >= N) return;
  const double* row = wp + static_cast<size_t>(n) * K;
  double w[B];
#pragma unroll
  for (int c = 0; c < B; ++c) w[c] = row[i0 + c];
  double S, Z;
  if (i0 % group_size == 0) {
    double lo = 0.0, hi = 0.0;
    for (int k = i0; k < i0 + group_size; ++k) {
      lo = fmin(lo, row[k]);
      hi = fmax(hi, row[k]);
    }
    const bool flat = hi == lo;
    const uint16_t sbits = flat ? 0x3C00 : half_ceil_bits((hi - lo) / 15.0);
    S = half_bits_to_double(sbits);
    Z = flat ? 0.0 : fmin(fmax(rint(-lo / S), 0.0), 15.0);
    const size_t gi = static_cast<size_t>(i0 / group_size) * N + n;
    scales[gi] = sbits;
    zeros[gi] = static_cast<uint8_t>(Z);
    sz[n] = make_double2(S, Z);
  } else {
    const double2 v = sz[n];
    S = v.x;
    Z = v.y;
  }
  uint8_t* crow = codes_p + static_cast<size_t>(n) * K + i0;
  double* erow = err + static_cast<size_t>(n) * err_stride;
#pragma unroll
  for (int c = 0; c < B; ++c) {
    const double q = fmin(fmax(rint(w[c] / S) + Z, 0.0), 15.0);
    const double e = (w[c] - (q - Z) * S) / u[c][c];
#pragma unroll
    for (int c2 = c + 1; c2 < B; ++c2) w[c2] = w[c2] - e * u[c][c2];
    crow[c] = static_cast<uint8_t>(q);
    erow[c] = e;
  }
}

#pragma clang fp contract(on)

// wp[n][k] -= sum_c err[n * err_stride + c] U[i0 + c][k], c < rank (a multiple of 32), for
// the columns k_begin <= k < k_end (64 x 64 tiles, grid: column tiles x row tiles).  The
// rank is taken in chunks of 32 through LDS into the same accumulators, which are
// subtracted from the weights once.
__global__ __launch_bounds__(256) void gptq_update_kernel(double* __restrict__ wp, const double* __restrict__ U,
                                                          const double* __restrict__ err, int err_stride, int N,
                                                          int K, int i0, int rank, int k_begin, int k_end) {
  constexpr int B = kGptqBlock, TILE = 64;
  __shared__ double es[TILE][B + 1];
  __shared__ double us[B][TILE];
  const int k0 = k_begin + blockIdx.x * TILE;
  const int n0 = blockIdx.y * TILE;
  const int tid = threadIdx.x;
  const int tr = tid / 16, tc = tid % 16;
  double acc[4][4];
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int c0 = 0; c0 < rank; c0 += B) {
    for (int e = tid; e < TILE * B; e += 256) {
      const int r = e / B, c = e % B;
      es[r][c] = n0 + r < N ? err[static_cast<size_t>(n0 + r) * err_stride + c0 + c] : 0.0;
    }
    for (int e = tid; e < B * TILE; e += 256) {
      const int c = e / TILE, j = e % TILE;
      us[c][j] = k0 + j < k_end ? U[static_cast<size_t>(i0 + c0 + c) * K + k0 + j] : 0.0;
    }
    __syncthreads();
    for (int c = 0; c < B; ++c)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(es[tr + 16 * a][c], us[c][tc + 16 * b], acc[a][b]);
    __syncthreads();
  }
  for (int a = 0; a < 4; ++a)
    for (int b = 0; b < 4; ++b) {
      const int n = n0 + tr + 16 * a, k = k0 + tc + 16 * b;
      if (n < N && k < k_end) wp[static_cast<size_t>(n) * K + k] -= acc[a][b];
    }
}

// codes[n][perm[i]] = codes_p[n][i]: back to the original channel order.
__global__ __launch_bounds__(256) void gptq_scatter_codes_kernel(const uint8_t* __restrict__ codes_p,
                                                                 const int32_t* __restrict__ perm, int N, int K,
                                                                 uint8_t* __restrict__ codes) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<size_t>(N) * K) return;
  const size_t n = i / K;
  codes[n * K + perm[i % K]] = codes_p[i];
}

}  // namespace w4a16
