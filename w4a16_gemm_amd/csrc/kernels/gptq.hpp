// GPTQ on the device ("AWQ + GPTQ Quantization, in depth", The two algorithms,
// compactly, the GPTQ half): the Hessian H = 2 X X^T of the calibration rows with
// damping, the upper Cholesky factor U of H^-1, and the column-by-column rounding
// with error feedback, all in binary64.
//
// U without forming H^-1: factor H = Ut^T Ut from the bottom-right corner (Ut^T
// upper), then U = (Ut^T)^-1, which is upper with a positive diagonal and satisfies
// U^T U = H^-1, so it is the upper Cholesky factor of H^-1.  Both are eliminations from
// the bottom, one pivot after the other (for each pivot p: every row r < p minus a
// multiple of row p), run with the pivots in blocks of 64: the block's own rows in one
// launch, the rows above it in another; the matrices stay in HBM.
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

// U[p][c] = X[p][c] / Ut[p][p], c >= p (grid: K).
__global__ __launch_bounds__(256) void gptq_trinv_finish_kernel(const double* __restrict__ Ut,
                                                                double* __restrict__ X, int K) {
  const int p = blockIdx.x;
  const double d = Ut[static_cast<size_t>(p) * K + p];
  double* row = X + static_cast<size_t>(p) * K;
  for (int c = p + static_cast<int>(threadIdx.x); c < K; c += 256) row[c] = row[c] / d;
}

// Blocked forms of the two eliminations, pivots taken 64 at a time from the bottom
// (block P = [p0, p0 + bs)).  Every element receives the same operations in the same
// order as it would one pivot at a time (for each pivot p of P, descending, one multiply
// and one subtraction with that pivot's multiplier: the factorisation's H[p][r] / H[p][p]
// applied to row p's entries c <= r, the inverse's Ut[p][r] / Ut[p][p] applied to row p's
// entries c >= p), so the results are the same bits; the matrices are read and written
// once per block instead of once per pivot.
constexpr int kGptqPivots = 64;

// Factorisation, the block's own rows: rows P of columns [c0, c0 + 64) (grid: one
// workgroup per 64 columns below p0, plus one for the block's diagonal part).  Each
// workgroup repeats the eliminations inside the diagonal part, which give the
// multipliers; the diagonal part's result goes to dg[i][j] (64 x 64), not into H, whose
// diagonal part the other workgroups of the launch are still reading.
__global__ __launch_bounds__(256) void gptq_chol_panel_kernel(double* __restrict__ H, int K, int p0, int bs,
                                                              double* __restrict__ dg) {
  constexpr int B = kGptqPivots;
  __shared__ double d[B][B];   // d[i][j] = H[p0 + i][p0 + j], j <= i
  __shared__ double t[B][B];   // t[i][c] = H[p0 + i][c0 + c]
  const int tid = threadIdx.x;
  const int npan = (p0 + B - 1) / B;
  const bool diag = static_cast<int>(blockIdx.x) == npan;
  const int c0 = static_cast<int>(blockIdx.x) * B;
  const int nc = diag ? 0 : min(B, p0 - c0);
  for (int e = tid; e < B * B; e += 256) {
    const int i = e / B, j = e % B;
    d[i][j] = (i < bs && j <= i) ? H[static_cast<size_t>(p0 + i) * K + p0 + j] : 0.0;
    t[i][j] = (i < bs && j < nc) ? H[static_cast<size_t>(p0 + i) * K + c0 + j] : 0.0;
  }
  __syncthreads();
  for (int pi = bs - 1; pi >= 1; --pi) {
    const double dp = d[pi][pi];
    // rows ri < pi: the diagonal part (columns cj <= ri) and the panel columns
    for (int e = tid; e < pi * B; e += 256) {
      const int ri = e / B, cj = e % B;
      const double f = d[pi][ri] / dp;
      if (cj <= ri) d[ri][cj] = d[ri][cj] - f * d[pi][cj];
      if (cj < nc) t[ri][cj] = t[ri][cj] - f * t[pi][cj];
    }
    __syncthreads();
  }
  for (int e = tid; e < B * B; e += 256) {
    const int i = e / B, j = e % B;
    if (diag) {
      if (i < bs && j <= i) dg[i * B + j] = d[i][j];
    } else if (i < bs && j < nc) {
      H[static_cast<size_t>(p0 + i) * K + c0 + j] = t[i][j];
    }
  }
}

// Factorisation, the rows above the block: H[r][c] for c <= r < p0 (64 x 64 tiles of the
// lower triangle, grid: tile pairs (tr >= tc) listed row by row, at least one), each
// element updated by the block's pivots in descending order with the multiplier
// H[p][r] / H[p][p] and row p's (final) entry H[p][c]; the pivots H[p][p] come from dg.
// Workgroup 0 also writes the block's diagonal part from dg into H (nothing in this
// launch reads it there).
__global__ __launch_bounds__(256) void gptq_chol_trail_kernel(double* __restrict__ H, int K, int p0, int bs,
                                                              const double* __restrict__ dg) {
  constexpr int B = kGptqPivots;
  if (blockIdx.x == 0)
    for (int e = threadIdx.x; e < B * B; e += 256) {
      const int i = e / B, j = e % B;
      if (i < bs && j <= i) H[static_cast<size_t>(p0 + i) * K + p0 + j] = dg[i * B + j];
    }
  __shared__ double fr[B][B];   // fr[pi][r] = H[p0 + pi][r0 + r] / H[p0 + pi][p0 + pi]
  __shared__ double hc[B][B];   // hc[pi][c] = H[p0 + pi][c0 + c]
  int tr = static_cast<int>((sqrt(8.0 * blockIdx.x + 1.0) - 1.0) / 2.0);
  while ((tr + 1) * (tr + 2) / 2 <= static_cast<int>(blockIdx.x)) ++tr;
  while (tr * (tr + 1) / 2 > static_cast<int>(blockIdx.x)) --tr;
  const int tc = static_cast<int>(blockIdx.x) - tr * (tr + 1) / 2;
  const int r0 = tr * B, c0 = tc * B;
  const int tid = threadIdx.x;
  for (int e = tid; e < B * B; e += 256) {
    const int i = e / B, j = e % B;
    const bool pin = i < bs;
    const double* prow = H + static_cast<size_t>(p0 + (pin ? i : 0)) * K;
    fr[i][j] = (pin && r0 + j < p0) ? prow[r0 + j] / dg[(pin ? i : 0) * (B + 1)] : 0.0;
    hc[i][j] = (pin && c0 + j < p0) ? prow[c0 + j] : 0.0;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = r0 + ty + 16 * a, c = c0 + tx + 16 * b;
      if (r >= p0 || c > r) continue;
      double v = H[static_cast<size_t>(r) * K + c];
      for (int pi = bs - 1; pi >= 0; --pi) v = v - fr[pi][ty + 16 * a] * hc[pi][tx + 16 * b];
      H[static_cast<size_t>(r) * K + c] = v;
    }
}

// Inverse, the block's own rows: X[p0 + i][c] for the columns c of one 64-column tile at
// or after p0 (grid: one workgroup per tile), with the block's multipliers Ut[p][r] /
// Ut[p][p] and only the columns c >= p of each pivot row, as in the one-pivot step.
__global__ __launch_bounds__(256) void gptq_trinv_panel_kernel(const double* __restrict__ Ut, double* __restrict__ X,
                                                               int K, int p0, int bs) {
  constexpr int B = kGptqPivots;
  __shared__ double f[B][B];   // f[pi][ri] = Ut[p0 + pi][p0 + ri] / Ut[p0 + pi][p0 + pi]
  __shared__ double t[B][B];   // t[i][c] = X[p0 + i][c0 + c]
  const int tid = threadIdx.x;
  const int c0 = p0 + static_cast<int>(blockIdx.x) * B;
  const int nc = min(B, K - c0);
  for (int e = tid; e < B * B; e += 256) {
    const int i = e / B, j = e % B;
    f[i][j] = (i < bs && j < i) ? Ut[static_cast<size_t>(p0 + i) * K + p0 + j] / Ut[static_cast<size_t>(p0 + i) * K + p0 + i]
                                : 0.0;
    t[i][j] = (i < bs && j < nc) ? X[static_cast<size_t>(p0 + i) * K + c0 + j] : 0.0;
  }
  __syncthreads();
  for (int pi = bs - 1; pi >= 1; --pi) {
    for (int e = tid; e < pi * B; e += 256) {
      const int ri = e / B, cj = e % B;
      if (cj < nc && c0 + cj >= p0 + pi) t[ri][cj] = t[ri][cj] - f[pi][ri] * t[pi][cj];
    }
    __syncthreads();
  }
  for (int e = tid; e < B * B; e += 256) {
    const int i = e / B, j = e % B;
    if (i < bs && j < nc) X[static_cast<size_t>(p0 + i) * K + c0 + j] = t[i][j];
  }
}

// Inverse, the rows above the block: X[r][c] for r < p0 and c >= p0 (64 x 64 tiles, grid:
// column tiles x row tiles), each element updated by the block's pivots in descending
// order with Ut[p][r] / Ut[p][p] and row p's (final) entry X[p][c], for the pivots p <= c.
__global__ __launch_bounds__(256) void gptq_trinv_trail_kernel(const double* __restrict__ Ut, double* __restrict__ X,
                                                               int K, int p0, int bs) {
  constexpr int B = kGptqPivots;
  __shared__ double fr[B][B];   // fr[pi][r] = Ut[p0 + pi][r0 + r] / Ut[p0 + pi][p0 + pi]
  __shared__ double xc[B][B];   // xc[pi][c] = X[p0 + pi][c0 + c]
  const int c0 = p0 + static_cast<int>(blockIdx.x) * B;
  const int r0 = static_cast<int>(blockIdx.y) * B;
  const int tid = threadIdx.x;
  for (int e = tid; e < B * B; e += 256) {
    const int i = e / B, j = e % B;
    const bool pin = i < bs;
    const double* urow = Ut + static_cast<size_t>(p0 + (pin ? i : 0)) * K;
    fr[i][j] = (pin && r0 + j < p0) ? urow[r0 + j] / urow[p0 + i] : 0.0;
    xc[i][j] = (pin && c0 + j < K) ? X[static_cast<size_t>(p0 + i) * K + c0 + j] : 0.0;
  }
  __syncthreads();
  const int ty = tid / 16, tx = tid % 16;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int r = r0 + ty + 16 * a, c = c0 + tx + 16 * b;
      if (r >= p0 || c >= K) continue;
      double v = X[static_cast<size_t>(r) * K + c];
      for (int pi = bs - 1; pi >= 0; --pi)
        if (c >= p0 + pi) v = v - fr[pi][ty + 16 * a] * xc[pi][tx + 16 * b];
      X[static_cast<size_t>(r) * K + c] = v;
    }
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
