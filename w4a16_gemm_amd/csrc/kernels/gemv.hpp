// Decode GEMV, M = 1: y[n] = sum_k x[k] * (q[n][k] - Z[g(k)][n]) * S[g(k)][n].
//
// At batch one every weight is read once for about two flops, so the kernel is
// bound by HBM bandwidth ("AWQ + GPTQ Quantization, in depth", What W4A16 buys and
// why decoding gets faster).  Everything is arranged to keep many bytes of packed
// weights in flight and to touch each weight with as few instructions as possible:
//
//  * Persistent grid, one workgroup per compute unit (or a small multiple).  Rows
//    are dealt out in units of one row per wavefront row-slot, round-robin over the
//    workgroups, so the whole grid sweeps through the weights together; the
//    workgroups of one XCD own neighbouring units and share the L2 lines of their
//    scales and zero points.
//  * A row's K input channels are split into 32-channel chunks (16 bytes of codes).
//    LPR lanes share a row; lane j owns chunks j, j+LPR, ... (CPL of them), so each
//    wave-wide 16-byte load is one contiguous run of the row.
//  * Each wavefront walks its rows with a DEPTH-deep register pipeline: the loads
//    of row t+DEPTH are issued as soon as row t has been consumed.  The first
//    DEPTH rows are requested before anything else happens in the workgroup.
//  * Activations are staged once in LDS (gathered through the stored order under
//    act order) and then held in registers: a lane owns the same chunks in every
//    row.  The scales and zero points of all the workgroup's rows are staged once in
//    LDS as one word per (row, group), transposed so that a lane's reads are
//    conflict-free.
//  * Codes are expanded by masking alone: a pair of nibbles in the mantissa bits of a
//    binary16 pair with a zero exponent field is the exact subnormal pair
//    (q, q') * 2^-24 (nibbles.hpp).  v_dot2_f32_f16 multiplies them with the
//    activations into two fp32 accumulators per chunk, one for the pairs taken from
//    the low nibbles of each byte and one, 16 times larger, for the high nibbles.
//    After the chunk t = acc_a + acc_b / 16 = 2^-24 * sum x q, and the zero point and
//    scale enter once per chunk through two fp32 values staged per (row, group):
//        row += t * (S * 2^24) + (-Z * S) * sum x.
//    9 VALU instructions per 8 weights in the inner loop, all but the dot products
//    plain 32-bit AND/shift.
//  * The LPR partial sums of a row are reduced inside the wavefront with DPP moves
//    only (mirrors within rows of 16 lanes, row broadcasts across them); the row
//    result is rounded once to binary16.
#pragma once

#include "nibbles.hpp"

namespace w4a16 {

// DPP move of a float: lanes of rows outside row_mask receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of L lanes (L a power of two <= 64), with VALU-only DPP
// moves (no LDS round trips).  Groups of up to 16 lanes: every lane ends with the
// total.  L = 32 and 64: the total ends in the group's last lane (31/63, 63).
template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f32<0xB1, 0xF>(v);     // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (L >= 4) v += dpp_f32<0x4E, 0xF>(v);     // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (L >= 8) v += dpp_f32<0x141, 0xF>(v);    // row_half_mirror: the other quad of 8
  if constexpr (L >= 16) v += dpp_f32<0x140, 0xF>(v);   // row_mirror: the other half of 16
  if constexpr (L >= 32) v += dpp_f32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  if constexpr (L >= 64) v += dpp_f32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

// Workgroup -> position in the sweep, so that the workgroups of one XCD (dispatch
// is round-robin over the 8 XCDs) own neighbouring row units.
__device__ __forceinline__ int xcd_block(int bid, int nblk) {
  if (nblk % 8 != 0) return bid;
  return (bid % 8) * (nblk / 8) + bid / 8;
}

// Row schedule.  Rows are grouped into units of STRIDE = WAVES * RPW consecutive rows
// (one row per wavefront row-slot); unit u is processed by workgroup u % nblk at step
// u / nblk.  At any moment the whole grid streams one contiguous window of the
// weights, and within a unit the wavefronts read neighbouring rows.
template <int LPR, int CPL, int WAVES, int DEPTH, bool EXACT, bool ACT>
__global__ __launch_bounds__(WAVES * 64) void gemv_m1_kernel(
    const half_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, half_t* __restrict__ y, int N, int K, int gshift, int steps) {
  static_assert(64 % LPR == 0, "lanes per row must divide the wavefront");
  constexpr int RPW = 64 / LPR;          // rows per wavefront per step
  constexpr int STRIDE = WAVES * RPW;    // rows per unit
  static_assert(STRIDE % 8 == 0, "a unit must cover whole 8-row groups of zero points");
  constexpr int NT = WAVES * 64;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rr = lane / LPR;
  const int j = lane % LPR;
  const int C = K >> 5;                  // 32-channel chunks per row
  const int W = K >> 3;                  // words per row
  const int G = K >> gshift;
  const int GP = G + 1;                  // padded slab row (words)
  const int nblk = gridDim.x;
  const int blk = xcd_block(blockIdx.x, nblk);
  const int my_row = wave * RPW + rr;    // row inside a unit
  auto row_of = [&](int t) { return (blk + t * nblk) * STRIDE + my_row; };

  half_t* xs = reinterpret_cast<half_t*>(smem);
  float2* sz = reinterpret_cast<float2*>(smem + static_cast<size_t>(K) * sizeof(half_t));

  // 1. the first DEPTH rows of this wavefront: request the weights now.  Loads are
  // unconditional (row clamped into the matrix, chunk clamped into the row) so that
  // no load sits in a divergent branch and the wait counts stay exact.
  uint4 wb[DEPTH][CPL];
  auto load_row = [&](uint4 (&dst)[CPL], int n) {
    const int nc = min(n, N - 1);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = EXACT ? j + LPR * i : min(j + LPR * i, C - 1);
      dst[i] = *reinterpret_cast<const uint4*>(qw + static_cast<size_t>(nc) * W + 4 * c);
    }
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_row(wb[d], row_of(d));  // clamped if steps < DEPTH

  // 2. activations -> LDS (stored order), and the workgroup's scales and zero points
  // -> a slab with (S * 2^24, -Z * S) in fp32 per (row slot, group), loaded 8 rows
  // (16 bytes of scales, one word of zeros) at a time.
  if constexpr (!ACT) {
    const uint4* src = reinterpret_cast<const uint4*>(x);
    uint4* dst = reinterpret_cast<uint4*>(xs);
    for (int i = tid; i < (K >> 3); i += NT) dst[i] = src[i];
  } else {
    const int32_t* perm = reinterpret_cast<const int32_t*>(qw + static_cast<size_t>(N) * W);
    for (int p = tid; p < K; p += NT) xs[p] = x[perm[p]];
  }
  {
    constexpr int OCT = STRIDE / 8;      // 8-row groups per unit
    const int items = steps * OCT * G;
    for (int it = tid; it < items; it += NT) {
      const int gi = it % G;
      const int so = it / G;             // (step, octet)
      const int t = so / OCT;
      const int o = so - t * OCT;
      const int n8 = (blk + t * nblk) * STRIDE + 8 * o;
      float2* dst = sz + (t * STRIDE + 8 * o) * GP + gi;
      if (n8 < N) {
        const uint4 sv = *reinterpret_cast<const uint4*>(scales + static_cast<size_t>(gi) * N + n8);
        const uint32_t zw = qzeros[static_cast<size_t>(gi) * (N >> 3) + (n8 >> 3)];
        const uint32_t s8[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float S = static_cast<float>(
              __builtin_bit_cast(half_t, static_cast<uint16_t>((s8[r >> 1] >> (16 * (r & 1))) & 0xFFFFu)));
          const float Z = static_cast<float>((zw >> (4 * r)) & 0xFu);
          dst[r * GP] = make_float2(S * 16777216.0f, -Z * S);   // both exact in fp32
        }
      }
    }
  }
  __syncthreads();

  // 3. this lane's activations, as pairs, and the per-chunk sums (dot2 with ones)
  half2_t xr[CPL][16];
  float xsum[CPL];
  int gcol[CPL];
  const half2_t ones = half2_t{static_cast<half_t>(1.0f), static_cast<half_t>(1.0f)};
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = j + LPR * i;
    gcol[i] = (c << 5) >> gshift;
    float sx = 0.f;
    if (EXACT || c < C) {
      const uint4* src = reinterpret_cast<const uint4*>(xs + 32 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = src[q];
        xr[i][4 * q + 0] = as_h2(v.x);
        xr[i][4 * q + 1] = as_h2(v.y);
        xr[i][4 * q + 2] = as_h2(v.z);
        xr[i][4 * q + 3] = as_h2(v.w);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) sx = __builtin_amdgcn_fdot2(xr[i][q], ones, sx, false);
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) xr[i][q] = half2_t{0, 0};
    }
    xsum[i] = sx;
  }

  // 4. rows.  Row t sits in register slot t % DEPTH; its loads were issued DEPTH
  // steps earlier.  The steady-state loop refills every slot unconditionally; the
  // last DEPTH steps run without refills, so no load is issued past the end (a wave
  // cannot retire before its loads return).
  auto row_step = [&](int t, uint4 (&w)[CPL]) {
    const int n = row_of(t);
    const float2* szr = sz + (t * STRIDE + my_row) * GP;
    // The CPL chunks are interleaved word by word: 2*CPL independent dot2
    // accumulation chains (each still summed in the same order).
    float aa[CPL], ab[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      aa[i] = 0.f;
      ab[i] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t word = q == 0 ? w[i].x : q == 1 ? w[i].y : q == 2 ? w[i].z : w[i].w;
        const SubPairs p = expand_word_subnormal(word);
        aa[i] = __builtin_amdgcn_fdot2(as_h2(p.a0), xr[i][4 * q + 0], aa[i], false);
        ab[i] = __builtin_amdgcn_fdot2(as_h2(p.b0), xr[i][4 * q + 1], ab[i], false);
        aa[i] = __builtin_amdgcn_fdot2(as_h2(p.a1), xr[i][4 * q + 2], aa[i], false);
        ab[i] = __builtin_amdgcn_fdot2(as_h2(p.b1), xr[i][4 * q + 3], ab[i], false);
      }
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = j + LPR * i;
      if (EXACT || c < C) {
        const float2 sc = szr[gcol[i]];
        const float tq = fmaf(ab[i], 0.0625f, aa[i]);  // 2^-24 * sum x q
        acc = fmaf(tq, sc.x, acc);                     // + S * sum x q
        acc = fmaf(sc.y, xsum[i], acc);                // - Z * S * sum x
      }
    }
    return acc;
  };
  auto finish = [&](int t, float acc) {
    const int n = row_of(t);
    acc = lane_group_sum<LPR>(acc);
    if (n < N && j == LPR - 1) y[n] = static_cast<half_t>(acc);
  };

  int t0 = 0;
  for (; t0 + 2 * DEPTH <= steps; t0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const float acc = row_step(t0 + d, wb[d]);
      load_row(wb[d], row_of(t0 + d + DEPTH));       // refill this slot
      finish(t0 + d, acc);
    }
  }
  // between DEPTH and 2*DEPTH - 1 steps remain (or fewer than DEPTH in total)
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (t0 + d < steps) {
      const float acc = row_step(t0 + d, wb[d]);
      if (t0 + d + DEPTH < steps) load_row(wb[d], row_of(t0 + d + DEPTH));
      finish(t0 + d, acc);
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d)
    if (t0 + DEPTH + d < steps) finish(t0 + DEPTH + d, row_step(t0 + DEPTH + d, wb[d]));
}

}  // namespace w4a16
