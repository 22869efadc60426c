// Decode GEMV, M = 1: y[n] = sum_k x[k] * (q[n][k] - Z[g(k)][n]) * S[g(k)][n].
//
// At batch one every weight is read once for about two flops, so the kernel is
// bound by HBM bandwidth ("AWQ + GPTQ Quantization, in depth", What W4A16 buys and
// why decoding gets faster).  The design keeps every per-weight step in registers:
//
//  * A row's K input channels are split into 32-channel chunks (16 bytes of codes).
//    LPR lanes share a row; lane j of the row owns chunks j, j+LPR, ... (CPL of
//    them), so each wave-wide 16-byte load is one contiguous run of the row.
//  * The activations are staged once per workgroup in LDS (gathered through the
//    stored order under act order) and then kept in registers: a lane always owns
//    the same chunks, for every row it visits.
//  * Codes are expanded with the 1024-offset trick (nibbles.hpp) and multiplied
//    with v_dot2_f32_f16 into two fp32 accumulators per chunk, one for the
//    (1024 + q) pairs and one for the (1024 + 16 q) pairs.  The accumulators start
//    at -1024 * (sum of the matching activations), so after the chunk
//        t = acc_a + acc_b / 16 = sum x q,
//    and the zero point and scale are applied once per chunk in fp32:
//        row += (t - Z * sum x) * S.
//    That is 9 VALU instructions per 8 weights in the inner loop.
//  * The LPR partial sums of a row are reduced across lanes with butterfly
//    shuffles; the row result is rounded once to binary16.
//  * Workgroups own contiguous row ranges (neighbouring rows share the cache lines
//    of their scales and zero points); each wave walks its rows with the next
//    row's loads issued before the current row is reduced.
#pragma once

#include "nibbles.hpp"

namespace w4a16 {

template <int LPR, int CPL, int WAVES, bool ACT>
__global__ __launch_bounds__(WAVES * 64) void gemv_m1_kernel(
    const half_t* __restrict__ x, const uint32_t* __restrict__ qw, const half_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, half_t* __restrict__ y, int N, int K, int gshift,
    int rows_per_block) {
  static_assert(64 % LPR == 0, "lanes per row must divide the wavefront");
  constexpr int RPW = 64 / LPR;  // rows per wave per pass
  extern __shared__ __align__(16) half_t xs[];

  const int tid = threadIdx.x;
  const int C = K >> 5;  // 32-channel chunks per row
  const int W = K >> 3;  // words per row

  // 1. activations -> LDS (stored order)
  if constexpr (!ACT) {
    const uint4* src = reinterpret_cast<const uint4*>(x);
    uint4* dst = reinterpret_cast<uint4*>(xs);
    for (int i = tid; i < (K >> 3); i += WAVES * 64) dst[i] = src[i];
  } else {
    const int32_t* perm = reinterpret_cast<const int32_t*>(qw + static_cast<size_t>(N) * W);
    for (int p = tid; p < K; p += WAVES * 64) xs[p] = x[perm[p]];
  }
  __syncthreads();

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rr = lane / LPR;
  const int j = lane % LPR;

  // 2. this lane's activations, as pairs, and the per-chunk sums
  half2_t xr[CPL][16];
  float init_a[CPL], init_b[CPL], xsum[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = j + LPR * i;
    float sa = 0.f, sb = 0.f;
    if (c < C) {
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
      for (int q = 0; q < 16; ++q) {
        const float s = static_cast<float>(xr[i][q].x) + static_cast<float>(xr[i][q].y);
        if (q & 1) sb += s; else sa += s;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) xr[i][q] = half2_t{0, 0};
    }
    init_a[i] = -1024.f * sa;
    init_b[i] = -1024.f * sb;
    xsum[i] = sa + sb;
  }

  // 3. rows
  const int row_begin = blockIdx.x * rows_per_block;
  const int row_end = min(N, row_begin + rows_per_block);
  constexpr int STRIDE = WAVES * RPW;

  uint4 wv[CPL];
  half_t sv[CPL];
  uint32_t zv[CPL];
  auto fetch = [&](int n) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = j + LPR * i;
      if (n < row_end && c < C) {
        wv[i] = *reinterpret_cast<const uint4*>(qw + static_cast<size_t>(n) * W + 4 * c);
        const int gi = (c << 5) >> gshift;
        sv[i] = scales[static_cast<size_t>(gi) * N + n];
        zv[i] = load_zero(qzeros, gi, N, n);
      } else {
        wv[i] = uint4{0, 0, 0, 0};
        sv[i] = 0;
        zv[i] = 0;
      }
    }
  };

  int n = row_begin + wave * RPW + rr;
  fetch(n);
  for (int base = row_begin + wave * RPW; base < row_end; base += STRIDE) {
    uint4 cw[CPL];
    half_t cs[CPL];
    uint32_t cz[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      cw[i] = wv[i];
      cs[i] = sv[i];
      cz[i] = zv[i];
    }
    const int cur = n;
    n += STRIDE;
    fetch(n);  // next row's loads in flight while this row is computed

    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      float aa = init_a[i], ab = init_b[i];
      const uint32_t words[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const Pairs p = expand_word(words[q]);
        aa = __builtin_amdgcn_fdot2(as_h2(p.a0), xr[i][4 * q + 0], aa, false);
        ab = __builtin_amdgcn_fdot2(as_h2(p.b0), xr[i][4 * q + 1], ab, false);
        aa = __builtin_amdgcn_fdot2(as_h2(p.a1), xr[i][4 * q + 2], aa, false);
        ab = __builtin_amdgcn_fdot2(as_h2(p.b1), xr[i][4 * q + 3], ab, false);
      }
      float t = fmaf(ab, 0.0625f, aa);                       // sum x q
      t = fmaf(-static_cast<float>(cz[i]), xsum[i], t);     // sum x (q - Z)
      acc = fmaf(t, static_cast<float>(cs[i]), acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (cur < row_end && j == 0) y[cur] = static_cast<half_t>(acc);
  }
}

}  // namespace w4a16
