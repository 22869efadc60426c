// MFMA GEMM for M > 1: y[M][N] = x[M][K] * W^[N][K]^T, W^ = binary16((q - Z) * S).
//
// Prefill is a dense contraction ("AWQ + GPTQ Quantization, in depth", What W4A16
// buys: prefill on long prompts is compute-bound), so it runs on the matrix cores
// with v_mfma_f32_16x16x32_f16 and fp32 accumulators.
//
//  * A workgroup of 4 wavefronts computes a BM x 256 tile of y; wavefront w owns
//    columns [64w, 64w + 64) of the tile and all BM rows, so every weight is
//    dequantised exactly once per workgroup.
//  * K advances in tiles of 128.  For each of its four 16-column blocks a lane loads
//    16 bytes of codes (32 consecutive input channels of one output row), expands
//    them in registers with the group's zero point and scale (nibbles.hpp) and uses
//    word s of the 16 bytes as its B operand of the s-th MFMA of the tile.  The A
//    operand of lane l in that MFMA is the 8 activations of the same input channels,
//    so the K order inside the tile is the one the code loads give, and the pairing
//    of activations with weights is exact.
//  * The activation tile (BM x 128 binary16) is staged through LDS, double
//    buffered; 16-byte chunks are XOR-swizzled by row so that the 16 rows one MFMA
//    operand reads hit distinct banks.
//  * Ragged M and N are masked; a ragged K tile reads zero activations.
#pragma once

#include "nibbles.hpp"

namespace w4a16 {

template <int BM>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const half_t* __restrict__ x, const uint32_t* __restrict__ qw, const half_t* __restrict__ scales,
    const uint32_t* __restrict__ qzeros, half_t* __restrict__ y, int M, int N, int K, int gshift) {
  static_assert(BM % 16 == 0 && BM >= 16, "BM must be a multiple of 16");
  constexpr int MB = BM / 16;                     // 16-row blocks per wavefront
  constexpr int ACH = BM * 16;                    // 16-byte activation chunks per K tile
  constexpr int APT = (ACH + 255) / 256;          // chunks per thread
  __shared__ uint4 lds_a[2][ACH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;  // row (A) / column (B) inside a 16-block
  const int lq = lane >> 4;  // which 32-channel quarter of the K tile
  const int m0 = blockIdx.y * BM;
  const int nw = blockIdx.x * 256 + wave * 64;
  const int W = K >> 3;
  const int KT = (K + 127) >> 7;

  uint4 areg[APT];
  auto load_a = [&](int t) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = tid + 256 * i;
      const int row = c >> 4, ch = c & 15;
      const int m = m0 + row, k = t * 128 + ch * 8;
      if (c < ACH && m < M && k < K)
        areg[i] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(m) * K + k);
      else
        areg[i] = uint4{0, 0, 0, 0};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = tid + 256 * i;
      if (c < ACH) {
        const int row = c >> 4, ch = c & 15;
        lds_a[buf][row * 16 + (ch ^ (row & 15))] = areg[i];
      }
    }
  };

  uint4 bw[4];
  half_t bs[4];
  uint32_t bz[4];
  auto load_b = [&](int t) {
    const int k = t * 128 + lq * 32;
    const bool kin = k < K;
    const int gi = kin ? (k >> gshift) : 0;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = min(nw + 16 * nb + lr, N - 1);
      bw[nb] = kin ? *reinterpret_cast<const uint4*>(qw + static_cast<size_t>(n) * W + (k >> 3))
                   : uint4{0, 0, 0, 0};
      bs[nb] = scales[static_cast<size_t>(gi) * N + n];
      bz[nb] = load_zero(qzeros, gi, N, n);
    }
  };

  float4_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  load_a(0);
  store_a(0);
  load_b(0);
  __syncthreads();

  for (int t = 0; t < KT; ++t) {
    uint4 cw[4];
    DequantConsts dc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      cw[nb] = bw[nb];
      dc[nb] = make_consts(bz[nb], bs[nb]);
    }
    if (t + 1 < KT) {
      load_a(t + 1);
      load_b(t + 1);
    }
    const uint4* at = lds_a[t & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t bf[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const uint32_t word = s == 0 ? cw[nb].x : s == 1 ? cw[nb].y : s == 2 ? cw[nb].z : cw[nb].w;
        bf[nb] = dequant_word(word, dc[nb]);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = 16 * mb + lr;
        const half8_t a = __builtin_bit_cast(half8_t, at[row * 16 + ((4 * lq + s) ^ lr)]);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[nb], acc[mb][nb], 0, 0, 0);
      }
    }
    if (t + 1 < KT) store_a((t + 1) & 1);
    __syncthreads();
  }

  // D layout of the 16x16 MFMA: lane l holds rows 4*(l/16) + r, column l % 16.
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = nw + 16 * nb + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * mb + 4 * lq + r;
        if (m < M && n < N) y[static_cast<size_t>(m) * N + n] = static_cast<half_t>(acc[mb][nb][r]);
      }
    }
}

}  // namespace w4a16
