// Small kernels around the two main ones: the weight view used for parity checks
// and the activation gather of act order.
#pragma once

#include "nibbles.hpp"

namespace w4a16 {

// w_out[n][k] = binary16((q - Z) * S) in the original input-channel order, built
// with the same dequant_word the GEMM uses for its weight operand.  One thread per
// packed word.
template <bool ACT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ qw,
                                                     const half_t* __restrict__ scales,
                                                     Zeros qzeros,
                                                     half_t* __restrict__ w_out, int N, int K,
                                                     int gshift) {
  const int W = K >> 3;
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<size_t>(N) * W) return;
  const int n = static_cast<int>(idx / W);
  const int wd = static_cast<int>(idx % W);
  const int p0 = wd * 8;
  const int gi = p0 >> gshift;
  const DequantConsts dc = make_consts(load_zero(qzeros, gi, N, n), scales[static_cast<size_t>(gi) * N + n]);
  const half8_t d = dequant_word(qw[idx], dc);
  half_t* row = w_out + static_cast<size_t>(n) * K;
  if constexpr (!ACT) {
    *reinterpret_cast<half8_t*>(row + p0) = d;
  } else {
    const int32_t* perm = reinterpret_cast<const int32_t*>(qw + static_cast<size_t>(N) * W);
#pragma unroll
    for (int e = 0; e < 8; ++e) row[perm[p0 + e]] = d[e];
  }
}

// 8-bit weights: w_out[n][k] = binary16((q - Z) * S) with dequant_word8, one thread per
// packed word (four channels).
template <bool ACT>
__global__ __launch_bounds__(256) void dequant8_kernel(const uint32_t* __restrict__ qw,
                                                      const half_t* __restrict__ scales, Zeros qzeros,
                                                      half_t* __restrict__ w_out, int N, int K, int gshift) {
  const int W = K >> 2;
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<size_t>(N) * W) return;
  const int n = static_cast<int>(idx / W);
  const int wd = static_cast<int>(idx % W);
  const int p0 = wd * 4;
  const int gi = p0 >> gshift;
  const DequantConsts dc = make_consts(load_zero<8>(qzeros, gi, N, n), scales[static_cast<size_t>(gi) * N + n]);
  const half4_t d = dequant_word8(qw[idx], dc);
  half_t* row = w_out + static_cast<size_t>(n) * K;
  if constexpr (!ACT) {
    *reinterpret_cast<half4_t*>(row + p0) = d;
  } else {
    const int32_t* perm = reinterpret_cast<const int32_t*>(qw + static_cast<size_t>(N) * W);
#pragma unroll
    for (int e = 0; e < 4; ++e) row[perm[p0 + e]] = d[e];
  }
}

// Act order, M > 1: xs[m][p] = x[m][perm[p]], so that the GEMM sees every group as
// a contiguous run of input channels.  A thread takes 8 consecutive stored positions
// (the order read once as two 16-byte loads) and writes them as one 16-byte store in
// every row of its grid-y slice.  Needs K % 8 == 0 and 16-byte aligned perm, x rows
// and xs rows (K % 32 == 0 and aligned buffers give all three).  One row per grid-y
// index up to 1024 rows: with 64 slices (each thread walking M / 64 rows) the
// act-order layer at M = 512, K = 4096 launched only 128 workgroups and took 6.1 us;
// with one row per slice 75.2 -> 73.5 us for the whole layer (same-process A/B,
// identical outputs), the skinny batches unchanged.
constexpr int kGatherRowsY = 1024;   // grid y: row slices

__global__ __launch_bounds__(256) void gather_x_kernel(const half_t* __restrict__ x,
                                                       const int32_t* __restrict__ perm,
                                                       half_t* __restrict__ xs, int M, int K) {
  const int p0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  if (p0 >= K) return;
  const int4 a = *reinterpret_cast<const int4*>(perm + p0);
  const int4 b = *reinterpret_cast<const int4*>(perm + p0 + 4);
  for (int m = blockIdx.y; m < M; m += gridDim.y) {
    const half_t* xr = x + static_cast<size_t>(m) * K;
    const half8_t v = {xr[a.x], xr[a.y], xr[a.z], xr[a.w], xr[b.x], xr[b.y], xr[b.z], xr[b.w]};
    *reinterpret_cast<half8_t*>(xs + static_cast<size_t>(m) * K + p0) = v;
  }
}

// Split-K skinny batches: y[i] = binary16(sum over the ks slices of part[s][i]), the
// slices added in order, one rounding.
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, half_t* __restrict__ y,
                                                         int ks, size_t count) {
  const size_t idx = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= count) return;
  float v = part[idx];
  for (int s = 1; s < ks; ++s) v += part[s * count + idx];
  y[idx] = static_cast<half_t>(v);
}

// Sum of squared differences of two binary16 arrays, one fp32 partial per workgroup
// (grid-stride, then a fixed-order tree in LDS); the host adds the partials in order.
__global__ __launch_bounds__(256) void sq_diff_kernel(const half_t* __restrict__ a, const half_t* __restrict__ b,
                                                      size_t count, float* __restrict__ partial) {
  __shared__ float red[256];
  float acc = 0.f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < count;
       i += static_cast<size_t>(gridDim.x) * 256) {
    const float d = static_cast<float>(a[i]) - static_cast<float>(b[i]);
    acc = fmaf(d, d, acc);
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

}  // namespace w4a16
