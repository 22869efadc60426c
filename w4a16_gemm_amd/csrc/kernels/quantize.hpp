// Round-to-nearest group quantiser on the device, writing the packed weight buffer,
// the binary16 scales and the packed zero points directly.
//
// It computes exactly what the host quantiser computes ("LLM Quantization: INT8, GPTQ,
// and AWQ Explained", What quantization actually does: find the range, pick a scale
// that spreads the grid across it, round to the nearest grid point; 16 levels at 4
// bits): every decision is taken in binary64 with the same IEEE operations (products
// with the per-channel factor, one division for the scale, rounding half to even,
// binary16 rounded up), with contraction into fused multiply-adds disabled, so the
// codes, scales and zero points are bit-identical to the host's.
//
// One thread per (output row, group of contiguous channels); the eight rows of one
// packed zero-point word are eight consecutive lanes, whose zero points are combined
// with lane shuffles.
#pragma once

#include "nibbles.hpp"

namespace w4a16 {

#pragma clang fp contract(off)

__device__ __forceinline__ double half_bits_to_double(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v = e == 0 ? ldexp(static_cast<double>(m), -24) : ldexp(static_cast<double>(m | 0x400), e - 25);
  return (h & 0x8000) ? -v : v;
}

// Binary16 rounded to nearest (ties to even) from a finite binary64 value.
__device__ __forceinline__ uint16_t double_to_half_bits(double d) {
  const uint16_t sign = signbit(d) ? 0x8000 : 0;
  const double a = fabs(d);
  if (a >= 65520.0) return sign | 0x7C00;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  const int ulp_exp = max(e - 11, -24);
  uint32_t r = static_cast<uint32_t>(rint(ldexp(a, -ulp_exp)));
  if (ulp_exp == -24) return sign | static_cast<uint16_t>(r);
  int E = ulp_exp + 10;
  if (r == 2048) {
    r = 1024;
    E += 1;
  }
  if (E > 15) return sign | 0x7C00;
  return sign | static_cast<uint16_t>(((E + 15) << 10) | (r - 1024));
}

// Smallest binary16 >= v (finite v > 0).
__device__ __forceinline__ uint16_t half_ceil_bits(double v) {
  uint16_t h = double_to_half_bits(v);
  if (half_bits_to_double(h) < v) h = static_cast<uint16_t>(h + 1);
  return h;
}

// Element e of a packed word sits in nibble (0, 4, 1, 5, 2, 6, 3, 7)[e].
__device__ __forceinline__ int nibble_of(int e) { return (e & 1) ? 4 + (e >> 1) : (e >> 1); }

// Grid: N * G threads, thread t -> group t / N, row t % N (rows fastest, so the rows of
// a zero-point word are neighbouring lanes).  Needs N % 8 == 0 and a block size that
// is a multiple of 8.
template <bool SYM>
__global__ __launch_bounds__(256) void quantize_rtn_kernel(const uint16_t* __restrict__ w,
                                                           const double* __restrict__ in_scale, int N, int K,
                                                           int group_size, uint32_t* __restrict__ qweight,
                                                           uint16_t* __restrict__ scales,
                                                           uint32_t* __restrict__ qzeros) {
  const int G = K / group_size;
  const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const bool live = t < static_cast<long long>(N) * G;
  const int n = live ? static_cast<int>(t % N) : 0;
  const int g = live ? static_cast<int>(t / N) : 0;
  const int k0 = g * group_size;
  const uint16_t* row = w + static_cast<size_t>(n) * K;
  auto value = [&](int k) {
    const double v = half_bits_to_double(row[k]);
    return in_scale ? v * in_scale[k] : v;
  };
  uint32_t z = 0;
  if (live) {
    double S, Z = 0.0;
    uint16_t sbits;
    bool flat;
    if constexpr (SYM) {
      double a = 0.0;
      for (int i = 0; i < group_size; ++i) a = fmax(a, fabs(value(k0 + i)));
      flat = a == 0.0;
      sbits = flat ? 0x3C00 : half_ceil_bits(a / 7.0);
      z = 8;
    } else {
      double lo = 0.0, hi = 0.0;
      for (int i = 0; i < group_size; ++i) {
        const double v = value(k0 + i);
        lo = fmin(lo, v);
        hi = fmax(hi, v);
      }
      flat = hi == lo;
      sbits = flat ? 0x3C00 : half_ceil_bits((hi - lo) / 15.0);
      if (!flat) {
        Z = fmin(fmax(rint(-lo / half_bits_to_double(sbits)), 0.0), 15.0);
        z = static_cast<uint32_t>(Z);
      }
    }
    S = half_bits_to_double(sbits);
    scales[static_cast<size_t>(g) * N + n] = sbits;
    uint32_t* out = qweight + static_cast<size_t>(n) * (K / 8) + k0 / 8;
    for (int wd = 0; wd < group_size / 8; ++wd) {
      uint32_t word = 0;
      for (int e = 0; e < 8; ++e) {
        uint32_t q;
        if (flat) {
          q = SYM ? 8u : 0u;
        } else if constexpr (SYM) {
          q = static_cast<uint32_t>(fmin(fmax(rint(value(k0 + 8 * wd + e) / S), -7.0), 7.0) + 8.0);
        } else {
          q = static_cast<uint32_t>(fmin(fmax(rint(value(k0 + 8 * wd + e) / S) + Z, 0.0), 15.0));
        }
        word |= q << (4 * nibble_of(e));
      }
      out[wd] = word;
    }
  }
  if constexpr (!SYM) {
    // zero points of rows 8j .. 8j + 7: lanes with the same t / 8
    const int lane8 = threadIdx.x & 7;
    uint32_t word = z << (4 * lane8);
    word |= __shfl_xor(word, 1);
    word |= __shfl_xor(word, 2);
    word |= __shfl_xor(word, 4);
    if (live && lane8 == 0) qzeros[static_cast<size_t>(g) * (N / 8) + n / 8] = word;
  }
}

// Activations divided by the per-channel factor, rounded once to binary16 (the AWQ fold
// on the activation side, as the host computes it).
__global__ __launch_bounds__(256) void fold_activations_kernel(const uint16_t* __restrict__ x,
                                                               const double* __restrict__ s, size_t count, int K,
                                                               uint16_t* __restrict__ out) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  out[i] = double_to_half_bits(half_bits_to_double(x[i]) / s[i % K]);
}

#pragma clang fp contract(on)

}  // namespace w4a16
