// Host-side (offline) entry points of the W4A16 library: packing, the round-to-
// nearest group quantiser, the AWQ scale and fold, and the act-order assignment.
// Plain C++ with no HIP dependency; built with -ffp-contract=off so that every
// binary64 operation is rounded exactly as written.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>
#include <vector>

#include "internal.hpp"

namespace w4a16 {

namespace {
thread_local std::string t_last_error;

constexpr int kLevels = 15;  // 16 grid points, "4 bits ... 16 levels"
constexpr int kSymLevels = 7;    // symmetric grid -7 .. 7 (stored code of 0: 8)
constexpr int kLevels8 = 255;    // 8-bit weights: 256 grid points
constexpr int kSymLevels8 = 127; // symmetric 8-bit grid -127 .. 127 (stored code of 0: 128)

// Exact binary16 -> binary64.
double half_to_double(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0) {
    v = std::ldexp(static_cast<double>(m), -24);
  } else if (e == 0x1F) {
    v = m ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(m | 0x400), e - 25);
  }
  return (h & 0x8000) ? -v : v;
}

// binary64 -> binary16, rounded to nearest, ties to even.
uint16_t double_to_half(double d) {
  const uint16_t sign = std::signbit(d) ? 0x8000 : 0;
  if (std::isnan(d)) return sign | 0x7E00;
  const double a = std::fabs(d);
  if (a >= 65520.0) return sign | 0x7C00;  // beyond max + half an ulp: infinity
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);                        // a = f * 2^e, f in [0.5, 1)
  const int ulp_exp = std::max(e - 11, -24);  // ulp of the binary16 result
  const double r = std::nearbyint(std::ldexp(a, -ulp_exp));  // ties to even
  uint32_t ri = static_cast<uint32_t>(r);
  if (ulp_exp == -24) return sign | static_cast<uint16_t>(ri);  // subnormal / first binade
  int E = ulp_exp + 10;
  if (ri == 2048) {
    ri = 1024;
    E += 1;
  }
  if (E > 15) return sign | 0x7C00;
  return sign | static_cast<uint16_t>(((E + 15) << 10) | (ri - 1024));
}

// Smallest binary16 value >= v, for finite v > 0.
uint16_t half_ceil(double v) {
  uint16_t h = double_to_half(v);
  if (half_to_double(h) < v) h = static_cast<uint16_t>(h + 1);
  return h;
}

// |x| * 2^24 for a binary16 x: an exact integer below 2^40.
int64_t half_abs_units(uint16_t h) {
  return static_cast<int64_t>(std::fabs(half_to_double(h)) * 16777216.0);
}

bool half_is_finite(uint16_t h) { return ((h >> 10) & 0x1F) != 0x1F; }

// Input channels of every group: contiguous runs, or the members named by g_idx.
int group_members(const int32_t* g_idx, int K, int group_size, std::vector<int32_t>& order) {
  order.resize(K);
  if (g_idx == nullptr) {
    for (int k = 0; k < K; ++k) order[k] = k;
    return W4A16_OK;
  }
  return check_gidx_and_sort(g_idx, K, group_size, order.data());
}
// Checks shared by the quantisers.
int check_quantize_args(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                        const double* in_scale, std::vector<int32_t>& order) {
  if (int st = check_shape(N, K, group_size)) return st;
  if (int st = group_members(g_idx, K, group_size, order)) return st;
  if (in_scale)
    for (int k = 0; k < K; ++k)
      if (!(in_scale[k] > 0.0) || !std::isfinite(in_scale[k]))
        return fail(W4A16_ERR_INVALID_ARG, "in_scale[%d] is not a positive finite number", k);
  const size_t nk = static_cast<size_t>(N) * K;
  for (size_t i = 0; i < nk; ++i)
    if (!half_is_finite(w[i])) return fail(W4A16_ERR_INVALID_ARG, "weight %zu is not finite", i);
  return W4A16_OK;
}

// Row n of the weights, times the per-input-channel factor if any, in binary64.
void load_row(const uint16_t* w, int K, int n, const double* in_scale, std::vector<double>& row) {
  for (int k = 0; k < K; ++k) {
    const double v = half_to_double(w[static_cast<size_t>(n) * K + k]);
    row[k] = in_scale ? v * in_scale[k] : v;
  }
}

// The stored channel order of a weight buffer: its act-order tail, checked to be a
// permutation that agrees with g_idx, or the identity.
int stored_order(const int32_t* tail, const int32_t* g_idx, int K, int group_size, std::vector<int32_t>& perm) {
  if (!g_idx) {
    for (int p = 0; p < K; ++p) perm[p] = p;
    return W4A16_OK;
  }
  std::vector<char> seen(K, 0);
  for (int p = 0; p < K; ++p) {
    const int32_t k = tail[p];
    if (k < 0 || k >= K || seen[k])
      return fail(W4A16_ERR_BAD_GIDX, "stored order is not a permutation at position %d", p);
    seen[k] = 1;
    if (g_idx[k] != p / group_size)
      return fail(W4A16_ERR_BAD_GIDX, "stored order disagrees with g_idx at position %d", p);
    perm[p] = k;
  }
  return W4A16_OK;
}

// Asymmetric round-to-nearest on the grid 0 .. levels (15 or 255).
int quantize_asym(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx, const double* in_scale,
                  int levels, uint8_t* codes, uint16_t* scales, uint8_t* zeros) {
  if (!w || !codes || !scales || !zeros) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  std::vector<int32_t> order;
  if (int st = check_quantize_args(w, N, K, group_size, g_idx, in_scale, order)) return st;
  const int G = K / group_size;
  const double L = static_cast<double>(levels);
  std::vector<double> row(K);
  for (int n = 0; n < N; ++n) {
    load_row(w, K, n, in_scale, row);
    for (int g = 0; g < G; ++g) {
      const int32_t* members = order.data() + static_cast<size_t>(g) * group_size;
      double lo = 0.0, hi = 0.0;
      for (int i = 0; i < group_size; ++i) {
        lo = std::min(lo, row[members[i]]);
        hi = std::max(hi, row[members[i]]);
      }
      uint8_t* qrow = codes + static_cast<size_t>(n) * K;
      const size_t gi = static_cast<size_t>(g) * N + n;
      if (hi == lo) {  // all-zero group
        scales[gi] = 0x3C00;  // 1.0
        zeros[gi] = 0;
        for (int i = 0; i < group_size; ++i) qrow[members[i]] = 0;
        continue;
      }
      const uint16_t sbits = half_ceil((hi - lo) / L);
      const double S = half_to_double(sbits);
      const double Z = std::min(std::max(std::nearbyint(-lo / S), 0.0), L);
      scales[gi] = sbits;
      zeros[gi] = static_cast<uint8_t>(Z);
      for (int i = 0; i < group_size; ++i) {
        const double q = std::nearbyint(row[members[i]] / S) + Z;
        qrow[members[i]] = static_cast<uint8_t>(std::min(std::max(q, 0.0), L));
      }
    }
  }
  return W4A16_OK;
}

// Symmetric round-to-nearest on the grid -levels .. levels (7 or 127), stored as
// code = q + levels + 1.
int quantize_sym(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx, const double* in_scale,
                 int levels, uint8_t* codes, uint16_t* scales) {
  if (!w || !codes || !scales) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  std::vector<int32_t> order;
  if (int st = check_quantize_args(w, N, K, group_size, g_idx, in_scale, order)) return st;
  const int G = K / group_size;
  const double L = static_cast<double>(levels);
  const uint8_t zero = static_cast<uint8_t>(levels + 1);
  std::vector<double> row(K);
  for (int n = 0; n < N; ++n) {
    load_row(w, K, n, in_scale, row);
    for (int g = 0; g < G; ++g) {
      const int32_t* members = order.data() + static_cast<size_t>(g) * group_size;
      double a = 0.0;
      for (int i = 0; i < group_size; ++i) a = std::max(a, std::fabs(row[members[i]]));
      uint8_t* qrow = codes + static_cast<size_t>(n) * K;
      const size_t gi = static_cast<size_t>(g) * N + n;
      if (a == 0.0) {  // all-zero group: S = 1, every code the zero
        scales[gi] = 0x3C00;
        for (int i = 0; i < group_size; ++i) qrow[members[i]] = zero;
        continue;
      }
      const uint16_t sbits = half_ceil(a / L);
      const double S = half_to_double(sbits);
      scales[gi] = sbits;
      for (int i = 0; i < group_size; ++i) {
        const double q = std::min(std::max(std::nearbyint(row[members[i]] / S), -L), L);
        qrow[members[i]] = static_cast<uint8_t>(q + zero);
      }
    }
  }
  return W4A16_OK;
}
}  // namespace

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return code;
}

void clear_error() { t_last_error.clear(); }

int check_shape(int N, int K, int group_size) {
  if (N <= 0 || K <= 0) return fail(W4A16_ERR_INVALID_ARG, "N and K must be positive (N=%d K=%d)", N, K);
  // groups of 32, 64 or 128 input channels, or one group per row (per-channel, g = K)
  if (group_size != 32 && group_size != 64 && group_size != 128 && group_size != K)
    return fail(W4A16_ERR_UNSUPPORTED, "group_size %d is not supported (32, 64, 128 or K=%d)", group_size, K);
  if (K % group_size != 0)
    return fail(W4A16_ERR_INVALID_ARG, "K=%d is not a multiple of group_size=%d", K, group_size);
  if (K % 32 != 0) return fail(W4A16_ERR_INVALID_ARG, "K=%d is not a multiple of 32", K);
  if (N % 8 != 0) return fail(W4A16_ERR_INVALID_ARG, "N=%d is not a multiple of 8", N);
  return W4A16_OK;
}

int act_order_rank(const uint16_t* xcal, int T, int K, std::vector<int32_t>& order) {
  // sum_t X^2 exactly, in units of 2^-48 (each square is below 2^80)
  std::vector<__int128> h(K, 0);
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      const uint16_t v = xcal[static_cast<size_t>(t) * K + k];
      if (!half_is_finite(v)) return fail(W4A16_ERR_INVALID_ARG, "calibration value not finite");
      const __int128 u = half_abs_units(v);
      h[k] += u * u;
    }
  order.resize(K);
  for (int k = 0; k < K; ++k) order[k] = k;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return h[a] > h[b]; });
  return W4A16_OK;
}

int check_gidx_and_sort(const int32_t* g_idx, int K, int group_size, int32_t* perm) {
  const int G = K / group_size;
  std::vector<int32_t> count(G, 0);
  for (int k = 0; k < K; ++k) {
    const int32_t gk = g_idx[k];
    if (gk < 0 || gk >= G)
      return fail(W4A16_ERR_BAD_GIDX, "g_idx[%d]=%d is outside [0, %d)", k, gk, G);
    ++count[gk];
  }
  for (int g = 0; g < G; ++g)
    if (count[g] != group_size)
      return fail(W4A16_ERR_BAD_GIDX, "group %d has %d members, expected %d", g, count[g], group_size);
  // counting sort: stable, ascending k inside each group
  std::vector<int32_t> next(G);
  for (int g = 0; g < G; ++g) next[g] = g * group_size;
  for (int k = 0; k < K; ++k) perm[next[g_idx[k]]++] = k;
  return W4A16_OK;
}

}  // namespace w4a16

using namespace w4a16;

extern "C" {

int w4a16_abi_version(void) { return W4A16_ABI_VERSION; }

const char* w4a16_last_error(void) { return t_last_error.c_str(); }

size_t w4a16_qweight_words(int N, int K, int act_order) {
  if (N <= 0 || K <= 0 || K % 8 != 0) return 0;
  return qweight_words(N, K, act_order != 0);
}

int w4a16_pack(const uint8_t* codes, const int32_t* g_idx, int group_size, int N, int K,
               int32_t* qweight) {
  clear_error();
  if (!codes || !qweight) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (int st = check_shape(N, K, group_size)) return st;
  std::vector<int32_t> perm;
  if (int st = group_members(g_idx, K, group_size, perm)) return st;
  const size_t nk = static_cast<size_t>(N) * K;
  for (size_t i = 0; i < nk; ++i)
    if (codes[i] > 15) return fail(W4A16_ERR_INVALID_ARG, "code %u at %zu is above 15", codes[i], i);
  const int W = K / 8;
  for (int n = 0; n < N; ++n) {
    const uint8_t* row = codes + static_cast<size_t>(n) * K;
    uint32_t* out = reinterpret_cast<uint32_t*>(qweight) + static_cast<size_t>(n) * W;
    for (int w = 0; w < W; ++w) {
      uint32_t word = 0;
      for (int e = 0; e < 8; ++e) word |= static_cast<uint32_t>(row[perm[8 * w + e]]) << (4 * kNibbleOf[e]);
      out[w] = word;
    }
  }
  if (g_idx)
    for (int p = 0; p < K; ++p) qweight[static_cast<size_t>(N) * W + p] = perm[p];
  return W4A16_OK;
}

int w4a16_unpack(const int32_t* qweight, const int32_t* g_idx, int group_size, int N, int K,
                 uint8_t* codes) {
  clear_error();
  if (!codes || !qweight) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (int st = check_shape(N, K, group_size)) return st;
  const int W = K / 8;
  std::vector<int32_t> perm(K);
  if (int st = stored_order(qweight + static_cast<size_t>(N) * W, g_idx, K, group_size, perm)) return st;
  for (int n = 0; n < N; ++n) {
    const uint32_t* in = reinterpret_cast<const uint32_t*>(qweight) + static_cast<size_t>(n) * W;
    uint8_t* row = codes + static_cast<size_t>(n) * K;
    for (int w = 0; w < W; ++w)
      for (int e = 0; e < 8; ++e) row[perm[8 * w + e]] = (in[w] >> (4 * kNibbleOf[e])) & 0xF;
  }
  return W4A16_OK;
}

size_t w8a16_qweight_words(int N, int K, int act_order) {
  if (N <= 0 || K <= 0 || K % 8 != 0) return 0;
  return qweight8_words(N, K, act_order != 0);
}

int w8a16_pack(const uint8_t* codes, const int32_t* g_idx, int group_size, int N, int K, int32_t* qweight) {
  clear_error();
  if (!codes || !qweight) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (int st = check_shape(N, K, group_size)) return st;
  std::vector<int32_t> perm;
  if (int st = group_members(g_idx, K, group_size, perm)) return st;
  const int W = K / 4;
  for (int n = 0; n < N; ++n) {
    const uint8_t* row = codes + static_cast<size_t>(n) * K;
    uint32_t* out = reinterpret_cast<uint32_t*>(qweight) + static_cast<size_t>(n) * W;
    for (int w = 0; w < W; ++w) {
      uint32_t word = 0;
      for (int e = 0; e < 4; ++e) word |= static_cast<uint32_t>(row[perm[4 * w + e]]) << (8 * kByteOf[e]);
      out[w] = word;
    }
  }
  if (g_idx)
    for (int p = 0; p < K; ++p) qweight[static_cast<size_t>(N) * W + p] = perm[p];
  return W4A16_OK;
}

int w8a16_unpack(const int32_t* qweight, const int32_t* g_idx, int group_size, int N, int K, uint8_t* codes) {
  clear_error();
  if (!codes || !qweight) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (int st = check_shape(N, K, group_size)) return st;
  const int W = K / 4;
  std::vector<int32_t> perm(K);
  if (int st = stored_order(qweight + static_cast<size_t>(N) * W, g_idx, K, group_size, perm)) return st;
  for (int n = 0; n < N; ++n) {
    const uint32_t* in = reinterpret_cast<const uint32_t*>(qweight) + static_cast<size_t>(n) * W;
    uint8_t* row = codes + static_cast<size_t>(n) * K;
    for (int w = 0; w < W; ++w)
      for (int e = 0; e < 4; ++e) row[perm[4 * w + e]] = (in[w] >> (8 * kByteOf[e])) & 0xFF;
  }
  return W4A16_OK;
}

int w8a16_pack_zeros(const uint8_t* zeros, int G, int N, int32_t* qzeros) {
  clear_error();
  if (!zeros || !qzeros) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (G <= 0 || N <= 0 || N % 8 != 0)
    return fail(W4A16_ERR_INVALID_ARG, "bad zero-point shape G=%d N=%d", G, N);
  for (int g = 0; g < G; ++g)
    for (int w = 0; w < N / 4; ++w) {
      uint32_t word = 0;
      for (int j = 0; j < 4; ++j) word |= static_cast<uint32_t>(zeros[static_cast<size_t>(g) * N + 4 * w + j]) << (8 * j);
      qzeros[static_cast<size_t>(g) * (N / 4) + w] = static_cast<int32_t>(word);
    }
  return W4A16_OK;
}

int w8a16_unpack_zeros(const int32_t* qzeros, int G, int N, uint8_t* zeros) {
  clear_error();
  if (!zeros || !qzeros) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (G <= 0 || N <= 0 || N % 8 != 0)
    return fail(W4A16_ERR_INVALID_ARG, "bad zero-point shape G=%d N=%d", G, N);
  for (int g = 0; g < G; ++g)
    for (int n = 0; n < N; ++n)
      zeros[static_cast<size_t>(g) * N + n] =
          (static_cast<uint32_t>(qzeros[static_cast<size_t>(g) * (N / 4) + n / 4]) >> (8 * (n % 4))) & 0xFF;
  return W4A16_OK;
}

int w4a16_pack_zeros(const uint8_t* zeros, int G, int N, int32_t* qzeros) {
  clear_error();
  if (!zeros || !qzeros) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (G <= 0 || N <= 0 || N % 8 != 0)
    return fail(W4A16_ERR_INVALID_ARG, "bad zero-point shape G=%d N=%d", G, N);
  for (int g = 0; g < G; ++g)
    for (int w = 0; w < N / 8; ++w) {
      uint32_t word = 0;
      for (int j = 0; j < 8; ++j) {
        const uint8_t z = zeros[static_cast<size_t>(g) * N + 8 * w + j];
        if (z > 15) return fail(W4A16_ERR_INVALID_ARG, "zero point %u above 15", z);
        word |= static_cast<uint32_t>(z) << (4 * j);
      }
      qzeros[static_cast<size_t>(g) * (N / 8) + w] = static_cast<int32_t>(word);
    }
  return W4A16_OK;
}

int w4a16_unpack_zeros(const int32_t* qzeros, int G, int N, uint8_t* zeros) {
  clear_error();
  if (!zeros || !qzeros) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (G <= 0 || N <= 0 || N % 8 != 0)
    return fail(W4A16_ERR_INVALID_ARG, "bad zero-point shape G=%d N=%d", G, N);
  for (int g = 0; g < G; ++g)
    for (int n = 0; n < N; ++n)
      zeros[static_cast<size_t>(g) * N + n] =
          (static_cast<uint32_t>(qzeros[static_cast<size_t>(g) * (N / 8) + n / 8]) >> (4 * (n % 8))) & 0xF;
  return W4A16_OK;
}

int w4a16_quantize(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                   const double* in_scale, uint8_t* codes, uint16_t* scales, uint8_t* zeros) {
  clear_error();
  return quantize_asym(w, N, K, group_size, g_idx, in_scale, kLevels, codes, scales, zeros);
}

int w4a16_quantize_sym(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                       const double* in_scale, uint8_t* codes, uint16_t* scales) {
  clear_error();
  return quantize_sym(w, N, K, group_size, g_idx, in_scale, kSymLevels, codes, scales);
}

int w8a16_quantize(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                   const double* in_scale, uint8_t* codes, uint16_t* scales, uint8_t* zeros) {
  clear_error();
  return quantize_asym(w, N, K, group_size, g_idx, in_scale, kLevels8, codes, scales, zeros);
}

int w8a16_quantize_sym(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                       const double* in_scale, uint8_t* codes, uint16_t* scales) {
  clear_error();
  return quantize_sym(w, N, K, group_size, g_idx, in_scale, kSymLevels8, codes, scales);
}

int w4a16_awq_scales(const uint16_t* xcal, int T, int K, double alpha, double* s) {
  clear_error();
  if (!xcal || !s) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (T <= 0 || K <= 0) return fail(W4A16_ERR_INVALID_ARG, "T and K must be positive");
  if (!(alpha >= 0.0) || !std::isfinite(alpha)) return fail(W4A16_ERR_INVALID_ARG, "alpha must be >= 0");
  std::vector<int64_t> total(K, 0);
  for (int t = 0; t < T; ++t)
    for (int k = 0; k < K; ++k) {
      const uint16_t h = xcal[static_cast<size_t>(t) * K + k];
      if (!half_is_finite(h)) return fail(W4A16_ERR_INVALID_ARG, "calibration value not finite");
      total[k] += half_abs_units(h);
    }
  const double denom = static_cast<double>(T) * 16777216.0;
  for (int k = 0; k < K; ++k) {
    const double mean = static_cast<double>(total[k]) / denom;
    if (mean == 0.0) {
      s[k] = 1.0;
    } else {
      s[k] = (alpha == 0.5) ? std::sqrt(mean) : std::pow(mean, alpha);
    }
  }
  return W4A16_OK;
}

int w4a16_awq_fold_activations(const uint16_t* x, int M, int K, const double* s, uint16_t* x_out) {
  clear_error();
  if (!x || !s || !x_out) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (M <= 0 || K <= 0) return fail(W4A16_ERR_INVALID_ARG, "M and K must be positive");
  for (int k = 0; k < K; ++k)
    if (!(s[k] > 0.0) || !std::isfinite(s[k]))
      return fail(W4A16_ERR_INVALID_ARG, "s[%d] is not a positive finite number", k);
  for (int m = 0; m < M; ++m)
    for (int k = 0; k < K; ++k) {
      const size_t i = static_cast<size_t>(m) * K + k;
      x_out[i] = double_to_half(half_to_double(x[i]) / s[k]);
    }
  return W4A16_OK;
}

int w4a16_act_order(const uint16_t* xcal, int T, int K, int group_size, int32_t* g_idx) {
  clear_error();
  if (!xcal || !g_idx) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (T <= 0) return fail(W4A16_ERR_INVALID_ARG, "T must be positive");
  if (int st = check_shape(8, K, group_size)) return st;
  std::vector<int32_t> order;
  if (int st = act_order_rank(xcal, T, K, order)) return st;
  for (int i = 0; i < K; ++i) g_idx[order[i]] = i / group_size;
  return W4A16_OK;
}

}  // extern "C"
