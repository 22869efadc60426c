// Driver for the sanitizer build of the library's host (offline) code: compiled with
// g++ -fsanitize=address,undefined together with csrc/host.cpp (no HIP), it calls every
// host entry point on seeded random shapes, including act order, per-channel groups,
// symmetric and 8-bit weights and refused arguments, and checks the round trips
// (unpack o pack = identity for codes and zero points) and the ranges of what the
// quantisers write.  Any finding of the sanitizers aborts with a non-zero status.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "w4a16.h"

namespace {

std::mt19937_64 rng(20261203);

uint16_t to_half(float f) {
  // round-to-nearest-even binary16 of a float in the normal range (test data only)
  uint32_t u;
  std::memcpy(&u, &f, 4);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const int e = static_cast<int>((u >> 23) & 0xFF) - 127 + 15;
  uint32_t m = u & 0x7FFFFFu;
  if (e <= 0) return static_cast<uint16_t>(sign);
  if (e >= 31) return static_cast<uint16_t>(sign | 0x7BFFu);
  uint32_t h = sign | (static_cast<uint32_t>(e) << 10) | (m >> 13);
  const uint32_t rem = m & 0x1FFFu;
  if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) ++h;
  return static_cast<uint16_t>(h);
}

int failures = 0;
void check(bool ok, const char* what, int N, int K, int g) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (N=%d K=%d g=%d): %s\n", what, N, K, g, w4a16_last_error());
    ++failures;
  }
}

std::vector<int32_t> random_gidx(int K, int g) {
  std::vector<int32_t> perm(K), gidx(K);
  for (int k = 0; k < K; ++k) perm[k] = k;
  std::shuffle(perm.begin(), perm.end(), rng);
  for (int i = 0; i < K; ++i) gidx[perm[i]] = i / g;
  return gidx;
}

void one_layer(int N, int K, int g, bool act, int bits) {
  const int G = K / g;
  std::normal_distribution<float> nd(0.f, 0.02f);
  std::vector<uint16_t> w(static_cast<size_t>(N) * K);
  for (auto& v : w) v = to_half(nd(rng));
  std::vector<int32_t> gidx = act ? random_gidx(K, g) : std::vector<int32_t>();
  const int32_t* gi = act ? gidx.data() : nullptr;
  std::vector<double> s(K);
  std::uniform_real_distribution<double> us(0.25, 4.0);
  for (auto& v : s) v = us(rng);
  std::vector<uint8_t> codes(static_cast<size_t>(N) * K), back(codes.size()), zeros(static_cast<size_t>(G) * N),
      zback(zeros.size());
  std::vector<uint16_t> scales(static_cast<size_t>(G) * N);
  const int top = bits == 4 ? 15 : 255;
  for (int sym = 0; sym < 2; ++sym) {
    int rc;
    if (bits == 4)
      rc = sym ? w4a16_quantize_sym(w.data(), N, K, g, gi, s.data(), codes.data(), scales.data())
               : w4a16_quantize(w.data(), N, K, g, gi, s.data(), codes.data(), scales.data(), zeros.data());
    else
      rc = sym ? w8a16_quantize_sym(w.data(), N, K, g, gi, nullptr, codes.data(), scales.data())
               : w8a16_quantize(w.data(), N, K, g, gi, nullptr, codes.data(), scales.data(), zeros.data());
    check(rc == W4A16_OK, "quantize", N, K, g);
    bool in_range = true;
    for (uint8_t c : codes) in_range &= c <= top;
    check(in_range, "codes in range", N, K, g);
    const size_t words = bits == 4 ? w4a16_qweight_words(N, K, act) : w8a16_qweight_words(N, K, act);
    std::vector<int32_t> qw(words);
    rc = bits == 4 ? w4a16_pack(codes.data(), gi, g, N, K, qw.data()) : w8a16_pack(codes.data(), gi, g, N, K, qw.data());
    check(rc == W4A16_OK, "pack", N, K, g);
    rc = bits == 4 ? w4a16_unpack(qw.data(), gi, g, N, K, back.data())
                   : w8a16_unpack(qw.data(), gi, g, N, K, back.data());
    check(rc == W4A16_OK && back == codes, "unpack(pack(codes)) == codes", N, K, g);
  }
  std::vector<int32_t> qz(static_cast<size_t>(G) * N / (bits == 4 ? 8 : 4));
  int rc = bits == 4 ? w4a16_pack_zeros(zeros.data(), G, N, qz.data()) : w8a16_pack_zeros(zeros.data(), G, N, qz.data());
  check(rc == W4A16_OK, "pack_zeros", N, K, g);
  rc = bits == 4 ? w4a16_unpack_zeros(qz.data(), G, N, zback.data()) : w8a16_unpack_zeros(qz.data(), G, N, zback.data());
  check(rc == W4A16_OK && zback == zeros, "unpack_zeros(pack_zeros(z)) == z", N, K, g);
}

void activations(int T, int K, int g) {
  std::normal_distribution<float> nd(0.f, 1.f);
  std::vector<uint16_t> x(static_cast<size_t>(T) * K), xo(x.size());
  for (auto& v : x) v = to_half(nd(rng));
  std::vector<double> s(K);
  check(w4a16_awq_scales(x.data(), T, K, 0.5, s.data()) == W4A16_OK, "awq_scales", T, K, g);
  bool pos = true;
  for (double v : s) pos &= v > 0.0 && std::isfinite(v);
  check(pos, "awq scales positive", T, K, g);
  check(w4a16_awq_fold_activations(x.data(), T, K, s.data(), xo.data()) == W4A16_OK, "fold", T, K, g);
  check(w4a16_awq_fold_activations(x.data(), T, K, s.data(), x.data()) == W4A16_OK, "fold in place", T, K, g);
  std::vector<int32_t> gidx(K), count(K / g, 0);
  check(w4a16_act_order(xo.data(), T, K, g, gidx.data()) == W4A16_OK, "act_order", T, K, g);
  bool ok = true;
  for (int32_t v : gidx) {
    ok &= v >= 0 && v < K / g;
    if (v >= 0 && v < K / g) ++count[v];
  }
  for (int c : count) ok &= c == g;
  check(ok, "act-order groups of exactly g members", T, K, g);
}

void refusals() {
  std::vector<uint8_t> codes(64 * 64, 3);
  std::vector<int32_t> qw(64 * 8 + 64);
  std::vector<int32_t> bad(64, 0);   // every channel in group 0: not g members per group
  check(w4a16_pack(codes.data(), nullptr, 48, 64, 64, qw.data()) == W4A16_ERR_UNSUPPORTED, "group 48 refused", 64, 64, 48);
  check(w4a16_pack(codes.data(), bad.data(), 32, 64, 64, qw.data()) == W4A16_ERR_BAD_GIDX, "bad g_idx refused", 64, 64, 32);
  check(w4a16_pack(codes.data(), nullptr, 32, 60, 64, qw.data()) == W4A16_ERR_INVALID_ARG, "N % 8 refused", 60, 64, 32);
  check(w4a16_pack(nullptr, nullptr, 32, 64, 64, qw.data()) == W4A16_ERR_INVALID_ARG, "NULL refused", 64, 64, 32);
  codes[5] = 16;
  check(w4a16_pack(codes.data(), nullptr, 32, 64, 64, qw.data()) == W4A16_ERR_INVALID_ARG, "code 16 refused", 64, 64, 32);
  check(w4a16_qweight_words(0, 64, 0) == 0, "empty layer has no words", 0, 64, 32);
}

}  // namespace

int main() {
  const int gs[] = {32, 64, 128};
  for (int it = 0; it < 40; ++it) {
    const int N = 8 * static_cast<int>(1 + rng() % 12);
    const int g = gs[rng() % 3];
    const int K = g * static_cast<int>(1 + rng() % 6);
    one_layer(N, K, g, rng() & 1, (rng() % 3 == 0) ? 8 : 4);
    one_layer(N, K, K, false, 4);                       // one group per row
    activations(static_cast<int>(1 + rng() % 40), K, g);
  }
  refusals();
  std::printf("host sanitizer driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
