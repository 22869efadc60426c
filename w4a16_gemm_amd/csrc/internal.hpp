// Shared host-side helpers of the W4A16 library: error state, argument checks and
// the private weight-buffer layout.  No HIP dependency.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "w4a16.h"

namespace w4a16 {

// Record `code` with a printf-style message as the calling thread's last error.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// N/K > 0, group_size in {32, 64, 128} or K, K % group_size == 0, K % 32 == 0,
// N % 8 == 0.
int check_shape(int N, int K, int group_size);

// g_idx (host memory): every value in [0, G) and every group exactly group_size
// members.  On success fills perm (size K) with the stable sort of k by g_idx[k].
int check_gidx_and_sort(const int32_t* g_idx, int K, int group_size, int32_t* perm);

// GPTQ act order ("AWQ + GPTQ Quantization, in depth", The two algorithms, compactly):
// input channels by descending sum_t X[t][k]^2 (exact), ties by ascending k.
// xcal binary16 [T][K] (host); fails on a non-finite value.
int act_order_rank(const uint16_t* xcal, int T, int K, std::vector<int32_t>& order);

// Private weight-buffer layout (the ABI treats it as opaque).
//   words [N][K/8]: word w of row n holds the codes of stored positions 8w..8w+7;
//   stored position p holds input channel p (contiguous groups) or perm[p] (act
//   order).  Element e of a word (position 8w+e) sits in nibble kNibbleOf[e], chosen
//   so that masking the word with 0x000F000F / 0x00F000F0 (and the same after a
//   shift by 8) yields the pairs (e0,e1), (e2,e3), (e4,e5), (e6,e7) as the low and
//   high halves of 32-bit registers, i.e. consecutive input channels, which is the
//   order in which the activations sit in memory.
//   tail (act order only): int32 perm[K].
constexpr int kNibbleOf[8] = {0, 4, 1, 5, 2, 6, 3, 7};

inline size_t qweight_words(int N, int K, bool act_order) {
  return static_cast<size_t>(N) * static_cast<size_t>(K / 8) + (act_order ? static_cast<size_t>(K) : 0);
}

// 8-bit weights: words [N][K/4], element e of a word (stored position 4w+e) in byte
// kByteOf[e], so that masking with 0x00FF00FF (and the same after a shift by 8) gives
// the pairs (e0,e1), (e2,e3) of consecutive input channels.  Same act-order tail.
// Zero points [G][N/4]: byte j of word [g][n/4] is Z of (g, 4 (n/4) + j).
constexpr int kByteOf[4] = {0, 2, 1, 3};

inline size_t qweight8_words(int N, int K, bool act_order) {
  return static_cast<size_t>(N) * static_cast<size_t>(K / 4) + (act_order ? static_cast<size_t>(K) : 0);
}

}  // namespace w4a16
