// Register-level expansion of packed 4-bit codes for gfx950.
//
// The packed word layout puts element e of a word in nibble {0,4,1,5,2,6,3,7}[e].
// With that order, two AND-OR operations per 16-bit half pair turn a word into
// four 32-bit registers, each holding two binary16 values of consecutive elements:
//
//   (w & 0x000F000F) | 0x64006400         -> (1024 + q_e0, 1024 + q_e1)
//   (w & 0x00F000F0) | 0x64006400         -> (1024 + 16 q_e2, 1024 + 16 q_e3)
//   ((w >> 8) & 0x000F000F) | 0x64006400  -> (1024 + q_e4, 1024 + q_e5)
//   ((w >> 8) & 0x00F000F0) | 0x64006400  -> (1024 + 16 q_e6, 1024 + 16 q_e7)
//
// 0x6400 is binary16 1024.0, whose ulp is 1, so OR-ing a 4-bit (or 4-bit << 4)
// integer into the mantissa gives the exact values above.  Every later step that
// turns them into q - Z is exact as well; the only rounding is the final
// multiplication by the binary16 scale, which is therefore the same rounding as
// binary16((q - Z) * S) ("AWQ + GPTQ Quantization, in depth", What W4A16 buys:
// the kernel expands the packed weights to 16 bits in registers with the group's
// scale and zero point).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Packed codes read once per launch (the decode GEMV streams every weight exactly once)
// go through a raw buffer resource over the code array: a 32-bit byte offset per lane
// instead of a 64-bit address (fewer VGPRs and address instructions), and the load is
// non-temporal, so the stream does not displace the scales, zero points and
// activations from the caches.  Measured on the 70B-class decode layer (same box):
// global load 23.1 us, global non-temporal 22.5 us, buffer non-temporal 21.9 us; the
// coherence-scope bits made no difference.  The skinny-batch kernel measured slower
// with the non-temporal hint (+2..4% at M = 2..8) and keeps plain loads.
constexpr uint32_t kBufferWord3 = 0x00020000u;   // gfx9 raw buffer: 32-bit data format
constexpr int kCpolNonTemporal = 2;             // cache-policy bits: nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t stream_rsrc(const uint32_t* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(p), 0, static_cast<int>(bytes), kBufferWord3);
}

__device__ __forceinline__ uint4 load_stream16(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_offset), 0,
                                                                         kCpolNonTemporal));
}

// The same 16-byte buffer load with the default cache policy.
__device__ __forceinline__ uint4 load_buffer16(__amdgpu_buffer_rsrc_t r, uint32_t byte_offset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_offset), 0, 0));
}

constexpr uint32_t kMagic = 0x64006400u;  // (1024.0, 1024.0) in binary16

struct Pairs {
  uint32_t a0;  // (1024 + q0, 1024 + q1)
  uint32_t b0;  // (1024 + 16 q2, 1024 + 16 q3)
  uint32_t a1;  // (1024 + q4, 1024 + q5)
  uint32_t b1;  // (1024 + 16 q6, 1024 + 16 q7)
};

// (a & mask) | c in one v_and_or_b32.  gfx9 VOP3 cannot encode two literal
// constants, so left to itself the compiler emits v_and_b32 + v_or_b32; the mask is
// passed in a scalar register and c in a vector register instead.  ALU only.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(c));
  return d;
}

__device__ __forceinline__ Pairs expand_word(uint32_t w) {
  Pairs p;
  p.a0 = and_or(w, 0x000F000Fu, kMagic);
  p.b0 = and_or(w, 0x00F000F0u, kMagic);
  const uint32_t v = w >> 8;
  p.a1 = and_or(v, 0x000F000Fu, kMagic);
  p.b1 = and_or(v, 0x00F000F0u, kMagic);
  return p;
}

// The same pairs without the 1024 offset: masking alone leaves q (or 16 q) in the
// mantissa of a binary16 with a zero exponent field, i.e. the exact subnormal
// q * 2^-24.  v_dot2_f32_f16 keeps binary16 subnormal inputs (the kernels run with
// fp16/fp64 denormals enabled), and every product with an activation is exact in
// fp32, so the 2^-24 can be folded into the scale afterwards.  One plain AND per
// pair, no offset to subtract.
struct SubPairs {
  uint32_t a0;  // (q0, q1) * 2^-24
  uint32_t b0;  // (q2, q3) * 16 * 2^-24
  uint32_t a1;  // (q4, q5) * 2^-24
  uint32_t b1;  // (q6, q7) * 16 * 2^-24
};

__device__ __forceinline__ SubPairs expand_word_subnormal(uint32_t w) {
  SubPairs p;
  p.a0 = w & 0x000F000Fu;
  p.b0 = w & 0x00F000F0u;
  const uint32_t v = w >> 8;
  p.a1 = v & 0x000F000Fu;
  p.b1 = v & 0x00F000F0u;
  return p;
}

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

// Per (group, output) constants for building binary16 weights (q - Z) * S.
struct DequantConsts {
  half2_t neg_1024_z;  // -(1024 + Z)
  half2_t neg_64_z;    // -(64 + Z)
  half2_t scale;       // S
};

// Built with integer operations: binary16 1024 is 0x6400 with an ulp of 1, so -(1024 +
// z) is 0xE400 | z for z < 1024; binary16 64 is 0x5400 with an ulp of 1/16, so -(64 +
// z) is 0xD400 | (z << 4) for z < 64 (4-bit zero points only use it).
__device__ __forceinline__ DequantConsts make_consts(uint32_t z, half_t s) {
  DequantConsts c;
  const uint32_t a = 0xE400u | z;
  const uint32_t b = 0xD400u | (z << 4);
  const uint32_t sb = __builtin_bit_cast(uint16_t, s);
  c.neg_1024_z = as_h2(a | (a << 16));
  c.neg_64_z = as_h2(b | (b << 16));
  c.scale = as_h2(sb | (sb << 16));
  return c;
}

// Eight binary16 weights binary16((q_e - Z) * S), e = 0..7, in element order.
__device__ __forceinline__ half8_t dequant_word(uint32_t w, const DequantConsts& c) {
  const Pairs p = expand_word(w);
  const half2_t sixteenth = half2_t{static_cast<half_t>(0.0625f), static_cast<half_t>(0.0625f)};
  const half2_t d0 = (as_h2(p.a0) + c.neg_1024_z) * c.scale;
  const half2_t d1 = __builtin_elementwise_fma(as_h2(p.b0), sixteenth, c.neg_64_z) * c.scale;
  const half2_t d2 = (as_h2(p.a1) + c.neg_1024_z) * c.scale;
  const half2_t d3 = __builtin_elementwise_fma(as_h2(p.b1), sixteenth, c.neg_64_z) * c.scale;
  return half8_t{d0.x, d0.y, d1.x, d1.y, d2.x, d2.y, d3.x, d3.y};
}

// 8-bit weights: four binary16 weights binary16((q_e - Z) * S), e = 0..3, of a word in
// the private byte order (element e in byte 0, 2, 1, 3): OR-ing a byte pair into the
// mantissas of 1024 gives (1024 + q) exactly, and (1024 + q) - (1024 + Z) = q - Z is
// exact, so the product with S is the only rounding.
__device__ __forceinline__ half4_t dequant_word8(uint32_t w, const DequantConsts& c) {
  const half2_t d0 = (as_h2((w & 0x00FF00FFu) | 0x64006400u) + c.neg_1024_z) * c.scale;
  const half2_t d1 = (as_h2(((w >> 8) & 0x00FF00FFu) | 0x64006400u) + c.neg_1024_z) * c.scale;
  return half4_t{d0.x, d0.y, d1.x, d1.y};
}

// Workgroup -> position in a sweep over row units, so that the workgroups of one XCD
// (dispatch is round-robin over the 8 XCDs) own neighbouring units: the streams of
// one XCD's L2 then cover one contiguous stretch of the weights.
__device__ __forceinline__ int xcd_block(int bid, int nblk) {
  if (nblk % 8 != 0) return bid;
  return (bid % 8) * (nblk / 8) + bid / 8;
}

// Zero points of a layer.  Asymmetric: packed words [G][N/8], Z of (group g, output n)
// in bits 4 (n % 8) .. +3 of word [g][n / 8].  Symmetric (sym != 0): every Z is 8
// (the signed code q - 8 in [-7, 7] times S, "LLM Quantization: INT8, GPTQ, and AWQ
// Explained", What quantization actually does: absmax) and nothing is stored; `words`
// then points at any readable word, every zero-point load of the kernels reads that one
// word (so the loads keep their place in the wait counts but stay in the cache), and
// the loaded words are replaced by kSymZeroWord.
// 8-bit weights: packed words [G][N/4], Z of (g, n) in byte n % 4 of word [g][n / 4]
// (so byte g N + n of the buffer); symmetric: every Z is 128.
constexpr uint32_t kSymZeroWord = 0x88888888u;
constexpr uint32_t kSymZeroWord8 = 0x80808080u;

struct Zeros {
  const uint32_t* words;
  int sym;
  __device__ __forceinline__ const uint32_t* at(size_t idx) const { return words + (sym ? 0 : idx); }
  __device__ __forceinline__ uint32_t word(uint32_t loaded) const { return sym ? kSymZeroWord : loaded; }
  __device__ __forceinline__ uint32_t word8(uint32_t loaded) const { return sym ? kSymZeroWord8 : loaded; }
};

// Zero point of (group gi, output n).
template <int BITS = 4>
__device__ __forceinline__ uint32_t load_zero(Zeros z, int gi, int N, int n) {
  if constexpr (BITS == 4) {
    if (z.sym) return 8u;
    return (z.words[static_cast<size_t>(gi) * (N >> 3) + (n >> 3)] >> ((n & 7) * 4)) & 0xFu;
  } else {
    if (z.sym) return 128u;
    return (z.words[static_cast<size_t>(gi) * (N >> 2) + (n >> 2)] >> ((n & 3) * 8)) & 0xFFu;
  }
}

}  // namespace w4a16
