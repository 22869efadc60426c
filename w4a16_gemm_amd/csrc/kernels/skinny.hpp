// Skinny batches (M <= 16, decode with a few sequences): y^T = W^ x^T on the matrix
// cores, with the dequantised weights as the A operand (16 output rows per MFMA) and
// the activations as the B operand (the M rows padded to 16 columns).
//
// Like the GEMV this is HBM-bound ("AWQ + GPTQ Quantization, in depth", What W4A16
// buys: decoding reads every weight once per token), so the layout is built around
// streaming the codes once with 16-byte loads:
//  * A workgroup of W wavefronts splits K: wavefront w owns channels
//    [128 T w, 128 T (w + 1)) and keeps the activations of that slice in registers
//    for the whole kernel (T x 4 fragments of 8 binary16 per lane).
//  * The workgroup walks blocks of 16 output rows (every grid-th block, the workgroups
//    of one XCD taking neighbouring ones; dealing consecutive blocks to different XCDs
//    measured 15% slower on the 70B-class layer).  Per block and slice step t, lane
//    (r, q) = (lane % 16, lane / 16) loads 16 bytes of row r: the 32 channels
//    [128 (T w + t) + 32 q, +32), whose four words are its A operands of four MFMAs.
//    The B operand of lane (m, q) in the j-th of them is x[m] at the channels of word
//    j of that load, so the k order inside an MFMA is a permutation that pairs every
//    weight with its own activation.
//  * The 32 channels of one load lie in one group (group size >= 32), so one scale
//    and one zero point per lane and step build the binary16 weights (q - Z) * S with
//    one rounding, as in the large-M GEMM.  The scales and zero points of a row block
//    are staged once in an LDS slab, double buffered, by all threads of the workgroup.
//  * The W partial 16 x 16 tiles are summed in LDS in a fixed order and rounded once
//    to binary16.  Codes of the next row block are in flight while a block is computed.
//  * Rows longer than 16 wavefronts x 4 steps x 128 channels (K > 8192) are split into
//    ks slices over the workgroups: the workgroups of slice s hold the activations of
//    channels [s K / ks, (s + 1) K / ks) and write fp32 partial tiles, which a second
//    kernel adds in slice order and rounds once.
// Act order: the caller gathers x into the stored channel order first (gather_x_kernel,
// at most 32 rows), so the kernel always reads contiguous activations.
#pragma once

#include "nibbles.hpp"

namespace w4a16 {

// Entry of the scale / zero slab: binary16 S and -(1024 + Z) in .x, -(64 + Z) in .y.
__device__ __forceinline__ uint2 slab_entry(half_t s, uint32_t z) {
  const half_t a = static_cast<half_t>(-1024.0f - static_cast<float>(z));
  const half_t b = static_cast<half_t>(-64.0f - static_cast<float>(z));
  return uint2{static_cast<uint32_t>(__builtin_bit_cast(uint16_t, s)) |
                   (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) << 16),
               static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b))};
}

__device__ __forceinline__ DequantConsts slab_consts(uint2 e) {
  const half_t s = __builtin_bit_cast(half_t, static_cast<uint16_t>(e.x & 0xFFFFu));
  const half_t a = __builtin_bit_cast(half_t, static_cast<uint16_t>(e.x >> 16));
  const half_t b = __builtin_bit_cast(half_t, static_cast<uint16_t>(e.y & 0xFFFFu));
  DequantConsts c;
  c.neg_1024_z = half2_t{a, a};
  c.neg_64_z = half2_t{b, b};
  c.scale = half2_t{s, s};
  return c;
}

// LDS bytes of the kernel for W wavefronts and G groups per row.
constexpr size_t skinny_lds_bytes(int waves, int groups) {
  return 2 * static_cast<size_t>(waves) * 256 * sizeof(float) + 2 * static_cast<size_t>(16) * groups * sizeof(uint2);
}

// T: 128-channel steps per wavefront (K = 128 T W).  SE: slab entries (16 G per row
// block) loaded per thread, SE * 64 W >= 16 G.
// SUB (group size 128, one group per step): the weight operand is the raw codes as
// binary16 subnormals q * 2^-24 (one AND per pair, as in the decode GEMV), the
// activations in the pair slots that carry 16 q are pre-scaled by 1/16 (exact), each
// step's four MFMAs accumulate one group's sum of q x into a fresh tile, and the
// group's scale and zero point enter once per step:
//     acc += (S * 2^24) * sum q x + (-Z * S) * sum x.
// ks > 1: gridDim.x = ks * (workgroups per slice); partial sums go to part [ks][M][N]
// (fp32) instead of y.
// BITS = 8: 8-bit weights (four per word, byte order 0, 2, 1, 3); a lane's 32 channels
// of a step are 32 bytes (two loads), MFMA j takes words 2j and 2j + 1, SUB uses the
// bytes as subnormals with both pairs of a word at weight 1 (no activation pre-scale),
// and the zero points are bytes.
template <int T, int SE, bool SUB, int BITS = 4>
__global__ __launch_bounds__(1024) void gemm_skinny_kernel(
    const half_t* __restrict__ x, const uint32_t* __restrict__ qw, const half_t* __restrict__ scales,
    Zeros qzeros, half_t* __restrict__ y, float* __restrict__ part, int M, int N, int K,
    int gshift, int ks) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int nthreads = blockDim.x;
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit weights");
  constexpr int NQ = BITS / 4;            // 16-byte loads per lane and step
  constexpr int WSH = BITS == 4 ? 3 : 2;  // log2 channels per word
  const int lr = lane & 15, lq = lane >> 4;
  const int Wd = K >> WSH;
  const int gs = gridDim.x / ks;                  // workgroups per slice
  const int slice = blockIdx.x / gs;
  const int Ks = K / ks;                          // channels per slice
  const int g0 = (slice * Ks) >> gshift;                    // first group of the slice
  const int G = ((slice * Ks + Ks - 1) >> gshift) - g0 + 1;  // groups of the slice (slab rows)
  const int slab_n = 16 * G;
  const int nblk = (N + 15) >> 4;
  const int kw = slice * Ks + wave * 128 * T;

  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem);                                              // [2][W][16 m][16 n]
  uint2* slab = reinterpret_cast<uint2*>(smem + 2 * static_cast<size_t>(nwaves) * 256 * sizeof(float));  // [2][G][16]

  // Codes of row block b for this lane (rows past N re-read row N - 1), read through a
  // buffer resource over the codes (N K / 2 < 2^31 bytes, checked by the host): 32-bit
  // byte offsets instead of 64-bit addresses.
  const __amdgpu_buffer_rsrc_t codes = stream_rsrc(qw, static_cast<uint32_t>(N) * static_cast<uint32_t>(Wd) * 4u);
  constexpr uint32_t kStepBytes = 16u * BITS;   // 128 channels
  auto code_offset = [&](int b) {   // bytes; step t adds kStepBytes t
    const int n = min(16 * b + lr, N - 1);
    return (static_cast<uint32_t>(n) * static_cast<uint32_t>(Wd) + static_cast<uint32_t>((kw >> WSH) + 4 * NQ * lq)) * 4u;
  };
  auto load_codes = [&](int b, uint4 (&cw)[T][NQ]) {
    const uint32_t off = code_offset(b);
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int q = 0; q < NQ; ++q) cw[t][q] = load_buffer16(codes, off + kStepBytes * t + 16u * q);
  };
  // The first row block's codes are requested before anything else: they come from HBM,
  // the activations (read by every workgroup) mostly from the L2, so the long wait
  // starts first.  Same-process A/B on the 70B-class layer: M = 2 / 16 24.74 / 30.60 ->
  // 24.51 / 30.09 us, the 1-4B down-projection at M = 16 13.62 -> 13.15 us.
  // Row blocks b, b + gs, ... of this slice (neighbours on one XCD).
  int b = xcd_block(blockIdx.x - slice * gs, gs);
  uint4 cw[T][NQ];
  load_codes(b, cw);

  // Activation slice: xr[t][j] = x[m][kw + 128 t + 32 q + 8 j, +8) for m = lane % 16;
  // zero for m >= M.  SUB: xs[t] = sum of x[m] over step t's 128 channels, and the
  // elements 2, 3, 6, 7 of every fragment scaled by 1/16.
  half8_t xr[T][4];
  float xs[T];
  {
    const int m = lr < M ? lr : 0;
    const half_t* xm = x + static_cast<size_t>(m) * K;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t v = *reinterpret_cast<const half8_t*>(xm + kw + 128 * t + 32 * lq + 8 * j);
        xr[t][j] = lr < M ? v : half8_t{};
      }
    if constexpr (SUB) {
      const half2_t ones = half2_t{static_cast<half_t>(1.0f), static_cast<half_t>(1.0f)};
      constexpr bool kPrescale = BITS == 4;   // the 16 q pair slots of 4-bit words
      const half_t sixteenth = static_cast<half_t>(0.0625f);
#pragma unroll
      for (int t = 0; t < T; ++t) {
        float sx = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            sx = __builtin_amdgcn_fdot2(half2_t{xr[t][j][e], xr[t][j][e + 1]}, ones, sx, false);
        // the group spans the four lane quarters q (lanes r, r + 16, r + 32, r + 48)
        sx += __shfl_xor(sx, 16);
        sx += __shfl_xor(sx, 32);
        xs[t] = sx;
        if constexpr (kPrescale) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xr[t][j][2] *= sixteenth;
            xr[t][j][3] *= sixteenth;
            xr[t][j][6] *= sixteenth;
            xr[t][j][7] *= sixteenth;
          }
        }
      }
    }
  }

  // Scale and zero word of slab entries tid + u * nthreads of row block b.  SE >= 2
  // (many groups: group size 32 or 64 at large K) stages whole 8-row items instead: item
  // it = (group it / 2, rows 8 (it % 2) .. +8 of the block), its 8 scales one 16-byte load
  // and its 8 zero points one word (8-bit: two), at most one item per thread (2 G <= SE
  // nthreads / 8); the slab entries are the same.
  constexpr bool kItems = SE >= 2;
  half_t sv[kItems ? 1 : SE];
  uint32_t zv[kItems ? 1 : SE];
  uint4 iv_s;
  uint2 iv_z;
  const int items = 2 * G;
  auto item_n0 = [&](int b, int it) { return min(16 * b + 8 * (it & 1), N - 8); };   // N % 8 == 0
  auto load_sz = [&](int b) {
    if constexpr (kItems) {
      const int it = min(tid, items - 1);
      const int gi = g0 + (it >> 1);
      const int n0 = item_n0(b, it);
      iv_s = *reinterpret_cast<const uint4*>(scales + static_cast<size_t>(gi) * N + n0);
      if constexpr (BITS == 4)
        iv_z.x = *qzeros.at(static_cast<size_t>(gi) * (N >> 3) + (n0 >> 3));
      else
        iv_z = *reinterpret_cast<const uint2*>(qzeros.at(static_cast<size_t>(gi) * (N >> 2) + (n0 >> 2)));
      return;
    }
#pragma unroll
    for (int u = 0; u < SE; ++u) {
      const int e = min(tid + u * nthreads, slab_n - 1);
      const int gi = g0 + (e >> 4);
      const int n = min(16 * b + (e & 15), N - 1);
      sv[u] = scales[static_cast<size_t>(gi) * N + n];
      if constexpr (BITS == 4)
        zv[u] = *qzeros.at(static_cast<size_t>(gi) * (N >> 3) + (n >> 3));
      else
        zv[u] = *qzeros.at(static_cast<size_t>(gi) * (N >> 2) + (n >> 2));
    }
  };
  auto write_slab = [&](int b, int buf) {
    if constexpr (kItems) {
      if (tid < items) {
        const int gi = tid >> 1, r0 = 8 * (tid & 1);
        const uint32_t s8[4] = {iv_s.x, iv_s.y, iv_s.z, iv_s.w};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const half_t S = __builtin_bit_cast(half_t, static_cast<uint16_t>((s8[r >> 1] >> (16 * (r & 1))) & 0xFFFFu));
          uint32_t z;
          if constexpr (BITS == 4) {
            z = (qzeros.word(iv_z.x) >> (4 * r)) & 0xFu;
          } else {
            z = (qzeros.word8(r < 4 ? iv_z.x : iv_z.y) >> (8 * (r & 3))) & 0xFFu;
          }
          uint2* dst = slab + buf * slab_n + gi * 16 + r0 + r;
          if constexpr (SUB) {
            const float Sf = static_cast<float>(S);
            *dst = __builtin_bit_cast(uint2, make_float2(Sf * 16777216.0f, -static_cast<float>(z) * Sf));
          } else {
            *dst = slab_entry(S, z);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < SE; ++u) {
      const int e = tid + u * nthreads;
      if (e < slab_n) {
        const int n = min(16 * b + (e & 15), N - 1);
        const uint32_t z = BITS == 4 ? (qzeros.word(zv[u]) >> ((n & 7) * 4)) & 0xFu
                                     : (qzeros.word8(zv[u]) >> ((n & 3) * 8)) & 0xFFu;
        if constexpr (SUB) {
          const float S = static_cast<float>(sv[u]);
          slab[buf * slab_n + e] = __builtin_bit_cast(uint2, make_float2(S * 16777216.0f, -static_cast<float>(z) * S));
        } else {
          slab[buf * slab_n + e] = slab_entry(sv[u], z);
        }
      }
    }
  };

  // One row block: partial tile from this wavefront's slice; each step's code slot is
  // refilled with the next row block's codes as soon as it has been used, so a load
  // has a whole row block of work to land.  The slab of the next block is written and
  // its successor's scales issued; the partial tiles are summed after the barrier.
  auto row_block = [&](int b, int i) {
    const int buf = i & 1;
    const uint32_t off_next = code_offset(b + gs);
    float4_t acc = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T; ++t) {
      // this step's words: 4 (4-bit, one per MFMA) or 8 (8-bit, two per MFMA)
      uint32_t wv[4 * NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        wv[4 * q + 0] = cw[t][q].x;
        wv[4 * q + 1] = cw[t][q].y;
        wv[4 * q + 2] = cw[t][q].z;
        wv[4 * q + 3] = cw[t][q].w;
      }
      auto refill = [&]() {
#pragma unroll
        for (int q = 0; q < NQ; ++q) cw[t][q] = load_buffer16(codes, off_next + kStepBytes * t + 16u * q);
      };
      if constexpr (SUB) {
        half8_t wf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (BITS == 4) {
            const SubPairs sp = expand_word_subnormal(wv[j]);
            wf[j] = __builtin_bit_cast(half8_t, uint4{sp.a0, sp.b0, sp.a1, sp.b1});
          } else {
            const uint32_t lo = wv[2 * j], hi = wv[2 * j + 1];
            wf[j] = __builtin_bit_cast(half8_t, uint4{lo & 0x00FF00FFu, (lo >> 8) & 0x00FF00FFu,
                                                      hi & 0x00FF00FFu, (hi >> 8) & 0x00FF00FFu});
          }
        }
        refill();
        float4_t part = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) part = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[j], xr[t][j], part, 0, 0, 0);
        // rows n = 4 q + r of the tile hold this lane's four results; their group's
        // (S * 2^24, -Z * S) are four consecutive slab entries
        const int gi = ((kw + 128 * t) >> 7) - g0;
        const float4* e4 = reinterpret_cast<const float4*>(slab + buf * slab_n + gi * 16 + 4 * lq);
        const float4 e01 = e4[0], e23 = e4[1];
        acc[0] = fmaf(e01.y, xs[t], fmaf(e01.x, part[0], acc[0]));
        acc[1] = fmaf(e01.w, xs[t], fmaf(e01.z, part[1], acc[1]));
        acc[2] = fmaf(e23.y, xs[t], fmaf(e23.x, part[2], acc[2]));
        acc[3] = fmaf(e23.w, xs[t], fmaf(e23.z, part[3], acc[3]));
      } else {
        const int gi = ((kw + 128 * t + 32 * lq) >> gshift) - g0;
        const DequantConsts dc = slab_consts(slab[buf * slab_n + gi * 16 + lr]);
        half8_t wf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (BITS == 4) {
            wf[j] = dequant_word(wv[j], dc);
          } else {
            const half4_t lo = dequant_word8(wv[2 * j], dc), hi = dequant_word8(wv[2 * j + 1], dc);
            wf[j] = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        }
        refill();
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(wf[j], xr[t][j], acc, 0, 0, 0);
      }
    }
    // D layout: lane (r, q) holds rows n = 4 q + 0..3 of column m = r.
    *reinterpret_cast<float4_t*>(red + ((buf * nwaves + wave) * 16 + lr) * 16 + 4 * lq) = acc;
    write_slab(b + gs, buf ^ 1);
    load_sz(b + 2 * gs);
    __syncthreads();
    if (tid < 256) {
      const int m = tid >> 4, n = 16 * b + (tid & 15);
      if (m < M && n < N) {
        const float* p = red + buf * nwaves * 256 + tid;
        float s = 0.f;
        for (int w = 0; w < nwaves; ++w) s += p[w * 256];
        if (ks == 1) y[static_cast<size_t>(m) * N + n] = static_cast<half_t>(s);
        else part[(static_cast<size_t>(slice) * M + m) * N + n] = s;
      }
    }
  };

  load_sz(b);
  write_slab(b, 0);
  load_sz(b + gs);
  __syncthreads();
  for (int i = 0; b < nblk; ++i, b += gs) row_block(b, i);
}

}  // namespace w4a16
