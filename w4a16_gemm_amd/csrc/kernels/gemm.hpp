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

#include <type_traits>

#include "nibbles.hpp"

namespace w4a16 {

// BITS = 8: 8-bit weights (four per word, byte order 0, 2, 1, 3); a lane's 32 channels
// are 32 bytes, and the s-th MFMA of the tile takes its words 2s and 2s + 1.
// BITS = 16: dense binary16 weights [N][K] (scales and zero points unused): the
// reference product of the AWQ search.
template <int BM, int BITS = 4>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(
    const half_t* __restrict__ x, const uint32_t* __restrict__ qw, const half_t* __restrict__ scales,
    Zeros qzeros, half_t* __restrict__ y, int M, int N, int K, int gshift) {
  static_assert(BM % 16 == 0 && BM >= 16, "BM must be a multiple of 16");
  static_assert(BITS == 4 || BITS == 8 || BITS == 16, "4-, 8- or 16-bit weights");
  constexpr int NQ = BITS / 4;                    // 16-byte pieces of a lane's 32 channels
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
  constexpr int WSH = BITS == 4 ? 3 : BITS == 8 ? 2 : 1;   // log2 channels per word
  const int W = K >> WSH;                         // words per row
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

  uint4 bw[4][NQ];
  half_t bs[4];
  uint32_t bz[4];
  auto load_b = [&](int t) {
    const int k = t * 128 + lq * 32;
    const bool kin = k < K;
    const int gi = kin ? (k >> gshift) : 0;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = min(nw + 16 * nb + lr, N - 1);
      const uint4* src = reinterpret_cast<const uint4*>(qw + static_cast<size_t>(n) * W + (k >> WSH));
#pragma unroll
      for (int q = 0; q < NQ; ++q) bw[nb][q] = kin ? src[q] : uint4{0, 0, 0, 0};
      if constexpr (BITS != 16) {
        bs[nb] = scales[static_cast<size_t>(gi) * N + n];
        bz[nb] = load_zero<BITS>(qzeros, gi, N, n);
      }
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
    uint4 cw[4][NQ];
    DequantConsts dc[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) cw[nb][q] = bw[nb][q];
      if constexpr (BITS != 16) dc[nb] = make_consts(bz[nb], bs[nb]);
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
        if constexpr (BITS == 16) {
          bf[nb] = __builtin_bit_cast(half8_t, cw[nb][s]);
        } else if constexpr (BITS == 4) {
          const uint4 c = cw[nb][0];
          const uint32_t word = s == 0 ? c.x : s == 1 ? c.y : s == 2 ? c.z : c.w;
          bf[nb] = dequant_word(word, dc[nb]);
        } else {
          const uint4 c = cw[nb][s >> 1];
          const half4_t lo = dequant_word8((s & 1) ? c.z : c.x, dc[nb]);
          const half4_t hi = dequant_word8((s & 1) ? c.w : c.y, dc[nb]);
          bf[nb] = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
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

// Large-M tile: a workgroup of 8 wavefronts (2 along M x 4 along N, two per SIMD)
// computes a 256 x 256 tile of y; wavefront (wm, wn) owns rows [128 wm, +128) and
// columns [64 wn, +64) with 8 x 4 blocks of 16x16 fp32 accumulators.
//  * K advances in tiles of 64 channels.  Lane (r, q) = (lane % 16, lane / 16) of a
//    wavefront holds, per 16-column block, the 16 codes of channels [16 q, 16 q + 16)
//    of its column: word s (8 codes) is its B operand of the tile's MFMA step s, and
//    its A operand in that step is the 8 activations of the same channels.
//  * Everything a tile needs goes through a 3-stage LDS ring filled with direct-to-LDS
//    loads two tiles ahead: the activation tile (256 rows x 64 channels, 32 KB), the
//    raw packed codes (256 columns x 64 channels, 8 KB) and the scales and packed zero
//    points of the groups of its two 32-channel halves (1.25 KB).  No registers hold
//    prefetched data, so two wavefronts per SIMD fit in 256 registers each.
//  * An activation row is 8 slots of 16 bytes; slot j of row r holds the row's chunk
//    j ^ (r % 8), which spreads the 16 rows of an MFMA operand over the LDS banks (the
//    reads still meet two-way bank conflicts; a conflict-free arrangement measured no
//    faster).
//  * Each wavefront dequantises its 64 columns in registers (the two wavefronts
//    sharing columns both do it).
//  * Tiles are dealt out per XCD (dispatch is round-robin over the 8 XCDs): when the
//    tile grid allows, XCD x takes a block of half the row panels by a quarter of the
//    column tiles (2 x 4 blocks over the grid), so that the x panels and code columns
//    one K step of its workgroups touches are as few as possible and stay in that
//    XCD's L2; otherwise consecutive tiles in row-panel order.
// Requirements: K % 64 == 0, group size >= 32 and M * K < 2^31.
__device__ __forceinline__ int xcd_tile(int bid, int tiles_m, int tiles_n) {
  const int ntiles = tiles_m * tiles_n;
  if (ntiles % 8 != 0) return bid;
  const int x = bid % 8, j = bid / 8;
  if (tiles_m % 2 != 0 || tiles_n % 4 != 0) return x * (ntiles / 8) + j;
  const int pa = tiles_m / 2, pb = tiles_n / 4;   // row panels and column tiles per XCD
  return (pa * (x % 2) + j / pb) * tiles_n + pb * (x / 2) + j % pb;
}

// LDS reads written as inline asm.  The compiler cannot tell which stage of the ring
// a direct-to-LDS load writes, so before every LDS read it would wait for all
// outstanding global loads, including the prefetch of later tiles; reads it does not
// see as LDS accesses are ordered by the explicit waits and barriers of the kernel
// instead.  Each block waits for its own results before it returns.
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));   // low half of a flat LDS address
}

// af[mb] = 16 bytes at addr + 2048 mb, mb = 0..7.
__device__ __forceinline__ void lds_read_a8(uint32_t addr, half8_t (&af)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8\n"
      "ds_read_b128 %1, %8 offset:2048\n"
      "ds_read_b128 %2, %8 offset:4096\n"
      "ds_read_b128 %3, %8 offset:6144\n"
      "ds_read_b128 %4, %8 offset:8192\n"
      "ds_read_b128 %5, %8 offset:10240\n"
      "ds_read_b128 %6, %8 offset:12288\n"
      "ds_read_b128 %7, %8 offset:14336\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]), "=&v"(af[6]),
        "=&v"(af[7])
      : "v"(addr)
      : "memory");
}

// The eight A fragments of lds_read_a8, plus for nb < NB: cw[nb] = 8 bytes at
// b_addr + 256 nb, the 16-bit sc[nb] at s_addr + 32 nb and the 32-bit zw[nb] at
// z_addr + 8 nb.  One asm statement per NB, waiting for all of its results.
template <int NB>
__device__ __forceinline__ void lds_read_tile(uint32_t a_addr, uint32_t b_addr, uint32_t s_addr, uint32_t z_addr,
                                              half8_t (&af)[8], uint2 (&cw)[NB], uint32_t (&sc)[NB],
                                              uint32_t (&zw)[NB]);
template <>
__device__ __forceinline__ void lds_read_tile<1>(uint32_t a_addr, uint32_t b_addr, uint32_t s_addr, uint32_t z_addr,
                                                 half8_t (&af)[8], uint2 (&cw)[1], uint32_t (&sc)[1],
                                                 uint32_t (&zw)[1]) {
  asm volatile(
      "ds_read_u16 %9, %13\n"
      "ds_read_b32 %10, %14\n"
      "ds_read_b64 %8, %12\n"
      "ds_read_b128 %0, %11\n"
      "ds_read_b128 %1, %11 offset:2048\n"
      "ds_read_b128 %2, %11 offset:4096\n"
      "ds_read_b128 %3, %11 offset:6144\n"
      "ds_read_b128 %4, %11 offset:8192\n"
      "ds_read_b128 %5, %11 offset:10240\n"
      "ds_read_b128 %6, %11 offset:12288\n"
      "ds_read_b128 %7, %11 offset:14336\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]), "=&v"(af[6]),
        "=&v"(af[7]), "=&v"(cw[0]), "=&v"(sc[0]), "=&v"(zw[0])
      : "v"(a_addr), "v"(b_addr), "v"(s_addr), "v"(z_addr)
      : "memory");
}

template <>
__device__ __forceinline__ void lds_read_tile<2>(uint32_t a_addr, uint32_t b_addr, uint32_t s_addr, uint32_t z_addr,
                                                 half8_t (&af)[8], uint2 (&cw)[2], uint32_t (&sc)[2],
                                                 uint32_t (&zw)[2]) {
  asm volatile(
      "ds_read_u16 %10, %16\n"
      "ds_read_u16 %11, %16 offset:32\n"
      "ds_read_b32 %12, %17\n"
      "ds_read_b32 %13, %17 offset:8\n"
      "ds_read_b64 %8, %15\n"
      "ds_read_b64 %9, %15 offset:256\n"
      "ds_read_b128 %0, %14\n"
      "ds_read_b128 %1, %14 offset:2048\n"
      "ds_read_b128 %2, %14 offset:4096\n"
      "ds_read_b128 %3, %14 offset:6144\n"
      "ds_read_b128 %4, %14 offset:8192\n"
      "ds_read_b128 %5, %14 offset:10240\n"
      "ds_read_b128 %6, %14 offset:12288\n"
      "ds_read_b128 %7, %14 offset:14336\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]), "=&v"(af[6]), "=&v"(af[7]), "=&v"(cw[0]), "=&v"(cw[1]), "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(zw[0]), "=&v"(zw[1])
      : "v"(a_addr), "v"(b_addr), "v"(s_addr), "v"(z_addr)
      : "memory");
}

template <>
__device__ __forceinline__ void lds_read_tile<3>(uint32_t a_addr, uint32_t b_addr, uint32_t s_addr, uint32_t z_addr,
                                                 half8_t (&af)[8], uint2 (&cw)[3], uint32_t (&sc)[3],
                                                 uint32_t (&zw)[3]) {
  asm volatile(
      "ds_read_u16 %11, %19\n"
      "ds_read_u16 %12, %19 offset:32\n"
      "ds_read_u16 %13, %19 offset:64\n"
      "ds_read_b32 %14, %20\n"
      "ds_read_b32 %15, %20 offset:8\n"
      "ds_read_b32 %16, %20 offset:16\n"
      "ds_read_b64 %8, %18\n"
      "ds_read_b64 %9, %18 offset:256\n"
      "ds_read_b64 %10, %18 offset:512\n"
      "ds_read_b128 %0, %17\n"
      "ds_read_b128 %1, %17 offset:2048\n"
      "ds_read_b128 %2, %17 offset:4096\n"
      "ds_read_b128 %3, %17 offset:6144\n"
      "ds_read_b128 %4, %17 offset:8192\n"
      "ds_read_b128 %5, %17 offset:10240\n"
      "ds_read_b128 %6, %17 offset:12288\n"
      "ds_read_b128 %7, %17 offset:14336\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]), "=&v"(af[6]), "=&v"(af[7]), "=&v"(cw[0]), "=&v"(cw[1]), "=&v"(cw[2]), "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(zw[0]), "=&v"(zw[1]), "=&v"(zw[2])
      : "v"(a_addr), "v"(b_addr), "v"(s_addr), "v"(z_addr)
      : "memory");
}

template <>
__device__ __forceinline__ void lds_read_tile<4>(uint32_t a_addr, uint32_t b_addr, uint32_t s_addr, uint32_t z_addr,
                                                 half8_t (&af)[8], uint2 (&cw)[4], uint32_t (&sc)[4],
                                                 uint32_t (&zw)[4]) {
  asm volatile(
      "ds_read_u16 %12, %22\n"
      "ds_read_u16 %13, %22 offset:32\n"
      "ds_read_u16 %14, %22 offset:64\n"
      "ds_read_u16 %15, %22 offset:96\n"
      "ds_read_b32 %16, %23\n"
      "ds_read_b32 %17, %23 offset:8\n"
      "ds_read_b32 %18, %23 offset:16\n"
      "ds_read_b32 %19, %23 offset:24\n"
      "ds_read_b64 %8, %21\n"
      "ds_read_b64 %9, %21 offset:256\n"
      "ds_read_b64 %10, %21 offset:512\n"
      "ds_read_b64 %11, %21 offset:768\n"
      "ds_read_b128 %0, %20\n"
      "ds_read_b128 %1, %20 offset:2048\n"
      "ds_read_b128 %2, %20 offset:4096\n"
      "ds_read_b128 %3, %20 offset:6144\n"
      "ds_read_b128 %4, %20 offset:8192\n"
      "ds_read_b128 %5, %20 offset:10240\n"
      "ds_read_b128 %6, %20 offset:12288\n"
      "ds_read_b128 %7, %20 offset:14336\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(af[0]), "=&v"(af[1]), "=&v"(af[2]), "=&v"(af[3]), "=&v"(af[4]), "=&v"(af[5]), "=&v"(af[6]), "=&v"(af[7]), "=&v"(cw[0]), "=&v"(cw[1]), "=&v"(cw[2]), "=&v"(cw[3]), "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(sc[3]), "=&v"(zw[0]), "=&v"(zw[1]), "=&v"(zw[2]), "=&v"(zw[3])
      : "v"(a_addr), "v"(b_addr), "v"(s_addr), "v"(z_addr)
      : "memory");
}

// An LDS pointer in the LDS address space (the destination operand of the buffer loads
// that write straight into LDS).
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t as_lds(void* p) { return (lds_ptr_t)(p); }

// Workgroup barrier without the memory fence of __syncthreads(), whose release would
// wait for every outstanding load, prefetches included.  Callers wait for exactly the
// loads and LDS reads that must be complete (s_waitcnt) before they call it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int kBigBM = 256, kBigBN = 256, kBigBK = 64, kBigStages = 3;
constexpr uint32_t kBigLdsA = kBigBM * kBigBK * 2;      // activations of one stage
constexpr uint32_t kBigLdsB = kBigBN * kBigBK / 2;      // packed codes of one stage
constexpr uint32_t kBigLdsS = 2 * kBigBN * 2;           // scales [half][column]
constexpr uint32_t kBigLdsZ = 2 * (kBigBN / 8) * 4;     // packed zero points [half][column / 8]
constexpr uint32_t kBigStage = kBigLdsA + kBigLdsB + kBigLdsS + kBigLdsZ;
constexpr size_t kBigLds = static_cast<size_t>(kBigStages) * kBigStage;

// 8-bit codes: twice the code bytes ([quarter of 16 channels][column] x 16 B) and the
// zero-point bytes of each half as one 16-byte load per lane ([half] x 512 B, byte
// `column` of a half at offset column).
constexpr uint32_t kBigLdsB8 = kBigBN * kBigBK;
constexpr uint32_t kBigLdsZ8 = 2 * 512;
constexpr uint32_t kBigStage8 = kBigLdsA + kBigLdsB8 + kBigLdsS + kBigLdsZ8;
constexpr size_t kBigLds8 = static_cast<size_t>(kBigStages) * kBigStage8;

template <int BITS>
constexpr uint32_t big_stage_bytes() { return BITS == 4 ? kBigStage : kBigStage8; }

// Direct-to-LDS loads of one K tile of a BM x BN output tile (BM = 32 MB, BN = 64 NB)
// into a stage of the LDS ring, laid out as for the widest tile (256 x 256) whatever
// the tile is.  N is the row pitch of scales, zero points and y; columns at or past
// n_end are not loaded.  BITS = 8: 8-bit codes (byte order 0, 2, 1, 3), two code loads
// per thread and stage (chunk c = tid + 512 i holds channels [16 (c / BL), +16) of
// column c % BL) and the zero-point bytes of each half as one 16-byte load per lane;
// needs N % 16 == 0.
template <int NB, int MB, int BITS>
struct BigLoader {
  static constexpr int BM = 32 * MB, BN = 64 * NB, BL = kBigBN, BK = kBigBK, NS = kBigStages;
  static constexpr int APT = BM * BK / 8 / 512;   // activation chunks (16 B) per thread per stage
  static constexpr int CL = BITS / 4;             // code loads (16 B) per thread per stage
  static constexpr uint32_t STAGE = big_stage_bytes<BITS>();
  static constexpr uint32_t LB = BITS == 4 ? kBigLdsB : kBigLdsB8;
  static_assert(NB >= 1 && NB <= 4, "tile width");
  static_assert(MB == 2 || MB == 4 || MB == 8, "tile height");
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit weights");
  static_assert(BL * BK / 32 == 512, "one 4-bit code chunk per thread per stage (of the widest tile)");
  static_assert(STAGE % 16 == 0, "stage alignment");

  // The activation and code streams are raw buffer loads into LDS: a buffer resource
  // over the tile's rows (x from row m0, the codes from column n0), a 32-bit byte offset
  // of the lane that does not change over the K loop (at most 256 rows or columns of one
  // row pitch) and the K tile's offset as the scalar offset, so the loop does no vector
  // address arithmetic.
  __amdgpu_buffer_rsrc_t xr;   // x from row m0
  __amdgpu_buffer_rsrc_t qr;   // codes from column n0
  const half_t* scales;
  Zeros qzeros;
  unsigned char* smem;
  int N, KT, gshift, wave, sz_half, s_col, z_word;
  uint32_t a_off[APT];
  uint32_t b_off[CL];

  __device__ __forceinline__ BigLoader(const half_t* x_, const uint32_t* qw_, const half_t* scales_, Zeros qz,
                                       unsigned char* smem_, int M, int N_, int K, int gshift_, int m0, int n0,
                                       int n_end, int tid, int wave_)
      : scales(scales_), qzeros(qz), smem(smem_), N(N_), KT(K / BK), gshift(gshift_), wave(wave_) {
    const int lane = tid & 63;
    const int W = K >> (BITS == 4 ? 3 : 2);   // words per row
    // sizes: (M - m0) rows of x (M K < 2^31 elements), the codes of columns n0.. n_end
    // (clamped to the 32-bit range; every offset used lies inside it)
    xr = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(x_ + static_cast<size_t>(m0) * K), 0,
                                           static_cast<int>(static_cast<uint32_t>(M - m0) * K * 2u), kBufferWord3);
    const unsigned long long qbytes = static_cast<unsigned long long>(n_end - n0) * W * 4ull;
    qr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw_ + static_cast<size_t>(n0) * W), 0,
                                           static_cast<int>(qbytes > 0xFFFFFFFFull ? 0xFFFFFFFFu
                                                                                   : static_cast<uint32_t>(qbytes)),
                                           kBufferWord3);
    // Activations: lane l of load i writes chunk c = (APT wave + i) * 64 + l = 8 row + slot,
    // which receives the row's chunk slot ^ (row % 8).  Rows past M re-read row M - 1.
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int c = (wave * APT + i) * 64 + lane;
      const int row = c >> 3, slot = c & 7;
      a_off[i] = static_cast<uint32_t>(min(row, M - 1 - m0) * K + 8 * (slot ^ (row & 7))) * 2u;
    }
    // Codes: chunk c = half * BL + column holds channels [32 half, +32) of the column;
    // columns past the tile (BN < BL) or past N re-read a column of the tile.
#pragma unroll
    for (int i = 0; i < CL; ++i) {
      const int c = tid + 512 * i;
      b_off[i] = static_cast<uint32_t>(min(min(c % BL, BN - 1), n_end - 1 - n0) * W + 4 * (c / BL)) * 4u;
    }
    // Scales (wavefront 0, 16 B per lane) and zero points (wavefront 1, 4 B per lane) of
    // half h = lane / 32: 8 columns, resp. one packed word of 8 columns, per lane.
    sz_half = lane >> 5;
    s_col = min(n0 + 8 * (lane & 31), n_end - 8);
    z_word = BITS == 4 ? min(n0 / 8 + (lane & 31), n_end / 8 - 1)
                       : min(n0 / 4 + 4 * (lane & 31), n_end / 4 - 4);   // 8-bit: 16 columns per lane
  }

  // Tile t goes to stage t % NS; tiles past the end re-load the last one into a stage
  // that is never read again.  The scale / zero load comes first, so that waiting for
  // tile t alone never waits for more than that load of tile t + 1.
  __device__ __forceinline__ void load(int t) const {
    unsigned char* stage = smem + (t % NS) * STAGE;
    load_sz_to(t, stage + kBigLdsA);
    load_a_to(t, stage);
    load_codes_to(t, stage + kBigLdsA);
  }
  // The parts of a tile's loads, to separate buffers: the scales and zero points of its
  // two 32-channel halves (to c + LB, c + LB + kBigLdsS), the activations (to a) and the
  // codes (to c); tiles past the end re-load the last one.
  __device__ __forceinline__ void load_sz_to(int t, unsigned char* c) const {
    const int tc = min(t, KT - 1);
    const int gi = (tc * BK + 32 * sz_half) >> gshift;
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(
          reinterpret_cast<const void*>(scales + static_cast<size_t>(gi) * N + s_col),
          reinterpret_cast<void*>(c + LB), 16, 0, 0);
    else if (wave == 1) {
      if constexpr (BITS == 4)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(qzeros.at(static_cast<size_t>(gi) * (N >> 3) + z_word)),
            reinterpret_cast<void*>(c + LB + kBigLdsS), 4, 0, 0);
      else
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void*>(qzeros.at(static_cast<size_t>(gi) * (N >> 2) + z_word)),
            reinterpret_cast<void*>(c + LB + kBigLdsS), 16, 0, 0);
    }
  }
  __device__ __forceinline__ void load_a_to(int t, unsigned char* a) const {
    const int tc = min(t, KT - 1);
#pragma unroll
    for (int i = 0; i < APT; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, as_lds(a + (wave * APT + i) * 64 * 16), 16,
          static_cast<int>(a_off[i]), tc * (BK * 2), 0, 0);
  }
  __device__ __forceinline__ void load_codes_to(int t, unsigned char* c) const {
    const int tc = min(t, KT - 1);
#pragma unroll
    for (int i = 0; i < CL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          qr, as_lds(c + (512 * i + wave * 64) * 16),
          16, static_cast<int>(b_off[i]), tc * (BK * BITS / 8), 0, 0);
  }
};

// 16x16x32 MFMA tile.  Lane (r, q) = (lane % 16, lane / 16) of a wavefront holds, per
// 16-column block, the 16 codes of channels [16 q, 16 q + 16) of its column.  BITS = 8:
// lane (r, q) reads the 16 bytes of channels [16 q, +16) of its column, MFMA step s
// takes words 2s and 2s + 1; zero points are bytes; LDS read with plain loads at every
// tile height.
template <int NB, int MB, int BITS = 4>
__device__ __forceinline__ void big_tile(const half_t* __restrict__ x, const uint32_t* __restrict__ qw,
                                         const half_t* __restrict__ scales, Zeros qzeros,
                                         half_t* __restrict__ y, int M, int N, int K, int gshift, int m0, int n0,
                                         int n_end, int prio) {
  // NB 16-column blocks and MB 16-row blocks per wavefront: the tile is BM x BN with
  // BM = 32 MB and BN = 64 NB.  MB = 8 reads LDS through the inline-asm blocks above;
  // the smaller tiles (few-row batches) use plain loads, which the compiler orders
  // against the barriers and (seeing no alias with the direct-to-LDS writes) does not
  // hold behind the prefetches.
  using Loader = BigLoader<NB, MB, BITS>;
  constexpr int BL = Loader::BL, NS = Loader::NS, APT = Loader::APT, CL = Loader::CL;
  constexpr uint32_t STAGE = Loader::STAGE, LB = Loader::LB;
  constexpr bool kAsmReads = MB == 8 && BITS == 4;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int KT = K / kBigBK;
  const Loader ld(x, qw, scales, qzeros, smem, M, N, K, gshift, m0, n0, n_end, tid, wave);
  auto load_tile = [&](int t) { ld.load(t); };

  float4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // This lane's LDS byte addresses in stage 0: A fragment mb of MFMA step s at
  // a_lane + 16 ((2 q + s) ^ (r % 8)) + 2048 mb; code words of block nb at b_lane +
  // 256 nb; scale of block nb at s_lane + 32 nb; zero word of block nb at z_lane + 8 nb.
  const uint32_t base = lds_offset(smem);
  const uint32_t a_lane = base + (wm * 16 * MB + lr) * 128;
  const uint32_t b_lane = BITS == 4 ? base + kBigLdsA + ((lq >> 1) * BL + wn * 16 * NB + lr) * 16 + (lq & 1) * 8
                                    : base + kBigLdsA + (lq * BL + wn * 16 * NB + lr) * 16;
  const uint32_t s_lane = base + kBigLdsA + LB + ((lq >> 1) * BL + wn * 16 * NB + lr) * 2;
  const uint32_t z_lane =
      BITS == 4 ? base + kBigLdsA + LB + kBigLdsS + ((lq >> 1) * (BL / 8) + wn * 2 * NB + (lr >> 3)) * 4
                : base + kBigLdsA + LB + kBigLdsS + (lq >> 1) * 512 + wn * 16 * NB + lr;   // a byte
  const int z_shift = 4 * (lr & 7);

  // At most APT + CL loads of this wavefront (its activation and code loads of tile
  // t + 1) are newer than the last load of tile t once tile t + 1 has been issued.
  load_tile(0);
  load_tile(1);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(APT + CL) : "memory");   // tile 0
  block_barrier();

  // Scale and zero-point constants of this lane's columns, rebuilt only when the K tile
  // starts a new group (every tile at group 32 or 64, every other one at 128, once for
  // one group per row).
  DequantConsts dc[NB];
  const int gmask = (1 << min(gshift, 30)) - 1;
  for (int t = 0; t < KT; ++t) {
    load_tile(t + NS - 1);
    const uint32_t so = (t % NS) * STAGE;
    half8_t af[MB];
    using CodeWords = std::conditional_t<BITS == 4, uint2, uint4>;
    CodeWords cw[NB];
    uint32_t sc[NB], zw[NB];
    const unsigned char* st = smem + so;   // plain-load view of the same stage
    if constexpr (kAsmReads) {
      lds_read_tile<NB>(a_lane + so + 16 * ((2 * lq) ^ (lr & 7)), b_lane + so, s_lane + so, z_lane + so, af, cw, sc,
                        zw);
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        cw[nb] = *reinterpret_cast<const CodeWords*>(st + (b_lane - base) + 256 * nb);
        sc[nb] = *reinterpret_cast<const uint16_t*>(st + (s_lane - base) + 32 * nb);
        if constexpr (BITS == 4)
          zw[nb] = *reinterpret_cast<const uint32_t*>(st + (z_lane - base) + 8 * nb);
        else
          zw[nb] = *(st + (z_lane - base) + 16 * nb);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        af[mb] = *reinterpret_cast<const half8_t*>(st + (a_lane - base) + 16 * ((2 * lq) ^ (lr & 7)) + 2048 * mb);
    }
    if (((t * kBigBK) & gmask) == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        dc[nb] = make_consts(BITS == 4 ? (qzeros.word(zw[nb]) >> z_shift) & 0xFu : (qzeros.sym ? 128u : zw[nb]),
                             __builtin_bit_cast(half_t, static_cast<uint16_t>(sc[nb])));
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s == 1) {
        if constexpr (kAsmReads) {
          lds_read_a8(a_lane + so + 16 * ((2 * lq + 1) ^ (lr & 7)), af);
        } else {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            af[mb] = *reinterpret_cast<const half8_t*>(st + (a_lane - base) + 16 * ((2 * lq + 1) ^ (lr & 7)) +
                                                       2048 * mb);
        }
      }
      half8_t bf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (BITS == 4) {
          bf[nb] = dequant_word(s == 0 ? cw[nb].x : cw[nb].y, dc[nb]);
        } else {
          const half4_t lo = dequant_word8(s == 0 ? cw[nb].x : cw[nb].z, dc[nb]);
          const half4_t hi = dequant_word8(s == 0 ? cw[nb].y : cw[nb].w, dc[nb]);
          bf[nb] = half8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      if (prio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
      if (prio) __builtin_amdgcn_s_setprio(0);
    }
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(APT + CL) : "memory");   // tile t + 1; own LDS reads done
    block_barrier();
  }
  // the clamped loads past the last tile must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // D layout of the 16x16 MFMA: lane l holds rows 4*(l/16) + r, column l % 16.
  const int nw = n0 + wn * 16 * NB;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = nw + 16 * nb + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 16 * MB + 16 * mb + 4 * lq + r;
        if (m < M && n < n_end) y[static_cast<size_t>(m) * N + n] = static_cast<half_t>(acc[mb][nb][r]);
      }
    }
}

// 32x32x16 MFMA tile (4-bit weights): the same LDS ring and loads as big_tile, with
// 32 x 32 output blocks (MB / 2 row blocks by NB / 2 column blocks per wavefront).  The
// 32x32x16 instruction does twice the work of the 16x16x32 one per issue from the same
// operand registers, and on this part more of the dequantisation's VALU work overlaps
// with it: a probe of independent MFMA chains with two wavefronts per SIMD ran 2.06
// PFLOP/s with two VALU instructions per 16K flops of 32x32x16 MFMAs, 1.71 PFLOP/s
// with 16x16x32 MFMAs.
//  * Lane l = 32 h + c of a wavefront stands for row (A) / column (B) c of a block.
//    Its 8 channels of MFMA step s (s = 0..3 over the 64-channel K tile) are the
//    channels [32 h + 8 s, +8): the contraction pairs each activation with the weight
//    of the same channel, in any assignment of channels to steps, and this one makes
//    a lane's four B words the contiguous 16-byte code chunk (half h, column) of the
//    stage, the scale and zero point of one group (group size >= 32).
//  * The A fragment of step s is chunk 4 h + s of its row, at slot (4 h + s) ^ (row % 8).
//  * D layout of the 32x32 MFMA: lane l holds column l % 32 and, in register r, row
//    8 (r / 4) + 4 (l / 32) + r % 4.
template <int NB, int MB>
__device__ __forceinline__ void big_tile32(const half_t* __restrict__ x, const uint32_t* __restrict__ qw,
                                           const half_t* __restrict__ scales, Zeros qzeros,
                                           half_t* __restrict__ y, int M, int N, int K, int gshift, int m0, int n0,
                                           int n_end, int prio) {
  using Loader = BigLoader<NB, MB, 4>;
  constexpr int BL = Loader::BL, NS = Loader::NS, APT = Loader::APT, CL = Loader::CL;
  constexpr uint32_t STAGE = Loader::STAGE, LB = Loader::LB;
  static_assert(NB % 2 == 0, "whole 32-column blocks per wavefront");
  constexpr int RB = MB / 2, CB = NB / 2;   // 32-row and 32-column blocks per wavefront
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lc = lane & 31;
  const int lh = lane >> 5;
  const int KT = K / kBigBK;
  const Loader ld(x, qw, scales, qzeros, smem, M, N, K, gshift, m0, n0, n_end, tid, wave);

  f32x16_t acc[RB][CB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;

  // Byte offsets inside a stage: A fragment rb of step s at a_lane + 4096 rb + 16 ((4 h +
  // s) ^ (c % 8)); code chunk of block cb at b_lane + 512 cb; its scale at s_lane + 64 cb
  // and zero word at z_lane + 16 cb.
  const int col = wn * 16 * NB + lc;   // column of block 0 inside the tile
  const uint32_t a_lane = (wm * 16 * MB + lc) * 128;
  const uint32_t b_lane = kBigLdsA + (lh * BL + col) * 16;
  const uint32_t s_lane = kBigLdsA + LB + (lh * BL + col) * 2;
  const uint32_t z_lane = kBigLdsA + LB + kBigLdsS + (lh * (BL / 8) + (col >> 3)) * 4;
  const int z_shift = 4 * (lc & 7);

  // At most APT + CL loads of this wavefront (its activation and code loads of tile
  // t + 1) are newer than the last load of tile t once tile t + 1 has been issued.
  ld.load(0);
  ld.load(1);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(APT + CL) : "memory");   // tile 0
  block_barrier();

  // constants rebuilt only when the K tile starts a new group (as in big_tile)
  DequantConsts dc[CB];
  const int gmask = (1 << min(gshift, 30)) - 1;
  for (int t = 0; t < KT; ++t) {
    ld.load(t + NS - 1);
    const unsigned char* st = smem + (t % NS) * STAGE;
    uint4 cw[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) cw[cb] = *reinterpret_cast<const uint4*>(st + b_lane + 512 * cb);
    if (((t * kBigBK) & gmask) == 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(st + s_lane + 64 * cb);
        const uint32_t zw = *reinterpret_cast<const uint32_t*>(st + z_lane + 16 * cb);
        dc[cb] = make_consts((qzeros.word(zw) >> z_shift) & 0xFu, __builtin_bit_cast(half_t, static_cast<uint16_t>(sc)));
      }
    }
    // A fragments one step ahead: the reads of step s + 1 are in flight during the
    // MFMAs of step s.
    half8_t af[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      af[0][rb] = *reinterpret_cast<const half8_t*>(st + a_lane + 4096 * rb + 16 * ((4 * lh) ^ (lc & 7)));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          af[(s + 1) & 1][rb] =
              *reinterpret_cast<const half8_t*>(st + a_lane + 4096 * rb + 16 * ((4 * lh + s + 1) ^ (lc & 7)));
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of this step's MFMAs
      half8_t bf[CB];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
        bf[cb] = dequant_word(s == 0 ? cw[cb].x : s == 1 ? cw[cb].y : s == 2 ? cw[cb].z : cw[cb].w, dc[cb]);
      if (prio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][rb], bf[cb], acc[rb][cb], 0, 0, 0);
      if (prio) __builtin_amdgcn_s_setprio(0);
    }
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(APT + CL) : "memory");   // tile t + 1; own LDS reads done
    block_barrier();
  }
  // the clamped loads past the last tile must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const int nw = n0 + wn * 16 * NB;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const int n = nw + 32 * cb + lc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 16 * MB + 32 * rb + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (m < M && n < n_end) y[static_cast<size_t>(m) * N + n] = static_cast<half_t>(acc[rb][cb][r]);
      }
    }
}

// 256-row tile with every code dequantised once per workgroup (4-bit weights): the same
// wavefront tiles and MFMA steps as big_tile, but in each K tile the 512 threads expand
// the stage's codes cooperatively, thread (half h, column c) the 32 channels [32 h, +32)
// of column c, into a binary16 weight tile in LDS, and the wavefronts read their B
// operands from it instead of dequantising their own columns (which the two wavefronts
// sharing a column both did).  LDS (159,488 B): activations double-buffered (2 x 32 KB),
// codes, scales and zero points triple-buffered (3 x 9,472 B) so that a tile's codes are
// in LDS one K tile before it is computed, and the weight tile double-buffered (2 x 32
// KB, rows of 8 chunks of 8 channels, chunk j of column c at slot j ^ (c % 8)).  K tile t:
// request the activations of t + 1 and the codes of t + 2, expand the codes of t + 1 into
// weight buffer (t + 1) % 2, run the MFMAs of t on activation and weight buffers t % 2,
// then one barrier.
constexpr uint32_t kLdsbA = kBigBM * kBigBK * 2;
constexpr uint32_t kLdsbC = kBigLdsB + kBigLdsS + kBigLdsZ;
constexpr uint32_t kLdsbW = kBigBN * kBigBK * 2;
constexpr uint32_t kLdsbOffC = 2 * kLdsbA;
constexpr uint32_t kLdsbOffW = kLdsbOffC + 3 * kLdsbC;
constexpr size_t kLdsbLds = static_cast<size_t>(kLdsbOffW) + 2 * kLdsbW;
static_assert(kLdsbLds <= 160 * 1024, "fits the LDS of a compute unit");

template <int NB>
__device__ __forceinline__ void big_tile_ldsb(const half_t* __restrict__ x, const uint32_t* __restrict__ qw,
                                              const half_t* __restrict__ scales, Zeros qzeros,
                                              half_t* __restrict__ y, int M, int N, int K, int gshift, int m0,
                                              int n0, int n_end, int prio) {
  constexpr int MB = 8;
  using Loader = BigLoader<NB, MB, 4>;
  constexpr int BL = Loader::BL, LB = Loader::LB;
  constexpr int BN = 64 * NB;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int KT = K / kBigBK;
  const Loader ld(x, qw, scales, qzeros, smem, M, N, K, gshift, m0, n0, n_end, tid, wave);
  auto a_buf = [&](int t) { return smem + (t & 1) * kLdsbA; };
  auto c_buf = [&](int t) { return smem + kLdsbOffC + (t % 3) * kLdsbC; };
  auto w_buf = [&](int t) { return smem + kLdsbOffW + (t & 1) * kLdsbW; };

  // The expansion task of this thread: half eh, column ec (threads past the tile's
  // 2 BN pairs have none).
  const int eh = tid / BL, ec = tid % BL;
  const bool expands = ec < BN;
  auto expand = [&](int t) {
    if (!expands) return;
    const unsigned char* c = c_buf(t);
    const uint4 w = *reinterpret_cast<const uint4*>(c + (eh * BL + ec) * 16);
    const uint32_t sb = *reinterpret_cast<const uint16_t*>(c + LB + (eh * BL + ec) * 2);
    const uint32_t zw = *reinterpret_cast<const uint32_t*>(c + LB + kBigLdsS + (eh * (BL / 8) + (ec >> 3)) * 4);
    const DequantConsts dc = make_consts((qzeros.word(zw) >> (4 * (ec & 7))) & 0xFu,
                                         __builtin_bit_cast(half_t, static_cast<uint16_t>(sb)));
    unsigned char* wt = w_buf(t) + ec * 128;
    const uint32_t words[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = 4 * eh + q;
      *reinterpret_cast<half8_t*>(wt + 16 * (j ^ (ec & 7))) = dequant_word(words[q], dc);
    }
  };

  float4_t acc[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Lane offsets: A fragment mb of step s at a_lane + 16 ((2 q + s) ^ (r % 8)) + 2048 mb;
  // B fragment nb of step s at b_lane + 2048 nb + 16 ((2 q + s) ^ (r % 8)).
  const int a_lane = (wm * 16 * MB + lr) * 128;
  const int b_lane = (wn * 16 * NB + lr) * 128;

  ld.load_sz_to(0, c_buf(0));
  ld.load_a_to(0, a_buf(0));
  ld.load_codes_to(0, c_buf(0));
  ld.load_sz_to(1, c_buf(1));
  ld.load_codes_to(1, c_buf(1));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  block_barrier();
  expand(0);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  block_barrier();

  for (int t = 0; t < KT; ++t) {
    ld.load_a_to(t + 1, a_buf(t + 1));
    ld.load_sz_to(t + 2, c_buf(t + 2));
    ld.load_codes_to(t + 2, c_buf(t + 2));
    if (t + 1 < KT) expand(t + 1);
    const unsigned char* at = a_buf(t);
    const unsigned char* wt = w_buf(t);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      half8_t af[MB], bf[NB];
      const int sl = 16 * ((2 * lq + s) ^ (lr & 7));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) bf[nb] = *reinterpret_cast<const half8_t*>(wt + b_lane + 2048 * nb + sl);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const half8_t*>(at + a_lane + 2048 * mb + sl);
      if (prio) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mb], bf[nb], acc[mb][nb], 0, 0, 0);
      if (prio) __builtin_amdgcn_s_setprio(0);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    block_barrier();
  }

  const int nw = n0 + wn * 16 * NB;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = nw + 16 * nb + lr;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 16 * MB + 16 * mb + 4 * lq + r;
        if (m < M && n < n_end) y[static_cast<size_t>(m) * N + n] = static_cast<half_t>(acc[mb][nb][r]);
      }
    }
}

// prio != 0: each MFMA cluster runs at wavefront priority 1 (s_setprio), the LDS reads
// and dequantisation between clusters at 0.
// One launch covers up to two column ranges: workgroups [0, split) take BM x 256
// tiles of columns [0, n_split), the rest BM x 64 NB2 tiles of columns [n_split, N),
// BM = 32 MB rows (256 for prefill; 128 / 64 for batches of up to 128 / 64 rows).
// With one wave of full tiles and one of narrower tiles, both rounds fill the device
// when the full-width tiles alone would leave most of a second round idle.
// LDSB: 256-row tiles of 4-bit weights dequantised once per workgroup (big_tile_ldsb).
template <int NB2, int MB, int BITS = 4, bool W32 = false, bool LDSB = false>
__global__ __launch_bounds__(512) void gemm_big_kernel(const half_t* __restrict__ x, const uint32_t* __restrict__ qw,
                                                       const half_t* __restrict__ scales,
                                                       Zeros qzeros, half_t* __restrict__ y,
                                                       int M, int N, int K, int gshift, int split, int n_split,
                                                       int prio) {
  static_assert(!W32 || BITS == 4, "the 32x32 tile takes 4-bit weights");
  static_assert(!LDSB || (BITS == 4 && MB == 8 && !W32), "the dequantise-once tile: 4-bit, 256 rows");
  constexpr int BM = 32 * MB;
  const int tiles_m = (M + BM - 1) / BM;
  const int bid = blockIdx.x;
  if (bid < split) {
    const int tiles_n = (n_split + 255) / 256;
    const int tile = xcd_tile(bid, tiles_m, tiles_n);
    if constexpr (LDSB)
      big_tile_ldsb<4>(x, qw, scales, qzeros, y, M, N, K, gshift, (tile / tiles_n) * BM, (tile % tiles_n) * 256,
                       min(N, n_split), prio);
    else if constexpr (W32)
      big_tile32<4, MB>(x, qw, scales, qzeros, y, M, N, K, gshift, (tile / tiles_n) * BM, (tile % tiles_n) * 256,
                        min(N, n_split), prio);
    else
      big_tile<4, MB, BITS>(x, qw, scales, qzeros, y, M, N, K, gshift, (tile / tiles_n) * BM, (tile % tiles_n) * 256,
                            min(N, n_split), prio);
  } else {
    constexpr int BN2 = 64 * NB2;
    const int tiles_n = (N - n_split + BN2 - 1) / BN2;
    const int tile = xcd_tile(bid - split, tiles_m, tiles_n);
    if constexpr (LDSB)
      big_tile_ldsb<NB2>(x, qw, scales, qzeros, y, M, N, K, gshift, (tile / tiles_n) * BM,
                         n_split + (tile % tiles_n) * BN2, N, prio);
    else if constexpr (W32 && NB2 % 2 == 0)
      big_tile32<NB2, MB>(x, qw, scales, qzeros, y, M, N, K, gshift, (tile / tiles_n) * BM,
                          n_split + (tile % tiles_n) * BN2, N, prio);
    else
      big_tile<NB2, MB, BITS>(x, qw, scales, qzeros, y, M, N, K, gshift, (tile / tiles_n) * BM,
                              n_split + (tile % tiles_n) * BN2, N, prio);
  }
}

}  // namespace w4a16
