// Decode GEMV, M = 1: y[n] = sum_k x[k] * (q[n][k] - Z[g(k)][n]) * S[g(k)][n].
//
// At batch one every weight is read once for about two flops, so the kernel is
// bound by HBM bandwidth ("AWQ + GPTQ Quantization, in depth", What W4A16 buys and
// why decoding gets faster).  Everything is arranged to keep many bytes of packed
// weights in flight and to touch each weight with as few instructions as possible:
//
//  * Persistent grid, one workgroup per compute unit (or a small multiple).  Rows
//    are dealt out in units of one row per wavefront row-slot, round-robin over the
//    workgroups, so the whole grid sweeps through the weights together; the
//    workgroups of one XCD own neighbouring units and share the L2 lines of their
//    scales and zero points.
//  * A row's K input channels are split into 32-channel chunks (16 bytes of codes).
//    LPR lanes share a row; lane j owns chunks j, j+LPR, ... (CPL of them), so each
//    wave-wide 16-byte load is one contiguous run of the row.
//  * Long rows (more than 256 chunks, K > 8192) are split into WPR contiguous slices,
//    one per wavefront, so that no lane holds more than four chunks of activations
//    (more would spill registers).  A slice is a shorter contiguous row in memory;
//    the WPR wavefronts of a row each take WPR rows per step, one slice of each, and
//    the WPR partial sums of a row are added in slice order before the rounding.
//  * Each wavefront walks its rows with a DEPTH-deep register pipeline: the loads
//    of row t+DEPTH are issued as soon as row t has been consumed.
//  * Activations are loaded once into registers (under act order gathered through
//    the stored order via LDS): a lane owns the same chunks in every row.
//  * Scales and zero points follow the sweep: the (S * 2^24, -Z * S) pairs of one
//    step's rows are staged in a two-slot LDS ring, requested two steps ahead and
//    published by the workgroup barrier that closes each step.  A thread stages EPT
//    rows of one group: EPT = 1 (one row, 2 bytes of scale; eight neighbouring threads
//    read one 16-byte run) when there are no more entries than threads, so that the
//    conversion is spread over all wavefronts instead of holding up the barrier, else
//    EPT = 8 (16 bytes of scales, one word of zero points).  Staging a step at a time
//    keeps those small scattered reads in the same DRAM pages as the weights being
//    streamed and spreads them over the kernel.
//  * Codes are expanded by masking alone: a pair of nibbles in the mantissa bits of a
//    binary16 pair with a zero exponent field is the exact subnormal pair
//    (q, q') * 2^-24 (nibbles.hpp).  v_dot2_f32_f16 multiplies them with the
//    activations into two fp32 accumulators per chunk, one for the pairs taken from
//    the low nibbles of each byte and one, 16 times larger, for the high nibbles.
//    After the chunk t = acc_a + acc_b / 16 = 2^-24 * sum x q, and the zero point and
//    scale enter once per chunk:
//        row += t * (S * 2^24) + (-Z * S) * sum x.
//    9 VALU instructions per 8 weights in the inner loop, all but the dot products
//    plain 32-bit AND/shift.
//  * The LPR partial sums of a row are reduced inside the wavefront with DPP moves
//    only (mirrors within rows of 16 lanes, row broadcasts across them); the row
//    result is rounded once to binary16.  Results wait in LDS and are stored at the
//    end: a store counts against the same wait counter as the loads, so stores in the
//    loop would hold back the waits for the weight pipeline.
#pragma once

#include <type_traits>

#include "nibbles.hpp"

namespace w4a16 {

// DPP move of a float: lanes of rows outside row_mask receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of L lanes (L a power of two <= 64), with VALU-only DPP
// moves (no LDS round trips).  Groups of up to 16 lanes: every lane ends with the
// total.  L = 32 and 64: the total ends in the group's last lane (31/63, 63).
template <int L>
__device__ __forceinline__ float lane_group_sum(float v) {
  if constexpr (L >= 2) v += dpp_f32<0xB1, 0xF>(v);     // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (L >= 4) v += dpp_f32<0x4E, 0xF>(v);     // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (L >= 8) v += dpp_f32<0x141, 0xF>(v);    // row_half_mirror: the other quad of 8
  if constexpr (L >= 16) v += dpp_f32<0x140, 0xF>(v);   // row_mirror: the other half of 16
  if constexpr (L >= 32) v += dpp_f32<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  if constexpr (L >= 64) v += dpp_f32<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}


// Row schedule.  Rows are grouped into units of STRIDE = WAVES * RPW consecutive rows
// (one row per wavefront row-slot); unit u is processed by workgroup u % nblk at step
// u / nblk.  At any moment the whole grid streams one contiguous window of the
// weights, and within a unit the wavefronts read neighbouring rows.
// LDS: scale/zero ring 2 * STRIDE * (G + 1) float2, row results steps * STRIDE * WPR floats,
// and under act order the gathered activations, K binary16.  Needs 8 OCT G / EPT <=
// WAVES * 64 (at most one staging task per thread and step) and an even DEPTH.
//
// BITS = 8 (8-bit weights, four codes per word in the byte order 0, 2, 1, 3): a 16-byte
// chunk is 16 channels, the pairs of a word are its bytes 0 and 2 and (after a shift by
// 8) 1 and 3 as subnormals q * 2^-24 (q < 256 fits the mantissa), both accumulated
// with weight 1, and the zero points are bytes.
//
// PRE (whole rows, or WPR slices of each): the workgroup owns `steps`
// consecutive units instead of every nblk-th one, and stages the (S * 2^24, -Z * S)
// pairs of all its rows once, before the first row: for every group the scales of its
// rows are one contiguous run, so the whole grid reads the scale and zero-point arrays
// front to back in a burst at the start instead of as scattered pieces between the code
// streams of every step.  The rows then run without a barrier.  LDS: steps * STRIDE *
// (G + 1) float2 instead of the ring.  Without act order and with at least 2 DEPTH
// steps (flags bit 0), the dot products of the first DEPTH rows are taken before the
// staging barrier and their register slots refilled at once; their scaling follows the
// barrier (the same operations in the same order, so the same bits).
// CT (with PRE): the table holds each pair as a 32-bit entry, binary16 S and the zero point
// above it, converted to (S * 2^24, -Z * S) when a row is scaled (the same fp32 values), so
// that tables of many groups (group size 32 on large layers) fit in LDS.
template <int LPR, int CPL, int WAVES, int DEPTH, bool EXACT, bool ACT, int EPT, int WPR, int BITS = 4,
          bool PRE = false, bool CT = false>
__global__ __launch_bounds__(WAVES * 64) void gemv_m1_kernel(
    const half_t* __restrict__ x, const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    Zeros qzeros, half_t* __restrict__ y, int N, int K, int gshift, int steps, int flags) {
  static_assert(64 % LPR == 0, "lanes per row must divide the wavefront");
  static_assert(DEPTH % 2 == 0, "the ring slot of row t is t % 2, the unrolled slot index");
  static_assert(WPR == 1 || (LPR == 64 && WAVES % WPR == 0 && WPR % DEPTH == 0),
                "split rows: one row per wavefront, whole register slots per step");
  static_assert(BITS == 4 || BITS == 8, "4- or 8-bit weights");
  static_assert(!PRE || EPT == 8, "staging once: 8-row items");
  static_assert(!CT || (PRE && BITS == 4), "the compact table: staging once, 4-bit zero points");
  constexpr int CSH = BITS == 4 ? 5 : 4;   // log2 channels per 16-byte chunk
  constexpr int XQ = 1 << (CSH - 3);       // 16-byte pieces of activations per chunk
  constexpr int XP = 4 * XQ;               // activation pairs per chunk
  constexpr int RPW = 64 / LPR;          // rows per wavefront per step
  constexpr int STRIDE = WAVES * RPW;    // rows per unit
  static_assert(STRIDE % 8 == 0, "a unit must cover whole 8-row groups of zero points");
  constexpr int OCT = STRIDE / 8;        // 8-row groups per unit
  constexpr int NT = WAVES * 64;
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rr = lane / LPR;
  const int j = lane % LPR;
  const int C = K >> CSH;                // 16-byte chunks per row
  const int CS = (C + WPR - 1) / WPR;    // chunks per slice
  const int h = WPR == 1 ? 0 : wave % WPR;   // this wavefront's slice
  const int W = K >> (BITS == 4 ? 3 : 2);  // words per row
  const int G = ((K - 1) >> gshift) + 1;  // groups per row (one per row when per-channel)
  const int GP = G + 1;                  // padded ring row (float2)
  const int nblk = gridDim.x;
  const int blk = xcd_block(blockIdx.x, nblk);
  // Row inside a unit at sub-step s (split rows: WPR sub-steps per step, WAVES / WPR
  // rows each), and the matrix row of the wavefront's seq-th row (seq = t WPR + s).
  auto unit_row = [&](int s) { return WPR == 1 ? wave * RPW + rr : wave / WPR + (WAVES / WPR) * s; };
  const int my_row = unit_row(0);
  // PRE: units blk * steps + t.
  auto row_of = [&](int seq) {
    return PRE ? (blk * steps + seq / WPR) * STRIDE + unit_row(seq % WPR)
               : (blk + (seq / WPR) * nblk) * STRIDE + unit_row(seq % WPR);
  };

  // PRE: the ring is the table of all the workgroup's rows, [steps][STRIDE][GP].
  float2* ring = reinterpret_cast<float2*>(smem);                                   // [2][STRIDE][GP]
  uint32_t* ringc = reinterpret_cast<uint32_t*>(smem);                              // CT: [steps][STRIDE][GP]
  float* ybuf = reinterpret_cast<float*>(smem + (PRE ? steps : 2) * static_cast<size_t>(STRIDE) * GP *
                                                    (CT ? sizeof(uint32_t) : sizeof(float2)));
  half_t* xs = reinterpret_cast<half_t*>(ybuf + static_cast<size_t>(steps) * STRIDE * WPR);

  // This lane's chunks (clamped into its slice and the row unless the split is exact)
  // and their groups; `live` chunks lie inside both.
  int chunk[CPL], gcol[CPL];
  bool live[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int local = j + LPR * i;
    chunk[i] = EXACT ? h * CS + local : min(h * CS + min(local, CS - 1), C - 1);
    live[i] = EXACT || (local < CS && h * CS + local < C);
    gcol[i] = (chunk[i] << CSH) >> gshift;
  }

  // Staging task of this thread: rows [8 o + r0, 8 o + r0 + EPT) of the unit, group g
  // (item (o, g) = 8 rows of one group, split over 8 / EPT threads with r0 fastest).
  static_assert(EPT == 1 || EPT == 8, "staging rows per thread");
  constexpr int TPI = 8 / EPT;
  const int tasks = OCT * G * TPI;
  const int ts_c = min(tid, tasks - 1);
  const int it_c = ts_c / TPI;
  const int it_g = it_c % G;
  const int it_o = it_c / G;
  const int st_r0 = (ts_c % TPI) * EPT;
  using ScaleBits = std::conditional_t<EPT == 8, uint4, uint16_t>;
  using ZeroBits = std::conditional_t<BITS == 4, uint32_t, uint2>;   // the zero points of 8 rows
  ScaleBits zs_s[2];
  ZeroBits zs_z[2];
  auto load_item = [&](int t, int set) {   // unconditional: rows and steps clamped
    const int n8 = min((blk + min(t, steps - 1) * nblk) * STRIDE + 8 * it_o, N - 8);
    if constexpr (EPT == 8)
      zs_s[set] = *reinterpret_cast<const uint4*>(scales + static_cast<size_t>(it_g) * N + n8);
    else
      zs_s[set] = scales[static_cast<size_t>(it_g) * N + n8 + st_r0];
    if constexpr (BITS == 4)
      zs_z[set] = *qzeros.at(static_cast<size_t>(it_g) * (N >> 3) + (n8 >> 3));
    else
      zs_z[set] = *reinterpret_cast<const uint2*>(qzeros.at(static_cast<size_t>(it_g) * (N >> 2) + (n8 >> 2)));
  };
  auto put_item = [&](int set, int slot) {
    if (tid < tasks) {
      float2* dst = ring + (slot * STRIDE + 8 * it_o + st_r0) * GP + it_g;
#pragma unroll
      for (int r = 0; r < EPT; ++r) {
        uint32_t bits;
        if constexpr (EPT == 8) {
          const uint32_t s8[4] = {zs_s[set].x, zs_s[set].y, zs_s[set].z, zs_s[set].w};
          bits = (s8[r >> 1] >> (16 * (r & 1))) & 0xFFFFu;
        } else {
          bits = zs_s[set];
        }
        const float S = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(bits)));
        float Z;
        if constexpr (BITS == 4) {
          Z = static_cast<float>((qzeros.word(zs_z[set]) >> (4 * (st_r0 + r))) & 0xFu);
        } else {
          const int zr = st_r0 + r;
          const uint32_t zw = qzeros.word8(zr < 4 ? zs_z[set].x : zs_z[set].y);
          Z = static_cast<float>((zw >> (8 * (zr & 3))) & 0xFFu);
        }
        dst[r * GP] = make_float2(S * 16777216.0f, -Z * S);   // both exact in fp32
      }
    }
  };

  // 1. Requests, smallest first so they do not queue behind the weights: the
  // activations of this lane's chunks (without act order straight into registers;
  // under act order the stored channel order, 16 bytes per load, all at once), the
  // staging items of steps 0 and 1, then the first DEPTH rows of codes.
  uint4 xv[CPL][XQ];
  // Under act order the stored order is read in 4-entry pieces, PPT per thread to
  // cover the whole row, PB of them in flight per round.
  constexpr int PPT = (WPR * LPR * CPL * (1 << CSH) / 4 + NT - 1) / NT;
  constexpr int PB = PPT < 4 ? PPT : 4;
  const int4* perm4 = reinterpret_cast<const int4*>(qw + static_cast<size_t>(N) * W);
  int4 pv[PB];
  if constexpr (!ACT) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int q = 0; q < XQ; ++q) xv[i][q] = reinterpret_cast<const uint4*>(x)[XQ * chunk[i] + q];
  } else {
#pragma unroll
    for (int u = 0; u < PB; ++u) pv[u] = perm4[min(tid + u * NT, (K >> 2) - 1)];
  }
  if constexpr (!PRE) {
    load_item(0, 0);
    load_item(1, 1);
  }
  uint4 wb[DEPTH][CPL];
  // the codes part of qweight, N K / 2 < 2^31 bytes (checked by the host)
  const __amdgpu_buffer_rsrc_t codes = stream_rsrc(qw, static_cast<uint32_t>(N) * static_cast<uint32_t>(W) * 4u);
  auto load_row = [&](uint4 (&dst)[CPL], int n) {   // unconditional: row clamped into the matrix
    const int nc = min(n, N - 1);
#pragma unroll
    for (int i = 0; i < CPL; ++i)
      dst[i] = load_stream16(codes, (static_cast<uint32_t>(nc) * static_cast<uint32_t>(W) + 4u * chunk[i]) * 4u);
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_row(wb[d], row_of(d));  // clamped if there are fewer rows

  // PRE: items (octet o of the workgroup's rows, group g), item g * OCTS + o, so that
  // neighbouring threads read neighbouring 16-byte pieces of one group's run of scales;
  // kPreBatch items per thread and round (the host allows at most two rounds), loads
  // clamped into the items so that every thread issues the same loads.
  constexpr int kPreBatch = CT ? 4 : 2;
  const int pre_octs = steps * OCT;
  const int pre_items = PRE ? pre_octs * G : 0;
  const int pre_r0 = blk * steps * STRIDE;
  uint4 ps[kPreBatch];
  ZeroBits pz[kPreBatch];
  auto pre_load = [&](int round) {
#pragma unroll
    for (int u = 0; u < kPreBatch; ++u) {
      const int it = min(tid + (round * kPreBatch + u) * NT, pre_items - 1);
      const int g = it / pre_octs, o = it - g * pre_octs;
      const int n8 = min(pre_r0 + 8 * o, N - 8);
      ps[u] = *reinterpret_cast<const uint4*>(scales + static_cast<size_t>(g) * N + n8);
      if constexpr (BITS == 4)
        pz[u] = *qzeros.at(static_cast<size_t>(g) * (N >> 3) + (n8 >> 3));
      else
        pz[u] = *reinterpret_cast<const uint2*>(qzeros.at(static_cast<size_t>(g) * (N >> 2) + (n8 >> 2)));
    }
  };
  auto pre_put = [&](int round) {
#pragma unroll
    for (int u = 0; u < kPreBatch; ++u) {
      const int it = tid + (round * kPreBatch + u) * NT;
      if (it < pre_items) {
        const int g = it / pre_octs, o = it - g * pre_octs;
        const uint32_t s8[4] = {ps[u].x, ps[u].y, ps[u].z, ps[u].w};
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          if constexpr (CT) {
            ringc[(8 * o + r) * GP + g] = ((s8[r >> 1] >> (16 * (r & 1))) & 0xFFFFu) |
                                          (((qzeros.word(pz[u]) >> (4 * r)) & 0xFu) << 16);
            continue;
          }
          const float S = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>((s8[r >> 1] >> (16 * (r & 1))) & 0xFFFFu)));
          float Z;
          if constexpr (BITS == 4) {
            Z = static_cast<float>((qzeros.word(pz[u]) >> (4 * r)) & 0xFu);
          } else {
            const uint32_t zw = qzeros.word8(r < 4 ? pz[u].x : pz[u].y);
            Z = static_cast<float>((zw >> (8 * (r & 3))) & 0xFFu);
          }
          ring[(8 * o + r) * GP + g] = make_float2(S * 16777216.0f, -Z * S);   // both exact in fp32
        }
      }
    }
  };
  const int pre_rounds = PRE ? (pre_items + kPreBatch * NT - 1) / (kPreBatch * NT) : 0;
  if constexpr (PRE) pre_load(0);

  // 2. Act order: gather the activations into LDS in stored order (all gathers of a
  // thread in flight together).  Step 0's items go to ring slot 0; the barrier
  // publishes both.
  if constexpr (ACT) {
#pragma unroll
    for (int r0 = 0; r0 < PPT; r0 += PB) {
      if (r0 > 0) {
#pragma unroll
        for (int u = 0; u < PB; ++u) pv[u] = perm4[min(tid + (r0 + u) * NT, (K >> 2) - 1)];
      }
      half_t g[PB][4];
#pragma unroll
      for (int u = 0; u < PB; ++u) {
        g[u][0] = x[pv[u].x];
        g[u][1] = x[pv[u].y];
        g[u][2] = x[pv[u].z];
        g[u][3] = x[pv[u].w];
      }
#pragma unroll
      for (int u = 0; u < PB; ++u)
        if (r0 + u < PPT && tid + (r0 + u) * NT < (K >> 2))
          *reinterpret_cast<uint2*>(xs + 4 * (tid + (r0 + u) * NT)) =
              uint2{static_cast<uint32_t>(__builtin_bit_cast(uint16_t, g[u][0])) |
                        (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, g[u][1])) << 16),
                    static_cast<uint32_t>(__builtin_bit_cast(uint16_t, g[u][2])) |
                        (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, g[u][3])) << 16)};
    }
  }
  // 3. this lane's activations as pairs (without act order straight from the loaded
  // registers, before the barrier; under act order from LDS after it), and the
  // per-chunk sums (dot2 with ones); chunks past the end of the row (inexact split)
  // contribute nothing.
  half2_t xr[CPL][XP];
  float xsum[CPL];
  auto build_xr = [&]() {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int q = 0; q < XQ; ++q) {
        const uint4 v = xv[i][q];
        xr[i][4 * q + 0] = live[i] ? as_h2(v.x) : half2_t{0, 0};
        xr[i][4 * q + 1] = live[i] ? as_h2(v.y) : half2_t{0, 0};
        xr[i][4 * q + 2] = live[i] ? as_h2(v.z) : half2_t{0, 0};
        xr[i][4 * q + 3] = live[i] ? as_h2(v.w) : half2_t{0, 0};
      }
  };
  // A row in two parts: the dot products of its codes with the activations (aa: pairs
  // from the low nibbles, ab: from the high ones), which need neither the staged scales
  // nor a barrier, and the scaling by the row's (S * 2^24, -Z * S) pairs.
  auto row_dots = [&](uint4 (&w)[CPL], float (&aa)[CPL], float (&ab)[CPL]) {
    // The CPL chunks are interleaved word by word: 2*CPL independent dot2
    // accumulation chains (each still summed in the same order).
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      aa[i] = 0.f;
      ab[i] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t word = q == 0 ? w[i].x : q == 1 ? w[i].y : q == 2 ? w[i].z : w[i].w;
        if constexpr (BITS == 4) {
          const SubPairs p = expand_word_subnormal(word);
          aa[i] = __builtin_amdgcn_fdot2(as_h2(p.a0), xr[i][4 * q + 0], aa[i], false);
          ab[i] = __builtin_amdgcn_fdot2(as_h2(p.b0), xr[i][4 * q + 1], ab[i], false);
          aa[i] = __builtin_amdgcn_fdot2(as_h2(p.a1), xr[i][4 * q + 2], aa[i], false);
          ab[i] = __builtin_amdgcn_fdot2(as_h2(p.b1), xr[i][4 * q + 3], ab[i], false);
        } else {   // bytes 0, 2 and 1, 3: elements (e0, e1) and (e2, e3)
          aa[i] = __builtin_amdgcn_fdot2(as_h2(word & 0x00FF00FFu), xr[i][2 * q + 0], aa[i], false);
          ab[i] = __builtin_amdgcn_fdot2(as_h2((word >> 8) & 0x00FF00FFu), xr[i][2 * q + 1], ab[i], false);
        }
      }
    }
  };
  auto row_finish = [&](int slot, int row, const float (&aa)[CPL], const float (&ab)[CPL]) {
    float2 sc[CPL];
    if constexpr (CT) {
      const uint32_t* szr = ringc + (slot * STRIDE + row) * GP;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint32_t e = szr[gcol[i]];
        const float S = static_cast<float>(__builtin_bit_cast(half_t, static_cast<uint16_t>(e & 0xFFFFu)));
        const float Z = static_cast<float>(e >> 16);
        sc[i] = make_float2(S * 16777216.0f, -Z * S);   // the pairs of the float table, exactly
      }
    } else {
      const float2* szr = ring + (slot * STRIDE + row) * GP;
#pragma unroll
      for (int i = 0; i < CPL; ++i) sc[i] = szr[gcol[i]];
    }
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float tq = fmaf(ab[i], BITS == 4 ? 0.0625f : 1.0f, aa[i]);  // 2^-24 * sum x q
      acc = fmaf(tq, sc[i].x, acc);                  // + S * sum x q
      acc = fmaf(sc[i].y, xsum[i], acc);             // - Z * S * sum x
    }
    return acc;
  };
  auto row_step = [&](int slot, int row, uint4 (&w)[CPL]) {
    float aa[CPL], ab[CPL];
    row_dots(w, aa, ab);
    return row_finish(slot, row, aa, ab);
  };

  if constexpr (!ACT) build_xr();
  if constexpr (PRE) {
    for (int round = 0; round < pre_rounds; ++round) {
      if (round > 0) pre_load(round);
      pre_put(round);
    }
  } else {
    put_item(0, 0);
  }
  // PRE without act order, at least 2 DEPTH rows per wavefront (flags bit 0): the first
  // DEPTH rows' dot products are taken before the barrier and their register slots
  // refilled with the next rows at once, so the second round of requests does not wait
  // for the staging, the barrier and the activation sums.
  float pa[DEPTH][CPL], pb[DEPTH][CPL];
  bool early = false;
  if constexpr (PRE && !ACT) {
    early = (flags & 1) != 0 && steps * WPR >= 2 * DEPTH;
    if (early) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        row_dots(wb[d], pa[d], pb[d]);
        load_row(wb[d], row_of(d + DEPTH));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();
  if constexpr (ACT) {
#pragma unroll
    for (int i = 0; i < CPL; ++i)
#pragma unroll
      for (int q = 0; q < XQ; ++q) xv[i][q] = reinterpret_cast<const uint4*>(xs)[XQ * chunk[i] + q];
    build_xr();
  }
  const half2_t ones = half2_t{static_cast<half_t>(1.0f), static_cast<half_t>(1.0f)};
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    float sx = 0.f;
#pragma unroll
    for (int q = 0; q < XP; ++q) sx = __builtin_amdgcn_fdot2(xr[i][q], ones, sx, false);
    xsum[i] = sx;
  }

  // 4. rows.  Row t sits in register slot t % DEPTH; its codes were requested DEPTH
  // steps earlier, its staging items two steps earlier into set t % 2, and they were
  // published into ring slot t % 2 by the barrier closing step t - 1.  Every step
  // (a) requests the items of step t + 2, (b) computes row t and refills its slot,
  // (c) stages step t + 1 and closes with the barrier.  The last DEPTH steps run
  // without code refills, so no load is issued past the end.
  // The row (slice) total ends in lane LPR - 1 of the row's lane group.
  auto keep = [&](int t, int row, float acc) {
    acc = lane_group_sum<LPR>(acc);
    if (j == LPR - 1) ybuf[(t * STRIDE + row) * WPR + h] = acc;
  };
  // one step; P = t % 2 at compile time (t0 is a multiple of the even DEPTH)
  auto step = [&](int t, int d, bool refill, auto P) {
    constexpr int p = decltype(P)::value;
    load_item(t + 2, p);                                  // (a) into the set just published
    const float acc = row_step(p, my_row, wb[d]);         // (b)
    if (refill) load_row(wb[d], row_of(t + DEPTH));
    __builtin_amdgcn_sched_barrier(0);
    keep(t, my_row, acc);
    put_item(p ^ 1, p ^ 1);                               // (c) step t + 1
    __syncthreads();
  };
  // Split rows: a step is WPR rows of this wavefront (seq = t WPR + s, register slot
  // s % DEPTH), each refilled with row seq + DEPTH; LAST = the final step, whose
  // refills past the end are dropped at compile time.
  auto split_step = [&](int t, auto P, auto LAST) {
    constexpr int p = decltype(P)::value;
    constexpr bool last = decltype(LAST)::value;
    load_item(t + 2, p);
#pragma unroll
    for (int s = 0; s < WPR; ++s) {
      const int row = unit_row(s);
      const float acc = row_step(p, row, wb[s % DEPTH]);
      if (!last || s + DEPTH < WPR) load_row(wb[s % DEPTH], row_of(t * WPR + s + DEPTH));
      __builtin_amdgcn_sched_barrier(0);
      keep(t, row, acc);
    }
    put_item(p ^ 1, p ^ 1);
    __syncthreads();
  };
  // PRE: the wavefront's seq-th row (slice) is row unit_row(seq % WPR) of step seq / WPR,
  // whose pairs are that row of the table; no staging and no barrier per step.
  auto pre_step = [&](int seq, int d, bool refill) {
    const int t = seq / WPR, row = unit_row(seq % WPR);
    const float acc = row_step(t, row, wb[d]);
    if (refill) load_row(wb[d], row_of(seq + DEPTH));
    __builtin_amdgcn_sched_barrier(0);
    keep(t, row, acc);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using More = std::false_type;
  using Last = std::true_type;
  if constexpr (PRE) {
    const int total = steps * WPR;   // rows (slices) of this wavefront
    int t0 = 0;
    if (early) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int t = d / WPR, row = unit_row(d % WPR);
        keep(t, row, row_finish(t, row, pa[d], pb[d]));
      }
      t0 = DEPTH;
    }
    for (; t0 + 2 * DEPTH <= total; t0 += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) pre_step(t0 + d, d, true);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (t0 + d < total) pre_step(t0 + d, d, t0 + d + DEPTH < total);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (t0 + DEPTH + d < total) pre_step(t0 + DEPTH + d, d, false);
    __syncthreads();   // every row result is in LDS
  } else if constexpr (WPR > 1) {
    int t = 0;
    for (; t + 2 < steps; t += 2) {
      split_step(t, I0{}, More{});
      split_step(t + 1, I1{}, More{});
    }
    if (t + 1 < steps) {
      split_step(t, I0{}, More{});
      split_step(t + 1, I1{}, Last{});
    } else {
      split_step(t, I0{}, Last{});
    }
  } else {

  int t0 = 0;
  for (; t0 + 2 * DEPTH <= steps; t0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; d += 2) {
      step(t0 + d, d, true, std::integral_constant<int, 0>{});
      step(t0 + d + 1, d + 1, true, std::integral_constant<int, 1>{});
    }
  }
  // between DEPTH and 2*DEPTH - 1 steps remain (or fewer than DEPTH in total)
#pragma unroll
  for (int d = 0; d < DEPTH; d += 2) {
    if (t0 + d < steps) step(t0 + d, d, t0 + d + DEPTH < steps, std::integral_constant<int, 0>{});
    if (t0 + d + 1 < steps) step(t0 + d + 1, d + 1, t0 + d + 1 + DEPTH < steps, std::integral_constant<int, 1>{});
  }
#pragma unroll
  for (int d = 0; d < DEPTH; d += 2) {
    if (t0 + DEPTH + d < steps) step(t0 + DEPTH + d, d, false, std::integral_constant<int, 0>{});
    if (t0 + DEPTH + d + 1 < steps) step(t0 + DEPTH + d + 1, d + 1, false, std::integral_constant<int, 1>{});
  }
  }

  // 5. the workgroup's rows: STRIDE consecutive outputs per step (the last step's
  // barrier published every result); split rows add their slices in order
  for (int idx = tid; idx < steps * STRIDE; idx += NT) {
    const int t = idx / STRIDE;
    const int n = PRE ? blk * steps * STRIDE + idx : (blk + t * nblk) * STRIDE + (idx - t * STRIDE);
    float v = ybuf[idx * WPR];
#pragma unroll
    for (int s = 1; s < WPR; ++s) v += ybuf[idx * WPR + s];
    if (n < N) y[n] = static_cast<half_t>(v);
  }
}

}  // namespace w4a16
