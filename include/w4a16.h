/*
 * w4a16.h -- C ABI of the W4A16 group-quantised linear layer for gfx950 (MI355X).
 *
 * The layer is y = x * W^T with W (out x in) stored as 4-bit codes q, one binary16
 * scale S and one 4-bit zero point Z per group of input channels, and
 *     W^[n][k] = (q[n][k] - Z[g(k)][n]) * S[g(k)][n]
 * ("LLM Quantization: A Deep Dive into GPTQ, AWQ, and Post-Training Quantization",
 * The Math of Quantization: q = round(x/S) + Z, x ~ (q - Z) * S).  The kernel loads
 * the packed 4-bit weights, expands them in registers with the group's scale and
 * zero point and multiplies them with 16-bit activations, accumulating in fp32
 * ("AWQ + GPTQ Quantization, in depth", What W4A16 buys and why decoding gets
 * faster).  A group is a run of group_size consecutive input channels of one output
 * row ("How do GPTQ and AWQ differ when quantizing Llama weights to 4 bits?", The
 * shared setting; FAQ on group_size 128), or, under GPTQ act order, the set of input
 * channels k with g_idx[k] equal to the group's number ("AWQ + GPTQ Quantization, in
 * depth", The two algorithms, compactly).
 *
 * Conventions for every entry point
 *   - binary16 values travel as uint16_t bit patterns; the stream is a hipStream_t
 *     passed as void* (NULL = the null stream).
 *   - shapes: M rows of activations, N output features, K input features,
 *     G = K / group_size groups per row.  Requirements: M, N, K > 0;
 *     group_size in {32, 64, 128}, or group_size == K for one scale (and zero point)
 *     per output row ("LLM Quantization: INT8, GPTQ, and AWQ Explained", What
 *     quantization actually does: per-channel); K % group_size == 0; K % 32 == 0;
 *     N % 8 == 0.
 *   - the caller owns every buffer.  The library keeps no pointer after a call
 *     returns.  Host entry points are synchronous.  Device entry points are
 *     asynchronous and stream-ordered: inputs must stay alive, and outputs are
 *     valid, only once the stream has passed the call.
 *   - every entry point returns a status (below); on failure nothing is launched
 *     and w4a16_last_error() (thread-local) describes the cause.  No exception
 *     crosses the ABI.  There is no silent fallback to a slower path: an argument
 *     no kernel supports is an error ("AWQ + GPTQ Quantization, in depth",
 *     Failure modes: kernel fallback).
 *
 * Layouts
 *   x        binary16 [M][K], row-major                               (device)
 *   y        binary16 [M][N], row-major, written once per element     (device)
 *   scales   binary16 [G][N], row-major: scale of (group, output)     (device)
 *   qzeros   int32 [G][N/8] or NULL (symmetric: every zero point 8): zero point of
 *            (group, n) in bits 4j..4j+3 of word
 *            [group][n/8], j = n % 8                                  (device)
 *   g_idx    int32 [K] or NULL: group of every input channel          (act order)
 *   qweight  int32 buffer of w4a16_qweight_words(N, K, act_order) words, written by
 *            w4a16_pack and read by the kernels.  Its internal layout is private to
 *            this library and may change with W4A16_ABI_VERSION; read it back only
 *            through w4a16_unpack.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define W4A16_ABI_VERSION 1

enum w4a16_status {
  W4A16_OK = 0,
  W4A16_ERR_INVALID_ARG = 1,  /* NULL pointer, non-positive size, K % group_size, N % 8,
                                 a code or zero point above 15 */
  W4A16_ERR_UNSUPPORTED = 2,  /* group_size not in {32, 64, 128} */
  W4A16_ERR_BAD_GIDX = 3,     /* g_idx value outside [0, G), a group without exactly
                                 group_size members, or a stored order that is not a
                                 permutation */
  W4A16_ERR_MISALIGNED = 4,   /* a device buffer not aligned to 16 bytes */
  W4A16_ERR_HIP = 5           /* HIP launch or runtime error; text in w4a16_last_error */
};

/* W4A16_ABI_VERSION of the built library.  Interface only (no passage of the pages
 * defines it). */
int w4a16_abi_version(void);

/* Text of the last failure on the calling thread ("" if none).  The pointer stays
 * valid until the thread's next call into the library.  Interface only. */
const char* w4a16_last_error(void);

/* Number of int32 words of the packed weight buffer: N*K/8, plus K when act_order is
 * non-zero (the stored input-channel order follows the codes).  0 on bad sizes.
 * Eight 4-bit codes per 32-bit word, i.e. 4 bits per weight before the per-group scale
 * and zero point ("AWQ + GPTQ Quantization, in depth", What W4A16 buys and why
 * decoding gets faster: packed 4-bit weights, 4.13 to 4.16 bits per weight with the
 * group's 16-bit scale and 4-bit zero point). */
size_t w4a16_qweight_words(int N, int K, int act_order);

/* ---------------------------------------------------------------------------------
 * Offline steps, host memory, synchronous.
 * ------------------------------------------------------------------------------ */

/* Asymmetric 4-bit round-to-nearest group quantiser ("LLM Quantization: INT8, GPTQ,
 * and AWQ Explained", What quantization actually does: find the range, pick a scale
 * that spreads the grid across it, round to the nearest grid point; 16 levels at 4
 * bits per Round-to-nearest, and where it falls apart).  Per (row n, group):
 *   w_lo = min(0, min w), w_hi = max(0, max w)
 *   S = smallest binary16 >= (w_hi - w_lo) / 15   (S = 1, Z = 0, q = 0 if w_hi == w_lo)
 *   Z = clamp(round(-w_lo / S), 0, 15),  q = clamp(round(w / S) + Z, 0, 15)
 * with round = half to even and all arithmetic in binary64.
 *   w         binary16 [N][K] weights (out x in)
 *   g_idx     int32 [K] group of each input channel, or NULL (group k / group_size)
 *   in_scale  binary64 [K] per-input-channel factor s, or NULL: the weights quantised
 *             are then w[n][k] * s[k] formed in binary64 (the AWQ fold, "AWQ + GPTQ
 *             Quantization, in depth", The two algorithms, compactly)
 *   codes     out uint8 [N][K];  scales out binary16 [G][N];  zeros out uint8 [G][N]
 * Errors: INVALID_ARG, UNSUPPORTED, BAD_GIDX (also for in_scale <= 0 or not finite). */
int w4a16_quantize(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                   const double* in_scale, uint8_t* codes, uint16_t* scales, uint8_t* zeros);

/* Symmetric 4-bit round-to-nearest group quantiser: the absmax scheme ("LLM
 * Quantization: INT8, GPTQ, and AWQ Explained", What quantization actually does: one
 * scale from the block's largest magnitude, round, clamp to the symmetric range) on the
 * grid -7 .. 7, as the symmetric W4A16 scheme of the GPTQ recipe ("AWQ + GPTQ
 * Quantization, in depth", Running it).  Per (row n, group):
 *   a = max |w|,  S = smallest binary16 >= a / 7   (S = 1 if a == 0)
 *   q = clamp(round(w / S), -7, 7),  codes = q + 8
 * so the zero point is 8 for every group and none is stored: pass qzeros = NULL to
 * w4a16_gemm / w4a16_dequant.  round = half to even, arithmetic in binary64; g_idx and
 * in_scale as for w4a16_quantize.
 *   codes out uint8 [N][K] (1 .. 15);  scales out binary16 [G][N]
 * Errors: INVALID_ARG, UNSUPPORTED, BAD_GIDX. */
int w4a16_quantize_sym(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                       const double* in_scale, uint8_t* codes, uint16_t* scales);

/* AWQ per-input-channel scale s[k] = (mean over the T calibration tokens of |X[t][k]|)
 * ** alpha ("AWQ + GPTQ Quantization, in depth", The two algorithms, compactly).  The
 * mean is formed exactly and rounded once; alpha == 0.5 uses the correctly rounded
 * square root.  A channel whose activations are all zero gets s = 1.
 *   xcal binary16 [T][K] (host);  s out binary64 [K].   Errors: INVALID_ARG. */
int w4a16_awq_scales(const uint16_t* xcal, int T, int K, double alpha, double* s);

/* Activation side of the AWQ fold: x_out[m][k] = binary16(x[m][k] / s[k]), rounded
 * once to nearest even ("How do GPTQ and AWQ differ...", AWQ: protect the salient
 * channels).  Host memory; x_out may alias x.  Errors: INVALID_ARG. */
int w4a16_awq_fold_activations(const uint16_t* x, int M, int K, const double* s, uint16_t* x_out);

/* GPTQ act-order group assignment ("AWQ + GPTQ Quantization, in depth", The two
 * algorithms, compactly: H = 2 X X^T; act order visits input channels by descending
 * diag(H)).  Channels are ordered by descending sum_t X[t][k]^2 (computed exactly),
 * ties by ascending k; the i-th channel in that order gets group i / group_size.
 *   xcal binary16 [T][K] (host);  g_idx out int32 [K].
 * Errors: INVALID_ARG, UNSUPPORTED. */
int w4a16_act_order(const uint16_t* xcal, int T, int K, int group_size, int32_t* g_idx);

/* Pack 4-bit codes into the library's weight buffer: eight codes per 32-bit word
 * ("AWQ + GPTQ Quantization, in depth", What W4A16 buys and why decoding gets faster:
 * the weights are stored as packed 4-bit integers; the codes are the q of q =
 * round(x/S) + Z in "LLM Quantization: A Deep Dive into GPTQ, AWQ, and Post-Training
 * Quantization", The Math of Quantization).  Act order stores each row in the order
 * in which GPTQ visits the input channels ("AWQ + GPTQ Quantization, in depth", The two
 * algorithms, compactly), so that every group is a contiguous run.
 *   codes   uint8 [N][K], values 0..15, in the original input-channel order
 *   g_idx   NULL (contiguous groups) or the act-order group of every input channel;
 *           then each row is stored in group-sorted order (stable sort of k by
 *           g_idx[k]) and that order follows the codes in the buffer
 *   qweight out int32 [w4a16_qweight_words(N, K, g_idx != NULL)]
 * Errors: INVALID_ARG, UNSUPPORTED, BAD_GIDX. */
int w4a16_pack(const uint8_t* codes, const int32_t* g_idx, int group_size, int N, int K,
               int32_t* qweight);

/* Inverse of w4a16_pack (same passages): codes out uint8 [N][K] in the original
 * input-channel order.
 * g_idx must be non-NULL exactly when the buffer was packed with one (only its
 * presence is used; the stored order is read from the buffer and checked).
 * Errors: INVALID_ARG, UNSUPPORTED, BAD_GIDX. */
int w4a16_unpack(const int32_t* qweight, const int32_t* g_idx, int group_size, int N, int K,
                 uint8_t* codes);

/* Zero points: zeros uint8 [G][N] (0..15) <-> qzeros int32 [G][N/8] (layout above).
 * One 4-bit zero point per (group, output row) ("AWQ + GPTQ Quantization, in depth",
 * What W4A16 buys and why decoding gets faster: a 4-bit zero point per group; Z is the
 * integer offset of q = round(x/S) + Z in "LLM Quantization: A Deep Dive...", The Math
 * of Quantization).  Errors: INVALID_ARG. */
int w4a16_pack_zeros(const uint8_t* zeros, int G, int N, int32_t* qzeros);
int w4a16_unpack_zeros(const int32_t* qzeros, int G, int N, uint8_t* zeros);

/* ---------------------------------------------------------------------------------
 * The layer, device memory, asynchronous on `stream`.
 * ------------------------------------------------------------------------------ */

/* y = x * W^T with W^ = (q - Z) * S, fp32 accumulation, y rounded once to binary16:
 * the dequantisation x ~ (q - Z) * S of "LLM Quantization: A Deep Dive into GPTQ, AWQ,
 * and Post-Training Quantization", The Math of Quantization, applied on the fly as in
 * "AWQ + GPTQ Quantization, in depth", What W4A16 buys and why decoding gets faster
 * (load the packed 4-bit weights, expand them to 16 bits in registers with the group's
 * scale and zero point, multiply with the 16-bit activations).
 * All pointers are device pointers.  qzeros NULL selects symmetric weights (every
 * zero point 8, codes from w4a16_quantize_sym; no zero points stored or read).
 * g_idx non-NULL selects the act-order layout
 * (qweight must have been packed with that g_idx; the kernels read the stored order
 * from qweight and gather x through it).  M == 1 runs the split-K GEMV (K <= 65536, at
 * most 512 groups per row and under 2 GB of codes, else the MFMA kernels; rows longer
 * than 8192 channels are split over several wavefronts); 2 <= M <= 32 (under 2 GB of codes)
 * the skinny-batch MFMA kernel (one launch per 16 rows; K > 8192 split over workgroups,
 * fp32 partials in workspace memory, summed by a second kernel); larger M the tiled MFMA
 * GEMM (64-, 128- or 256-row tiles), which under act order first gathers x into
 * workspace memory.  Shapes a kernel cannot take (K not a multiple of 128 for the skinny
 * kernel, of 64 for the large tiles) fall to a smaller tiled MFMA kernel, never to the
 * host.
 * Workspace: only those two paths use one (4 * ks * min(M, 16) * N bytes for ks K slices,
 * resp. 2 * M * K bytes).  It is owned by the library, one per (device, stream), grown
 * with hipMalloc when a call needs more and otherwise reused; no call allocates once its
 * stream's workspace is large enough, and no workspace is ever freed before the process
 * ends (a captured graph may still use it).  Growth is refused (UNSUPPORTED) while the
 * stream is being captured: before capturing such a call, run one of at least the same
 * workspace size eagerly on the capturing stream.  The stream must belong to the current
 * device.
 * Environment (read when the library is loaded and by w4a16_reload_env, never per call):
 * W4A16_DEBUG_CHECKS=1 also validates g_idx (synchronous copy); W4A16_FORCE_PATH=gemv|gemm
 * selects a kernel family (for tests); W4A16_TUNE_* switches force other kernels or tile
 * shapes (parity coverage and measurements only).  W4A16_FORCE_PATH and W4A16_TUNE_* are
 * ignored unless W4A16_TUNE=1 is set too.
 * Errors: INVALID_ARG, UNSUPPORTED, MISALIGNED, BAD_GIDX (debug only), HIP. */
int w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
               const int32_t* qzeros, const int32_t* g_idx, int group_size, int M, int N,
               int K, uint16_t* y, void* stream);

/* w4a16_gemm for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): same arguments, same
 * kernels and bit-identical results, but the scratch memory of the K-split skinny
 * launches and of the act-order gather comes from one fixed 16 MiB array in device
 * memory, a static copy per GPU (held until the process ends), instead of the growing
 * workspace.  The call allocates nothing, ever (its first call on a device resolves the
 * array's address there).  A call whose scratch would exceed 16 MiB (under act order
 * with M > 1, 2 * M * K bytes of gathered activations; for a skinny batch whose K is split
 * over ks slices, 4 * ks * min(M, 16) * N bytes more) is refused with UNSUPPORTED before
 * anything is launched.  Every call on a GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams, or several host
 * threads) race on it and must be serialised by the caller; calls on one stream are
 * ordered and safe.  Errors as w4a16_gemm. */
int w4a16_gemm_noalloc(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
                       const int32_t* qzeros, const int32_t* g_idx, int group_size, int M, int N,
                       int K, uint16_t* y, void* stream);

/* Debug/parity view of the weights: w_out[n][k] = binary16((q - Z) * S) in the
 * original input-channel order ("LLM Quantization: A Deep Dive...", The Math of
 * Quantization: x ~ (q - Z) * S), computed with the same device arithmetic that builds
 * the GEMM's weight operand.  Device pointers; qzeros NULL = symmetric (Z = 8).
 * Errors as w4a16_gemm. */
int w4a16_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                  const int32_t* g_idx, int group_size, int N, int K, uint16_t* w_out,
                  void* stream);

/* Re-reads the W4A16_* environment switches described at w4a16_gemm (they are read
 * once, when the library is loaded).  For tests and measurements; must not run while
 * another thread is inside a device entry point.  Interface only.  Returns W4A16_OK. */
int w4a16_reload_env(void);

/* The round-to-nearest quantiser and packing on the device, for contiguous groups:
 * writes exactly what w4a16_quantize (sym == 0) or w4a16_quantize_sym (sym != 0)
 * followed by w4a16_pack and w4a16_pack_zeros write on the host (every decision taken
 * in binary64 with the same operations), directly into the device buffers.
 *   w         binary16 [N][K] (device);  in_scale binary64 [K] (device) or NULL, must be
 *             positive and finite (not checked)
 *   qweight   out int32 [N][K/8];  scales out binary16 [G][N];  qzeros out int32 [G][N/8]
 *             (unused and may be NULL when sym != 0)
 * Asynchronous on `stream`.  Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int w4a16_quantize_device(const uint16_t* w, int N, int K, int group_size, const double* in_scale,
                          int sym, int32_t* qweight, uint16_t* scales, int32_t* qzeros, void* stream);

/* AWQ scale search ("AWQ + GPTQ Quantization, in depth", The two algorithms,
 * compactly: s = (mean over tokens of |X|) ** alpha for alpha on a grid in [0, 1], loss
 * = norm(W X - Wq X), keep the best).  For every alphas[i]: s = w4a16_awq_scales(xcal,
 * alpha), the layer quantised as w4a16_quantize(w, in_scale = s) does (on the device,
 * w4a16_quantize_device), and
 *   losses[i] = || xcal W^T - binary16(xcal / s) W^_alpha^T ||_F
 * over the T calibration rows, with the reference product on binary16 weights and the
 * candidate on w4a16_gemm (both on the device, fp32 accumulation, binary16 outputs),
 * squared differences summed in fp32 per workgroup and in binary64 in a fixed order.
 * *best = the first index of the smallest loss.  Host inputs w binary16 [N][K], xcal
 * binary16 [T][K]; device memory is allocated for the call and freed before it returns;
 * the work runs on `stream` and the call returns when the losses are on the host.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int w4a16_awq_search(const uint16_t* w, const uint16_t* xcal, int N, int K, int T, int group_size,
                     const double* alphas, int n_alpha, double* losses, int* best, void* stream);

/* GPTQ quantiser ("AWQ + GPTQ Quantization, in depth", The two algorithms, compactly,
 * the GPTQ half and its pseudocode; "How do GPTQ and AWQ differ...", GPTQ: quantize
 * then compensate).  With X = xcal^T (input channels x tokens):
 *   H = 2 X X^T + damp * mean(diag(2 X X^T)) * I,   U = upper Cholesky factor of H^-1
 * then every input channel j in visiting order is rounded on the grid of its group and
 * its error (w_j - w^_j) / U[j][j] is fed to the channels not yet visited through
 * row j of U.  The visiting order is the channel order, or with act_order != 0 the
 * order of w4a16_act_order (descending sum_t X[t][k]^2, exact, ties by ascending k),
 * whose g_idx is written.  A group's grid is the asymmetric one of w4a16_quantize
 * (range including 0, S = smallest binary16 >= (hi - lo) / 15, Z = clamp(round(-lo / S),
 * 0, 15), round half to even), from the group's weights as they stand when its first
 * channel is reached.  Binary64 throughout; the results equal the column-by-column
 * definition up to the rounding of the factorisation and of the blocked updates.
 *   w       binary16 [N][K] (host);  xcal binary16 [T][K] (host);  damp >= 0 (0.01 is
 *           typical)
 *   codes   out uint8 [N][K], original channel order;  scales out binary16 [G][N];
 *   zeros   out uint8 [G][N];  g_idx out int32 [K] (act_order != 0; may be NULL
 *           otherwise)
 * Pack with w4a16_pack / w4a16_pack_zeros (passing g_idx under act order).  Device
 * memory (about 8 (N K + T K + 2 K^2) bytes) is allocated for the call and freed before
 * it returns; the work runs on `stream`; the call returns when the outputs are on the
 * host.  Errors: INVALID_ARG (also when the damped H is not positive definite),
 * UNSUPPORTED, HIP. */
int w4a16_gptq(const uint16_t* w, const uint16_t* xcal, int N, int K, int T, int group_size, int act_order,
               double damp, uint8_t* codes, uint16_t* scales, uint8_t* zeros, int32_t* g_idx, void* stream);

/* ---------------------------------------------------------------------------------
 * 8-bit weights (W8A16): the same layer with 256-level codes ("AWQ + GPTQ
 * Quantization, in depth", 4-bit bigger or 8-bit smaller).  Same conventions,
 * shapes, error codes and act order as above; codes and zero points are bytes.
 *   qweight  int32 buffer of w8a16_qweight_words(N, K, act_order) words (private
 *            layout: four codes per word; the act-order tail as above)
 *   qzeros   int32 [G][N/4] or NULL (symmetric: every zero point 128): zero point of
 *            (group, n) in bits 8j..8j+7 of word [group][n/4], j = n % 4
 * ------------------------------------------------------------------------------ */

size_t w8a16_qweight_words(int N, int K, int act_order);

/* Asymmetric round-to-nearest on 256 levels: as w4a16_quantize with 255 for 15
 * (S = smallest binary16 >= (w_hi - w_lo) / 255, Z and q clamped to [0, 255]).
 * Errors as w4a16_quantize. */
int w8a16_quantize(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                   const double* in_scale, uint8_t* codes, uint16_t* scales, uint8_t* zeros);

/* Symmetric: the int8 absmax scheme of "LLM Quantization: INT8, GPTQ, and AWQ
 * Explained", What quantization actually does, per group: S = smallest binary16 >=
 * max |w| / 127, q = clamp(round(w / S), -127, 127), codes = q + 128 (1 .. 255); pass
 * qzeros = NULL to the device calls.  Errors as w4a16_quantize. */
int w8a16_quantize_sym(const uint16_t* w, int N, int K, int group_size, const int32_t* g_idx,
                       const double* in_scale, uint8_t* codes, uint16_t* scales);

/* Pack / unpack codes uint8 [N][K] (0..255) to / from the 8-bit weight buffer; g_idx as
 * for w4a16_pack.  Errors: INVALID_ARG, UNSUPPORTED, BAD_GIDX. */
int w8a16_pack(const uint8_t* codes, const int32_t* g_idx, int group_size, int N, int K,
               int32_t* qweight);
int w8a16_unpack(const int32_t* qweight, const int32_t* g_idx, int group_size, int N, int K,
                 uint8_t* codes);

/* Zero points: zeros uint8 [G][N] <-> qzeros int32 [G][N/4].  Errors: INVALID_ARG. */
int w8a16_pack_zeros(const uint8_t* zeros, int G, int N, int32_t* qzeros);
int w8a16_unpack_zeros(const int32_t* qzeros, int G, int N, uint8_t* zeros);

/* y = x * W^T for 8-bit weights, device memory, asynchronous on `stream`.  M == 1
 * runs the split-K GEMV (K <= 32768, at most 512 groups per row, N*K < 2^31), larger M
 * the skinny and tiled MFMA kernels (act order at M > 1: x gathered into the
 * workspace first, which works as for w4a16_gemm).  qzeros NULL = symmetric.  Errors as
 * w4a16_gemm. */
int w8a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales,
               const int32_t* qzeros, const int32_t* g_idx, int group_size, int M, int N,
               int K, uint16_t* y, void* stream);

/* binary16((q - Z) * S) of an 8-bit weight buffer, [N][K] in the original channel
 * order (debug/parity view).  Errors as w4a16_gemm. */
int w8a16_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                  const int32_t* g_idx, int group_size, int N, int K, uint16_t* w_out,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
