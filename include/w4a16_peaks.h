/* Achievable-peak probes of the part the library runs on (a separate library,
 * libw4a16_peaks.so, used by the bench to put the measured rates of the W4A16
 * kernels beside what the hardware sustains on plain streams and MFMA loops).
 *
 * Both calls launch one kernel on `stream` (a hipStream_t; NULL = the default
 * stream) and return at once; time them with events on that stream.  They allocate
 * nothing.  Return value: 0 on success, 1 for an invalid argument, 5 for a launch
 * error (text from w4a16_peaks_last_error, thread-local).
 */
#ifndef W4A16_PEAKS_H
#define W4A16_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: every 16-byte chunk of the device buffer `buf` (`bytes` > 0, a
 * multiple of 16, at most 2^31 - 16; 16-byte aligned) is loaded once with
 * non-temporal 16-byte loads by a grid of `blocks` workgroups of 512 threads
 * (grid-stride over the chunks, four loads in flight per thread).  The XOR of each
 * thread's words goes to out[blocks * 512] (device memory), so no load is dead. */
int w4a16_peak_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, void* stream);

/* MFMA loop: `blocks` workgroups of 8 wavefronts (one per compute unit: each takes
 * 96 KB of LDS), every wavefront running `iters` rounds of four independent
 * v_mfma_f32_32x32x16_f16 accumulation chains (32768 flops each) from registers.
 * Flops per launch: blocks * 8 * iters * 4 * 32768.  One float per thread goes to
 * out[blocks * 512] (device memory). */
int w4a16_peak_mfma_f16(float* out, int iters, int blocks, void* stream);

const char* w4a16_peaks_last_error(void);

#ifdef __cplusplus
}
#endif

#endif
