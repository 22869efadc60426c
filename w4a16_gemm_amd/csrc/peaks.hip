// Achievable-peak probes: a plain streaming read and an MFMA loop, timed by the
// bench beside the W4A16 kernels (include/w4a16_peaks.h).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "w4a16_peaks.h"

namespace {

thread_local char g_error[256] = "";

int fail(int code, const char* msg) {
  snprintf(g_error, sizeof g_error, "%s", msg);
  return code;
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kUnroll = 4;
constexpr size_t kMfmaLds = 96 * 1024;   // one workgroup per compute unit

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4_t* __restrict__ buf, long long chunks,
                                                               uint32_t* __restrict__ out) {
  const long long stride = static_cast<long long>(gridDim.x) * kThreads;
  long long c = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; c + (kUnroll - 1) * stride < chunks; c += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + c + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; c < chunks; c += stride) {
    const u32x4_t v = __builtin_nontemporal_load(buf + c);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void mfma_loop_kernel(float* __restrict__ out, int iters) {
  extern __shared__ unsigned char lds[];   // occupancy only
  const int t = threadIdx.x;
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<_Float16>(((t + i) & 7) * 0.01f);
    b[i] = static_cast<_Float16>(((3 * t + i) & 7) * 0.01f);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) s += acc[j][0] + acc[j][15];
  if (t == 0) lds[0] = 0;
  out[static_cast<size_t>(blockIdx.x) * kThreads + t] = s;
}

}  // namespace

extern "C" {

int w4a16_peak_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, void* stream) {
  g_error[0] = '\0';
  if (!buf || !out || blocks <= 0 || bytes == 0 || bytes % 16 != 0 || bytes > (size_t{1} << 31) - 16 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(1, "stream read: NULL pointer, blocks <= 0, or bytes not a positive multiple of 16 below 2^31");
  (void)hipGetLastError();   // the launch check below reports this launch, not an earlier call's failure
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4_t*>(buf), static_cast<long long>(bytes / 16), out);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : fail(5, hipGetErrorString(e));
}

int w4a16_peak_mfma_f16(float* out, int iters, int blocks, void* stream) {
  g_error[0] = '\0';
  if (!out || iters <= 0 || blocks <= 0) return fail(1, "mfma loop: NULL output, iters <= 0 or blocks <= 0");
  static const hipError_t lds_ok = hipFuncSetAttribute(reinterpret_cast<const void*>(mfma_loop_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(kMfmaLds));
  if (lds_ok != hipSuccess) return fail(5, hipGetErrorString(lds_ok));
  (void)hipGetLastError();
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(kThreads), kMfmaLds, static_cast<hipStream_t>(stream),
                     out, iters);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : fail(5, hipGetErrorString(e));
}

const char* w4a16_peaks_last_error(void) { return g_error; }

}  // extern "C"
