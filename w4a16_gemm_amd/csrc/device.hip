// Device entry points of the W4A16 library: argument checks, kernel selection and
// launches.  Every launch is asynchronous on the caller's stream; launch errors are
// reported as W4A16_ERR_HIP with the HIP error text.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.hpp"
#include "kernels/aux.hpp"
#include "kernels/gemm.hpp"
#include "kernels/gemv.hpp"
#include "kernels/gptq.hpp"
#include "kernels/quantize.hpp"
#include "kernels/skinny.hpp"

namespace w4a16 {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Group of input channel k: k >> gshift.  Groups of 32 / 64 / 128 channels, or one
// group per row (g = K, any multiple of 32): a shift that sends every channel to group 0.
constexpr int kPerChannelShift = 30;
int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 128 ? 7 : kPerChannelShift; }

// Groups covering channels [k0, k0 + len) (len > 0).
int groups_in(int k0, int len, int gshift) { return ((k0 + len - 1) >> gshift) - (k0 >> gshift) + 1; }

int env_int(const char* name, int fallback) {
  const char* v = std::getenv(name);
  if (!v || !*v) return fallback;
  return std::atoi(v);
}

enum class Path { kAuto, kGemv, kGemm };

// Environment switches, read once per process (at the first device call, or again by
// w4a16_reload_env), never on the per-call path.  All but debug_checks and force_path
// only force alternative kernels or tile shapes, for parity coverage and measurements.
struct Knobs {
  int debug_checks = 0;         // W4A16_DEBUG_CHECKS: validate g_idx (synchronous)
  Path force_path = Path::kAuto;   // W4A16_FORCE_PATH=gemv|gemm
  int gemv_lpr = 0;             // W4A16_TUNE_GEMV_LPR: lanes per row of the GEMV
  int gemv_blocks_per_cu = 1;   // W4A16_TUNE_GEMV_BLOCKS_PER_CU
  int gemv_pre = 1;             // W4A16_TUNE_GEMV_PRE: stage all scales once (0 never, 1 when it fits, 2 not compact)
  int gemv_early = 1;           // W4A16_TUNE_GEMV_EARLY: first rows' dot products before the staging barrier
  int gemm_prio = 1;            // W4A16_TUNE_GEMM_PRIO: wavefront priority in the large tiles
  int gemm_mfma32 = 1;          // W4A16_TUNE_GEMM_MFMA32: 32x32 blocks (0 never, 1 small tiles, 2 all)
  int gemm_split = 2;           // W4A16_TUNE_GEMM_SPLIT: two tile widths per launch (1: only within two rounds)
  int gemm_ldsb = 0;            // W4A16_TUNE_GEMM_LDSB: 256-row tiles dequantised once into LDS
  int gemm_big_mb = 0;          // W4A16_TUNE_GEMM_BIG_MB: forced row blocks per wavefront (0 = auto)
  int gemm_big_min_m = 0;       // W4A16_TUNE_GEMM_BIG_MIN_M (0 = default)
  int gemm_big = 1;             // W4A16_TUNE_GEMM_BIG: large-tile kernel allowed
  int skinny_chunk_max_m = 0;   // W4A16_TUNE_SKINNY_CHUNK_MAX_M (0 = default)
  int gemm_skinny = 1;          // W4A16_TUNE_GEMM_SKINNY: skinny kernel allowed
};

// The kernel-choice switches (W4A16_FORCE_PATH, W4A16_TUNE_*) are honoured only when
// W4A16_TUNE=1 is set as well, so that a stray variable in a serving environment cannot
// change which kernels run; W4A16_DEBUG_CHECKS only adds checks and needs no opt-in.
Knobs read_knobs() {
  Knobs k;
  k.debug_checks = env_int("W4A16_DEBUG_CHECKS", 0);
  if (env_int("W4A16_TUNE", 0) != 1) return k;
  const char* v = std::getenv("W4A16_FORCE_PATH");
  if (v && std::strcmp(v, "gemv") == 0) k.force_path = Path::kGemv;
  if (v && std::strcmp(v, "gemm") == 0) k.force_path = Path::kGemm;
  k.gemv_lpr = env_int("W4A16_TUNE_GEMV_LPR", 0);
  k.gemv_blocks_per_cu = env_int("W4A16_TUNE_GEMV_BLOCKS_PER_CU", 1);
  k.gemv_pre = env_int("W4A16_TUNE_GEMV_PRE", 1);
  k.gemv_early = env_int("W4A16_TUNE_GEMV_EARLY", 1);
  k.gemm_prio = env_int("W4A16_TUNE_GEMM_PRIO", 1);
  k.gemm_mfma32 = env_int("W4A16_TUNE_GEMM_MFMA32", 1);
  k.gemm_split = env_int("W4A16_TUNE_GEMM_SPLIT", 2);
  k.gemm_ldsb = env_int("W4A16_TUNE_GEMM_LDSB", 0);
  k.gemm_big_mb = env_int("W4A16_TUNE_GEMM_BIG_MB", 0);
  k.gemm_big_min_m = env_int("W4A16_TUNE_GEMM_BIG_MIN_M", 0);
  k.gemm_big = env_int("W4A16_TUNE_GEMM_BIG", 1);
  k.skinny_chunk_max_m = env_int("W4A16_TUNE_SKINNY_CHUNK_MAX_M", 0);
  k.gemm_skinny = env_int("W4A16_TUNE_GEMM_SKINNY", 1);
  return k;
}

Knobs g_knobs = read_knobs();   // at library load; w4a16_reload_env reads again

const Knobs& knobs() { return g_knobs; }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return W4A16_OK;
  return fail(W4A16_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int check_launch(const char* what) { return hip_status(hipGetLastError(), what); }

// Start of every entry point that launches work: the library's own error cleared, and
// the runtime's last-error state too.  hipGetLastError reports the last failure of any
// runtime call made on the thread, by any component, until it is read; without this, a
// launch check could report an earlier failure of someone else's call as its own.
void begin_call() {
  clear_error();
  (void)hipGetLastError();
}

// --- scratch memory ------------------------------------------------------------
//
// Two layer paths need device memory beyond x, the weights and y: the fp32 partial
// tiles of skinny launches whose K is split over workgroups, and x gathered into the
// stored channel order for act-order batches of more than one row.  The entry point
// decides where it comes from; the kernels only see a pointer.
using ScratchFn = int (*)(hipStream_t st, size_t bytes, void** out);

// w4a16_gemm / w8a16_gemm: a library-owned workspace per (device, stream).  Calls on
// one stream are ordered, so they share it; calls on different streams never do.  It
// grows (by at least 2x) when a call needs more, with hipMalloc on the calling thread,
// which is refused while the stream is being captured into a graph: a captured call
// must follow an eager call of at least the same workspace size on the same stream.  A
// grown-out buffer is kept, not freed, because a captured graph may still use it; the
// memory is held until the process ends (at most twice the largest request per stream).
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;

int workspace_scratch(hipStream_t st, size_t bytes, void** out) {
  int dev = 0;
  if (int rc = hip_status(hipGetDevice(&dev), "hipGetDevice")) return rc;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& ws = g_ws[{dev, reinterpret_cast<uintptr_t>(st)}];
  if (ws.bytes >= bytes) {
    *out = ws.ptr;
    return W4A16_OK;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (int rc = hip_status(hipStreamIsCapturing(st, &cap), "hipStreamIsCapturing")) return rc;
  if (cap != hipStreamCaptureStatusNone)
    return fail(W4A16_ERR_UNSUPPORTED,
                "this call needs %zu bytes of workspace on a stream under graph capture, which holds %zu: "
                "run a call of at least this size on the same stream before capturing",
                bytes, ws.bytes);
  constexpr size_t kGrain = size_t{2} << 20;
  const size_t want = std::max((bytes + kGrain - 1) / kGrain * kGrain, 2 * ws.bytes);
  void* p = nullptr;
  if (int rc = hip_status(hipMalloc(&p, want), "hipMalloc (workspace)")) return rc;
  if (ws.ptr) ws.retired.push_back(ws.ptr);
  ws.ptr = p;
  ws.bytes = want;
  *out = p;
  return W4A16_OK;
}

// Zero points as the kernels take them: NULL qzeros = symmetric (Z = 8 everywhere); the
// kernels' zero-point loads then all read the first word of the scales and ignore it.
Zeros layer_zeros(const int32_t* qzeros, const uint16_t* scales) {
  if (qzeros) return Zeros{reinterpret_cast<const uint32_t*>(qzeros), 0};
  return Zeros{reinterpret_cast<const uint32_t*>(scales), 1};
}

// Same validation for every device entry point.
int check_device_args(const void* const* ptrs, int nptrs, int N, int K, int group_size) {
  for (int i = 0; i < nptrs; ++i)
    if (!ptrs[i]) return fail(W4A16_ERR_INVALID_ARG, "NULL device buffer (argument %d)", i);
  if (int st = check_shape(N, K, group_size)) return st;
  for (int i = 0; i < nptrs; ++i)
    if (!aligned16(ptrs[i])) return fail(W4A16_ERR_MISALIGNED, "device buffer %d is not 16-byte aligned", i);
  return W4A16_OK;
}

// Optional (W4A16_DEBUG_CHECKS=1) check of a device-resident g_idx against the order
// stored in the weight buffer.  Synchronous.
int debug_check_gidx(const int32_t* g_idx, const int32_t* tail_dev, int K, int group_size, hipStream_t stream) {
  if (knobs().debug_checks == 0) return W4A16_OK;
  if (int st = hip_status(hipStreamSynchronize(stream), "hipStreamSynchronize")) return st;
  std::vector<int32_t> h(K), tail(K), perm(K);
  if (int st = hip_status(hipMemcpy(h.data(), g_idx, sizeof(int32_t) * K, hipMemcpyDeviceToHost), "hipMemcpy"))
    return st;
  if (int st = hip_status(hipMemcpy(tail.data(), tail_dev, sizeof(int32_t) * K, hipMemcpyDeviceToHost), "hipMemcpy"))
    return st;
  if (int st = check_gidx_and_sort(h.data(), K, group_size, perm.data())) return st;
  for (int p = 0; p < K; ++p)
    if (tail[p] != perm[p])
      return fail(W4A16_ERR_BAD_GIDX, "g_idx does not match the order stored in qweight at %d", p);
  return W4A16_OK;
}

// w4a16_gemm_noalloc: a fixed array in device memory, one copy per GPU (each GPU that
// runs the entry point holds it until the process ends), shared by every call on that
// GPU.  Calls that overlap on one GPU race on it.  Every byte a call reads from it was
// written earlier by the same call (the gather writes all M x K gathered activations,
// every K slice writes all of its M x N partial sums), so nothing needs clearing.
constexpr size_t kStaticScratchBytes = size_t{16} << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

// The array's device address on each GPU.  In host code `scratch` names a host-side
// stand-in, not device memory: only these addresses may be handed to kernels.
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// Resolves the current device's copy of the array (once per device; the first call of
// the entry point on a device does it before anything else).
int static_scratch_setup(void** out) {
  int dev = 0;
  if (int rc = hip_status(hipGetDevice(&dev), "hipGetDevice")) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(W4A16_ERR_UNSUPPORTED, "device %d beyond the supported %d", dev, kMaxDevices);
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (int rc = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress (scratch)")) return rc;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return W4A16_OK;
}

int static_scratch(hipStream_t, size_t bytes, void** out) {
  if (bytes > kStaticScratchBytes)
    return fail(W4A16_ERR_UNSUPPORTED,
                "this call needs %zu bytes of scratch memory; the no-allocation entry point has %zu "
                "(use w4a16_gemm, whose workspace grows)",
                bytes, kStaticScratchBytes);
  return static_scratch_setup(out);
}

// --- GEMV (M = 1) ---------------------------------------------------------------

constexpr int kGemvWaves = 8;
constexpr size_t kGemvLdsBudget = 144 * 1024;  // of the 160 KB of a gfx950 CU

struct GemvShape {
  int lpr = 0;  // lanes per row
  int cpl = 0;  // 16-byte chunks per lane per row (slice)
  bool exact = false;
  int wpr = 1;  // wavefronts per row: slices of a long row
};

// Lanes per row, chunks per lane and slices for C 16-byte chunks per row (K / 32 at
// 4 bits, K / 16 at 8 bits).  Up to 256 chunks (K <= 8192 at 4 bits): an exact split with the widest rows first, else the widest
// split, at most 4 chunks per lane (more spill the activations out of registers).
// Longer rows: one wavefront per slice, 2, 4 or 8 slices of at most 256 chunks.
GemvShape pick_gemv_shape(int C) {
  if (C <= 256) {
    for (int lpr : {64, 32, 16, 8})
      if (C % lpr == 0 && C / lpr <= 4) return {lpr, C / lpr, true, 1};
    for (int lpr : {64, 32, 16, 8})
      if (lpr <= C || lpr == 8) return {lpr, (C + lpr - 1) / lpr, false, 1};
  }
  for (int wpr : {2, 4, 8}) {
    const int cs = (C + wpr - 1) / wpr;
    if (cs <= 256) return {64, (cs + 63) / 64, C % wpr == 0 && cs % 64 == 0, wpr};
  }
  return {};
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Register-pipeline depth: about 8 KB of codes in flight per wavefront.
constexpr int gemv_depth(int cpl) { return cpl >= 3 ? 2 : 8 / cpl; }

template <int LPR, int CPL, bool EXACT, bool ACT, int EPT, int WPR, int BITS, bool PRE = false, bool CT = false>
int launch_gemv_e(dim3 grid, size_t shmem, hipStream_t st, const half_t* x, const uint32_t* qw,
                   const uint16_t* s, Zeros z, half_t* y, int N, int K, int gshift, int steps) {
  auto kern = gemv_m1_kernel<LPR, CPL, kGemvWaves, gemv_depth(CPL), EXACT, ACT, EPT, WPR, BITS, PRE, CT>;
  // Dynamic LDS above 64 KB has to be allowed per kernel (once per process).
  static const hipError_t lds_ok = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       static_cast<int>(kGemvLdsBudget));
  if (shmem > 64 * 1024)
    if (int rc = hip_status(lds_ok, "hipFuncSetAttribute")) return rc;
  hipLaunchKernelGGL(kern, grid, dim3(kGemvWaves * 64), shmem, st, x, qw, s, z, y, N, K, gshift, steps,
                     knobs().gemv_early != 0 ? 1 : 0);
  return check_launch("gemv launch");
}

// Staging rows per thread: one row (EPT = 1) is compiled only for exact splits
// without act order, the decode shapes of large layers; everything else stages
// whole 8-row items.  ept == 0: every row staged once (PRE).
template <int LPR, int CPL, bool EXACT, bool ACT, int BITS>
int launch_gemv_t(int ept, dim3 grid, size_t shmem, hipStream_t st, const half_t* x, const uint32_t* qw,
                   const uint16_t* s, Zeros z, half_t* y, int N, int K, int gshift, int steps) {
  if (ept == 0)
    return launch_gemv_e<LPR, CPL, EXACT, ACT, 8, 1, BITS, true>(grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
  if constexpr (CPL == 4 && EXACT && BITS == 4 && (LPR == 64 || LPR == 32))
    if (ept == -1)
      return launch_gemv_e<LPR, CPL, EXACT, ACT, 8, 1, BITS, true, true>(grid, shmem, st, x, qw, s, z, y, N, K, gshift,
                                                                         steps);
  if constexpr (EXACT && !ACT)
    if (ept == 1)
      return launch_gemv_e<LPR, CPL, EXACT, ACT, 1, 1, BITS>(grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
  return launch_gemv_e<LPR, CPL, EXACT, ACT, 8, 1, BITS>(grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
}

template <int LPR, bool EXACT, bool ACT, int BITS>
int launch_gemv_cpl(int cpl, int ept, dim3 grid, size_t shmem, hipStream_t st, const half_t* x, const uint32_t* qw,
                     const uint16_t* s, Zeros z, half_t* y, int N, int K, int gshift, int steps) {
  switch (cpl) {
    case 1: return launch_gemv_t<LPR, 1, EXACT, ACT, BITS>(ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    case 2: return launch_gemv_t<LPR, 2, EXACT, ACT, BITS>(ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    case 3: return launch_gemv_t<LPR, 3, EXACT, ACT, BITS>(ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    default: return launch_gemv_t<LPR, 4, EXACT, ACT, BITS>(ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
  }
}

// Split rows (K > 8192): 64 lanes per row slice, 3 or 4 chunks per lane, whole 8-row
// staging items (a row has more than 64 groups); ept == 0: every row staged once (PRE).
template <int WPR, bool EXACT, bool ACT, int BITS>
int launch_gemv_split(int cpl, int ept, dim3 grid, size_t shmem, hipStream_t st, const half_t* x, const uint32_t* qw,
                       const uint16_t* s, Zeros z, half_t* y, int N, int K, int gshift, int steps) {
  if (ept == 0) {
    if (cpl == 3)
      return launch_gemv_e<64, 3, EXACT, ACT, 8, WPR, BITS, true>(grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    return launch_gemv_e<64, 4, EXACT, ACT, 8, WPR, BITS, true>(grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
  }
  if (cpl == 3) return launch_gemv_e<64, 3, EXACT, ACT, 8, WPR, BITS>(grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
  return launch_gemv_e<64, 4, EXACT, ACT, 8, WPR, BITS>(grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
}

template <bool EXACT, bool ACT, int BITS>
int launch_gemv_lpr(const GemvShape& sh, int ept, dim3 grid, size_t shmem, hipStream_t st, const half_t* x,
                     const uint32_t* qw, const uint16_t* s, Zeros z, half_t* y, int N, int K,
                     int gshift, int steps) {
  if (sh.wpr > 1) {
    switch (sh.wpr) {
      case 2: return launch_gemv_split<2, EXACT, ACT, BITS>(sh.cpl, ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
      case 4: return launch_gemv_split<4, EXACT, ACT, BITS>(sh.cpl, ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
      default: return launch_gemv_split<8, EXACT, ACT, BITS>(sh.cpl, ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    }
  }
  switch (sh.lpr) {
    case 64: return launch_gemv_cpl<64, EXACT, ACT, BITS>(sh.cpl, ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    case 32: return launch_gemv_cpl<32, EXACT, ACT, BITS>(sh.cpl, ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    case 16: return launch_gemv_cpl<16, EXACT, ACT, BITS>(sh.cpl, ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
    default: return launch_gemv_cpl<8, EXACT, ACT, BITS>(sh.cpl, ept, grid, shmem, st, x, qw, s, z, y, N, K, gshift, steps);
  }
}

// LDS of one workgroup: the two-slot scale/zero ring (unit rows x (G+1) float2 each),
// the row (slice) results, and the gathered activations under act order.
// pre: the table of all the workgroup's rows instead of the ring.
size_t gemv_lds_bytes(int K, int G, int unit, int steps, int wpr, bool act, bool pre = false, bool ct = false) {
  return (pre ? steps : 2) * static_cast<size_t>(unit) * (G + 1) * (ct ? 1 : 2) * sizeof(float) +
         static_cast<size_t>(steps) * unit * wpr * sizeof(float) + (act ? static_cast<size_t>(K) * sizeof(half_t) : 0);
}

// Launch plan of the GEMV for one layer; ok == false: the GEMV does not take it (the
// caller routes the layer to the MFMA kernels).
struct GemvPlan {
  bool ok = false;
  GemvShape sh;
  int blocks = 0, steps = 0, ept = 8;   // ept 0: every row staged once (PRE); -1: PRE, compact table
  size_t shmem = 0;
};

GemvPlan plan_gemv_for(const GemvShape& sh, int N, int K, int gshift, bool act, int bits);

// The GEMV's launch plan.  Rows of at most 256 chunks: the exact split with the most
// chunks per lane (up to 4) that still gives about 1.5 rounds of row units over the
// compute units, else the default shape of pick_gemv_shape.  Measured at M = 1 (lanes per
// row forced, same process): K = 1024 / 2048 / 4096 rows with enough of them run 18% /
// 16% / 8–11% faster with 4 / 2 / 4 chunks per lane than with the widest exact split,
// and K = 4096 at N = 4096 (one round of 16-row units) 5% slower, hence the row-unit bound.
GemvPlan plan_gemv(int N, int K, int gshift, bool act, int bits = 4) {
  const int C = K / (bits == 4 ? 32 : 16);   // 16-byte chunks per row
  GemvShape sh = pick_gemv_shape(C);
  if (sh.lpr == 0) return GemvPlan{};
  // measurements only: lanes per row forced (rows of at most 256 chunks)
  const int lpr = knobs().gemv_lpr;
  if (sh.wpr == 1 && (lpr == 8 || lpr == 16 || lpr == 32 || lpr == 64) && (C + lpr - 1) / lpr <= 4)
    return plan_gemv_for({lpr, (C + lpr - 1) / lpr, C % lpr == 0, 1}, N, K, gshift, act, bits);
  if (sh.wpr == 1) {
    const int cus = device_cus();
    for (int l : {8, 16, 32}) {
      if (C % l != 0 || C / l > 4 || l >= sh.lpr) continue;
      const long long units = (N + kGemvWaves * (64 / l) - 1) / (kGemvWaves * (64 / l));
      if (2 * units < 3LL * cus) continue;
      const GemvPlan p = plan_gemv_for({l, C / l, true, 1}, N, K, gshift, act, bits);
      if (p.ok) return p;
    }
  }
  return plan_gemv_for(sh, N, K, gshift, act, bits);
}

GemvPlan plan_gemv_for(const GemvShape& sh, int N, int K, int gshift, bool act, int bits) {
  GemvPlan p;
  p.sh = sh;
  if (static_cast<long long>(N) * K * bits / 8 >= (1LL << 31)) return p;   // 32-bit byte offsets into the codes
  const int G = groups_in(0, K, gshift);
  const int unit = kGemvWaves * (64 / p.sh.lpr);                    // rows per unit
  if ((unit / 8) * G > kGemvWaves * 64) return p;                   // one staging item per thread and step
  p.ept = unit * G <= kGemvWaves * 64 ? 1 : 8;                      // staging rows per thread
  const int units = (N + unit - 1) / unit;
  const int per_cu = knobs().gemv_blocks_per_cu;
  p.blocks = std::min(units, std::max(1, device_cus() * std::max(1, per_cu)));
  if (p.blocks >= 8) p.blocks -= p.blocks % 8;                      // whole XCD rounds
  p.steps = (units + p.blocks - 1) / p.blocks;
  while (gemv_lds_bytes(K, G, unit, p.steps, p.sh.wpr, act) > kGemvLdsBudget && p.blocks < units) {
    p.blocks = std::min(units, p.blocks * 2);
    p.steps = (units + p.blocks - 1) / p.blocks;
  }
  p.shmem = gemv_lds_bytes(K, G, unit, p.steps, p.sh.wpr, act);
  p.ok = p.shmem <= kGemvLdsBudget;
  // Staging every row once (PRE): at most two rounds of two 8-row items per thread, and
  // the table within the LDS budget.  The workgroups own consecutive units, so as many
  // workgroups as it takes at `steps` units each (whole XCD rounds when there are
  // enough).  Split rows (K > 8192) too, from three steps on: the table holds whole rows,
  // each slice reads its groups.  Same-process A/B against the per-step ring: N = 8192 at
  // K = 12288, group 64 (4 steps) 12.60 -> 11.66 us, K = 16384 / 28672 (4 steps) -0.5%,
  // but N = 4096, K = 14336 (2 steps) 8.94 -> 9.25 us; 8-bit split rows (K = 8192, N = 28672,
  // 14 steps) 36.08 -> 37.73 us, so those keep the ring.
  if (p.ok && knobs().gemv_pre != 0 && p.steps >= (p.sh.wpr > 1 ? 3 : 2) && (p.sh.wpr == 1 || bits == 4)) {
    int blocks = (units + p.steps - 1) / p.steps;
    if (blocks >= 8) blocks += (8 - blocks % 8) % 8;
    const long long items = static_cast<long long>(p.steps) * (unit / 8) * G;
    const size_t shmem = gemv_lds_bytes(K, G, unit, p.steps, p.sh.wpr, act, true);
    const size_t shmem_ct = gemv_lds_bytes(K, G, unit, p.steps, p.sh.wpr, act, true, true);
    const bool ct_ok = p.sh.wpr == 1 && p.sh.cpl == 4 && p.sh.exact && bits == 4 &&
                       (p.sh.lpr == 64 || p.sh.lpr == 32) && knobs().gemv_pre != 2;
    if (items <= 4LL * kGemvWaves * 64 && shmem <= kGemvLdsBudget) {
      p.blocks = blocks;
      p.ept = 0;
      p.shmem = shmem;
    } else if (ct_ok && items <= 8LL * kGemvWaves * 64 && shmem_ct <= kGemvLdsBudget) {
      // many groups (group 32 on large layers): the compact table, two rounds of four items
      p.blocks = blocks;
      p.ept = -1;
      p.shmem = shmem_ct;
    }
  }
  return p;
}

template <int BITS = 4>
int run_gemv(const GemvPlan& p, bool act, const half_t* x, const uint32_t* qw, const uint16_t* s,
             Zeros z, half_t* y, int N, int K, int gshift, hipStream_t st) {
  const dim3 grid(p.blocks);
  if (p.sh.exact) {
    if (act) return launch_gemv_lpr<true, true, BITS>(p.sh, p.ept, grid, p.shmem, st, x, qw, s, z, y, N, K, gshift, p.steps);
    return launch_gemv_lpr<true, false, BITS>(p.sh, p.ept, grid, p.shmem, st, x, qw, s, z, y, N, K, gshift, p.steps);
  }
  if (act) return launch_gemv_lpr<false, true, BITS>(p.sh, p.ept, grid, p.shmem, st, x, qw, s, z, y, N, K, gshift, p.steps);
  return launch_gemv_lpr<false, false, BITS>(p.sh, p.ept, grid, p.shmem, st, x, qw, s, z, y, N, K, gshift, p.steps);
}

// --- GEMM (M > 1) ---------------------------------------------------------------

template <int BM, int BITS = 4>
void launch_gemm_bm(hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s, Zeros z,
                    half_t* y, int M, int N, int K, int gshift) {
  const dim3 grid((N + 255) / 256, (M + BM - 1) / BM);
  hipLaunchKernelGGL((gemm_mfma_kernel<BM, BITS>), grid, dim3(256), 0, st, x, qw, s, z, y, M, N, K, gshift);
}

// The tiled MFMA kernel with the row-block height for M.
template <int BITS>
int run_gemm_tiled(hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s, Zeros z, half_t* y,
                   int M, int N, int K, int gshift) {
  if (M <= 16)
    launch_gemm_bm<16, BITS>(st, x, qw, s, z, y, M, N, K, gshift);
  else if (M <= 32)
    launch_gemm_bm<32, BITS>(st, x, qw, s, z, y, M, N, K, gshift);
  else if (M <= 64)
    launch_gemm_bm<64, BITS>(st, x, qw, s, z, y, M, N, K, gshift);
  else
    launch_gemm_bm<128, BITS>(st, x, qw, s, z, y, M, N, K, gshift);
  return check_launch("gemm launch");
}

// Skinny-batch kernel shape: W wavefronts of T 128-channel steps (K = 128 T W), SE
// slab entries per thread.  waves == 0: not applicable.
struct SkinnyShape {
  int waves = 0, t = 0, se = 0;
  int ks = 1;   // K slices over the workgroups (fp32 partials summed by a second kernel)
};

constexpr int kSkinnyMaxM = 16;       // rows of one skinny launch (one MFMA column tile)
constexpr int kSkinnyChunkMaxM = 32;  // larger M: tiled GEMM kernels
constexpr int kBigMinM = 33;          // the large-tile kernel from here on (when K allows)

// The whole row in one workgroup when it fits (K <= 8192), else the fewest K slices
// that fit; per slice the most wavefronts (fewest slab entries per thread).
SkinnyShape pick_skinny_shape(int M, int K, int gshift, int bits = 4) {
  SkinnyShape sh;
  if (M > kSkinnyMaxM) return sh;
  for (int ks : {1, 2, 4, 8}) {
    if (K % (128 * ks) != 0) continue;
    const int Ks = K / ks;
    const int kc = Ks / 128;
    for (int t : {1, 2, 4}) {
      if (bits == 8 && t > 2) break;   // 8-bit codes take twice the registers per step
      if (kc % t != 0 || kc / t > 16) continue;
      const int waves = kc / t;
      const int entries = 16 * groups_in(0, Ks, gshift);
      const int se = (entries + 64 * waves - 1) / (64 * waves);
      if (se > 4) break;
      sh.waves = waves;
      sh.t = t;
      sh.se = se <= 1 ? 1 : (se <= 2 ? 2 : 4);
      sh.ks = ks;
      return sh;
    }
  }
  return sh;
}

// ks > 1: partial sums to part [ks][M][N] fp32, then sum_slices_kernel into y.
template <int T, int SE, bool SUB, int BITS = 4>
int launch_skinny_t(const SkinnyShape& sh, hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s,
                    Zeros z, half_t* y, float* part, int M, int N, int K, int gshift) {
  static const hipError_t lds_ok =
      hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_skinny_kernel<T, SE, SUB, BITS>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (int rc = hip_status(lds_ok, "hipFuncSetAttribute")) return rc;
  const size_t lds = skinny_lds_bytes(sh.waves, groups_in(0, K / sh.ks, gshift));
  const int nblk = (N + 15) / 16;
  const int per_cu = std::max(1, 16 / sh.waves);
  const int per_slice = std::min(nblk, std::max(1, device_cus() * per_cu / sh.ks));
  hipLaunchKernelGGL((gemm_skinny_kernel<T, SE, SUB, BITS>), dim3(per_slice * sh.ks), dim3(64 * sh.waves), lds, st, x,
                     qw, s, z, y, part, M, N, K, gshift, sh.ks);
  if (int rc = check_launch("skinny gemm launch")) return rc;
  if (sh.ks == 1) return W4A16_OK;
  const size_t count = static_cast<size_t>(M) * N;
  hipLaunchKernelGGL(sum_slices_kernel, dim3(static_cast<unsigned>((count + 255) / 256)), dim3(256), 0, st, part, y,
                     sh.ks, count);
  return check_launch("slice sum launch");
}

template <int BITS = 4>
int launch_skinny(const SkinnyShape& sh, hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s,
                  Zeros z, half_t* y, float* part, int M, int N, int K, int gshift) {
#define W4A16_SKINNY(T_, SE_)                                                                                    \
  if (sh.t == T_ && sh.se == SE_)                                                                              \
    return gshift == 7 ? launch_skinny_t<T_, SE_, true, BITS>(sh, st, x, qw, s, z, y, part, M, N, K, gshift) \
                       : launch_skinny_t<T_, SE_, false, BITS>(sh, st, x, qw, s, z, y, part, M, N, K, gshift);
  W4A16_SKINNY(1, 1) W4A16_SKINNY(1, 2) W4A16_SKINNY(1, 4)
  W4A16_SKINNY(2, 1) W4A16_SKINNY(2, 2) W4A16_SKINNY(2, 4)
  if constexpr (BITS == 4) {
    W4A16_SKINNY(4, 1) W4A16_SKINNY(4, 2) W4A16_SKINNY(4, 4)
  }
#undef W4A16_SKINNY
  return fail(W4A16_ERR_UNSUPPORTED, "no skinny kernel for T=%d SE=%d", sh.t, sh.se);
}

// The skinny kernel once per 16 rows of x and y.  Scratch (one request, before anything
// is launched): under act order x gathered into the stored channel order (2 M K bytes,
// gather_x_kernel), then the K slices' fp32 partial tiles, reused by the launches of
// every 16 rows.  Gathering inside the kernel instead (each lane's activations read
// through the stored order) spilled its registers: on the act-order layer (K = 4096,
// N = 11008, group 32) M = 2 / 4 / 16 took 19.7 / 22.9 / 42.2 us that way and
// 12.9 / 13.0 / 15.4 us with the separate gather.
template <int BITS>
int run_skinny(const SkinnyShape& sk, bool act, hipStream_t st, const half_t* hx, const uint32_t* hq,
               const half_t* hs, Zeros hz, half_t* hy, int M, int N, int K, int gshift, ScratchFn scratch) {
  const size_t xs_bytes = act ? (static_cast<size_t>(M) * K * sizeof(half_t) + 255) / 256 * 256 : 0;
  const size_t part_bytes = sk.ks > 1 ? static_cast<size_t>(sk.ks) * std::min(M, kSkinnyMaxM) * N * sizeof(float) : 0;
  unsigned char* base = nullptr;
  if (xs_bytes + part_bytes > 0)
    if (int rc = scratch(st, xs_bytes + part_bytes, reinterpret_cast<void**>(&base))) return rc;
  float* part = part_bytes > 0 ? reinterpret_cast<float*>(base + xs_bytes) : nullptr;
  const half_t* x = hx;
  if (act) {
    const auto* perm = reinterpret_cast<const int32_t*>(hq + static_cast<size_t>(N) * (K >> (BITS == 4 ? 3 : 2)));
    auto* xs = reinterpret_cast<half_t*>(base);
    hipLaunchKernelGGL(gather_x_kernel, dim3(static_cast<unsigned>((K / 8 + 255) / 256), std::min(M, kGatherRowsY)),
                       dim3(256), 0, st, hx, perm, xs, M, K);
    if (int rc = check_launch("gather launch")) return rc;
    x = xs;
  }
  int rc = W4A16_OK;
  for (int m0 = 0; m0 < M && rc == W4A16_OK; m0 += kSkinnyMaxM) {
    const int mc = std::min(kSkinnyMaxM, M - m0);
    rc = launch_skinny<BITS>(sk, st, x + static_cast<size_t>(m0) * K, hq, hs, hz, hy + static_cast<size_t>(m0) * N,
                             part, mc, N, K, gshift);
  }
  return rc;
}


// Large-M GEMM.  BM x 256 tiles (BM = 256 rows; 128 or 64 when the whole batch fits in
// fewer rows, so that small batches do not pay for padding rows), except (a) when the
// last round of workgroups over the compute units would be partly idle: then whole
// rounds of full-width tiles cover the first columns and one round of narrower tiles
// (64 NB2 wide) the rest, so that no round leaves compute units idle (the 2048-row
// prefill: one round of each; 4096 rows, K = 4096, N = 14336: three rounds of full tiles
// and one of 256 x 128, 468.8 -> 440.1 us against 3.5 rounds of full tiles, same-process
// A/B; W4A16_TUNE_GEMM_SPLIT=1 splits only within two rounds); (b) when they would not
// fill one round: then narrower tiles for all columns.
// Wavefronts raise their priority (s_setprio 1) for each MFMA cluster and drop it after
// (W4A16_TUNE_GEMM_PRIO=0: off), so that the two wavefronts of a SIMD drift into opposite
// phases, one issuing MFMAs while the other reads LDS and dequantises.  Same-process A/B
// (order alternated, identical outputs): M = 100 / 200 / 300 on the 32x32 tile 49.9 / 27.1 /
// 50.2 -> 46.1 / 25.2 / 46.3 us; 256-row tiles M = 4096 485 -> 472 us, the act-order layer
// at M = 512 78.3 -> 73.8 us, the prefill ~1.5%.
template <int NB2, int MB, int BITS, bool W32, bool LDSB = false>
int launch_big_t(hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s, Zeros z, half_t* y,
                 int M, int N, int K, int gshift, int split, int n_split, int grid) {
  constexpr size_t lds = LDSB ? kLdsbLds : BITS == 4 ? kBigLds : kBigLds8;
  static const hipError_t lds_ok = hipFuncSetAttribute(
      reinterpret_cast<const void*>(gemm_big_kernel<NB2, MB, BITS, W32, LDSB>),
      hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (int rc = hip_status(lds_ok, "hipFuncSetAttribute")) return rc;
  hipLaunchKernelGGL((gemm_big_kernel<NB2, MB, BITS, W32, LDSB>), dim3(grid), dim3(512), lds, st, x, qw, s, z, y, M,
                     N, K, gshift, split, n_split, knobs().gemm_prio);
  return check_launch("gemm launch");
}

// 64- and 128-row tiles of 4-bit weights run the 32x32x16 MFMA tile (W4A16_TUNE_GEMM_MFMA32=0:
// the 16x16x32 one; 2: the 32x32x16 one at every tile height).  Same-process A/B on random layers: M = 100 (K 4096, N 14336) 46.0 -> 40.1 us,
// M = 200 (K 2048, N 4096) 24.8 -> 22.4 us, M = 48 36.5 -> 35.1 us; with 256-row tiles it measured
// no faster (M = 2048 237 vs 239 us, M = 4096 459 vs 480 us), so those keep the 16x16x32 tile.
template <int NB2, int MB, int BITS>
int launch_big(hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s, Zeros z, half_t* y,
               int M, int N, int K, int gshift, int split, int n_split, int grid) {
  if constexpr (BITS == 4) {
    const int mode = knobs().gemm_mfma32;
    if (mode == 2 || (mode == 1 && MB <= 4))
      return launch_big_t<NB2, MB, BITS, true>(st, x, qw, s, z, y, M, N, K, gshift, split, n_split, grid);
    // measurements: the dequantise-once tile (W4A16_TUNE_GEMM_LDSB=1)
    if constexpr (MB == 8)
      if (knobs().gemm_ldsb != 0)
        return launch_big_t<NB2, MB, BITS, false, true>(st, x, qw, s, z, y, M, N, K, gshift, split, n_split, grid);
  }
  return launch_big_t<NB2, MB, BITS, false>(st, x, qw, s, z, y, M, N, K, gshift, split, n_split, grid);
}

template <int MB, int BITS>
int run_gemm_big_t(hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s, Zeros z,
                   half_t* y, int M, int N, int K, int gshift) {
  constexpr int BM = 32 * MB;
  const int tiles_m = (M + BM - 1) / BM;
  const int cus = device_cus();
  const int full = tiles_m * ((N + 255) / 256);
  if (full > cus && cus % tiles_m == 0 && knobs().gemm_split != 0) {
    const int per_panel = cus / tiles_m;                        // column tiles per row panel and round
    const int rounds = full <= 2 * cus || knobs().gemm_split == 1 ? 1 : ((N + 255) / 256) / per_panel;
    const int n_split = 256 * per_panel * rounds;
    const int rest = N - n_split;
    const int nb2 = (((rest + per_panel - 1) / per_panel) + 63) / 64;   // 64-column blocks per narrow tile
    if (rest > 0 && nb2 >= 1 && nb2 <= 3) {
      const int split = tiles_m * per_panel * rounds;   // full-width tiles: columns [0, n_split)
      const int grid = split + tiles_m * ((rest + 64 * nb2 - 1) / (64 * nb2));
      if (nb2 == 1) return launch_big<1, MB, BITS>(st, x, qw, s, z, y, M, N, K, gshift, split, n_split, grid);
      if (nb2 == 2) return launch_big<2, MB, BITS>(st, x, qw, s, z, y, M, N, K, gshift, split, n_split, grid);
      return launch_big<3, MB, BITS>(st, x, qw, s, z, y, M, N, K, gshift, split, n_split, grid);
    }
  }
  // One round or less: the narrowest tiles that still fit in one round keep the most
  // compute units busy (a BM x 128 tile takes about half as long as a BM x 256 one).
  if (full < cus && knobs().gemm_split != 0) {
    for (int nb : {2, 3}) {
      const int tiles = tiles_m * ((N + 64 * nb - 1) / (64 * nb));
      if (tiles <= cus)
        return nb == 2 ? launch_big<2, MB, BITS>(st, x, qw, s, z, y, M, N, K, gshift, 0, 0, tiles)
                       : launch_big<3, MB, BITS>(st, x, qw, s, z, y, M, N, K, gshift, 0, 0, tiles);
    }
  }
  return launch_big<3, MB, BITS>(st, x, qw, s, z, y, M, N, K, gshift, full, N, full);
}

// Output elements one compute unit works through with BM = 32 MB row tiles, following
// the tile choice of run_gemm_big_t (the busiest unit).
long long big_work_per_cu(int MB, int M, int N, int cus) {
  const long long BM = 32LL * MB;
  const int tiles_m = static_cast<int>((M + BM - 1) / BM);
  const int full = tiles_m * ((N + 255) / 256);
  if (full > cus && cus % tiles_m == 0) {
    const int per_panel = cus / tiles_m;
    const int rounds = full <= 2 * cus || knobs().gemm_split == 1 ? 1 : ((N + 255) / 256) / per_panel;
    const int rest = N - 256 * per_panel * rounds;
    const int nb2 = (((rest + per_panel - 1) / per_panel) + 63) / 64;
    if (rest > 0 && nb2 >= 1 && nb2 <= 3) return rounds * BM * 256 + BM * 64 * nb2;
  }
  if (full < cus)
    for (int nb : {2, 3})
      if (tiles_m * ((N + 64 * nb - 1) / (64 * nb)) <= cus) return BM * 64 * nb;
  return static_cast<long long>((full + cus - 1) / cus) * BM * 256;
}

template <int BITS>
int run_gemm_big(hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s, Zeros z, half_t* y,
                 int M, int N, int K, int gshift) {
  // Above 128 rows: 128-row tiles when their smaller tiles fill the device enough better
  // to make up for doing ~1.28x the work per output (twice the dequantisation per MFMA;
  // measured: the 2048-row layer 351 vs 241 us at 0.88x the work per unit).
  int mb_auto = M <= 64 ? 2 : M <= 128 ? 4 : 8;
  if (mb_auto == 8 && knobs().gemm_split != 0) {
    const int cus = device_cus();
    if (static_cast<double>(big_work_per_cu(4, M, N, cus)) * 1.28 < static_cast<double>(big_work_per_cu(8, M, N, cus)))
      mb_auto = 4;
  }
  const int mb = knobs().gemm_big_mb != 0 ? knobs().gemm_big_mb : mb_auto;
  if (mb == 2) return run_gemm_big_t<2, BITS>(st, x, qw, s, z, y, M, N, K, gshift);
  if (mb == 4) return run_gemm_big_t<4, BITS>(st, x, qw, s, z, y, M, N, K, gshift);
  return run_gemm_big_t<8, BITS>(st, x, qw, s, z, y, M, N, K, gshift);
}

// Batches past the skinny kernel: the large-tile kernel where its 32-bit element offsets
// and load widths allow (K % 64 == 0; 8-bit weights also N % 16 == 0 for the 16-byte
// zero-point loads), else the tiled kernel.
template <int BITS>
int run_gemm(hipStream_t st, const half_t* x, const uint32_t* qw, const half_t* s, Zeros z,
             half_t* y, int M, int N, int K, int gshift) {
  if (M >= (knobs().gemm_big_min_m > 0 ? knobs().gemm_big_min_m : kBigMinM) && K % kBigBK == 0 &&
      (BITS == 4 || N % 16 == 0) && static_cast<long long>(M) * K < (1LL << 31) &&
      static_cast<long long>(N) * (K / 32 * BITS) < (1LL << 31) && knobs().gemm_big != 0)
    return run_gemm_big<BITS>(st, x, qw, s, z, y, M, N, K, gshift);
  return run_gemm_tiled<BITS>(st, x, qw, s, z, y, M, N, K, gshift);
}

// Act order above the skinny batches: x gathered into the stored channel order in
// scratch memory, then the plain GEMM on the gathered rows.
template <int BITS>
int run_gemm_act(hipStream_t st, const half_t* hx, const uint32_t* hq, const int32_t* perm, const half_t* hs,
                 Zeros hz, half_t* hy, int M, int N, int K, int gshift, ScratchFn scratch) {
  half_t* xs = nullptr;
  if (int rc = scratch(st, static_cast<size_t>(M) * K * sizeof(half_t), reinterpret_cast<void**>(&xs))) return rc;
  hipLaunchKernelGGL(gather_x_kernel, dim3(static_cast<unsigned>((K / 8 + 255) / 256), std::min(M, kGatherRowsY)),
                     dim3(256), 0, st, hx, perm, xs, M, K);
  if (int rc = check_launch("gather launch")) return rc;
  return run_gemm<BITS>(st, xs, hq, hs, hz, hy, M, N, K, gshift);
}

// The 4-bit layer call; `scratch` provides the memory of the K-split skinny launches and
// of the act-order gather.
int gemm4(const uint16_t* x, const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
          const int32_t* g_idx, int group_size, int M, int N, int K, uint16_t* y, void* stream, ScratchFn scratch) {
  if (M <= 0) return fail(W4A16_ERR_INVALID_ARG, "M must be positive (M=%d)", M);
  const void* ptrs[] = {x, qweight, scales, y, qzeros};   // qzeros may be NULL: symmetric
  if (int st = check_device_args(ptrs, qzeros ? 5 : 4, N, K, group_size)) return st;
  const bool act = g_idx != nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act)
    if (int s = debug_check_gidx(g_idx, qweight + qweight_words(N, K, false), K, group_size, st)) return s;

  const int gshift = log2_group(group_size);
  const auto* hx = reinterpret_cast<const half_t*>(x);
  const auto* hq = reinterpret_cast<const uint32_t*>(qweight);
  const auto* hs = reinterpret_cast<const half_t*>(scales);
  const Zeros hz = layer_zeros(qzeros, scales);
  auto* hy = reinterpret_cast<half_t*>(y);

  const Path forced = knobs().force_path;
  const GemvPlan gp = M == 1 ? plan_gemv(N, K, gshift, act) : GemvPlan{};
  if (forced == Path::kGemv && !gp.ok)
    return fail(W4A16_ERR_UNSUPPORTED,
                "the GEMV path needs M == 1, K <= 65536, N*K/2 < 2^31 and at most 512 groups per row "
                "(M=%d N=%d K=%d group_size=%d)",
                M, N, K, group_size);
  if (gp.ok && forced != Path::kGemm)
    return run_gemv(gp, act, hx, hq, reinterpret_cast<const uint16_t*>(scales), hz, hy, N, K, gshift, st);

  // Up to kSkinnyChunkMaxM rows: the skinny kernel once per 16 rows of x and y.  Every
  // launch streams the whole weight matrix again, so from three launches on the
  // large-tile kernel with 64-row tiles is faster.
  // (The skinny kernel, like the GEMV, addresses the codes with 32-bit byte offsets.)
  const SkinnyShape sk = pick_skinny_shape(std::min(M, kSkinnyMaxM), K, gshift);
  if (sk.waves != 0 && static_cast<long long>(N) * K / 2 < (1LL << 31) &&
      M <= (knobs().skinny_chunk_max_m > 0 ? knobs().skinny_chunk_max_m : kSkinnyChunkMaxM) &&
      knobs().gemm_skinny != 0) {
    return run_skinny<4>(sk, act, st, hx, hq, hs, hz, hy, M, N, K, gshift, scratch);
  }

  if (!act) return run_gemm<4>(st, hx, hq, hs, hz, hy, M, N, K, gshift);
  return run_gemm_act<4>(st, hx, hq, qweight + qweight_words(N, K, false), hs, hz, hy, M, N, K, gshift, scratch);
}

}  // namespace
}  // namespace w4a16

using namespace w4a16;

extern "C" {

int w4a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
               const int32_t* g_idx, int group_size, int M, int N, int K, uint16_t* y, void* stream) {
  begin_call();
  return gemm4(x, qweight, scales, qzeros, g_idx, group_size, M, N, K, y, stream, workspace_scratch);
}

int w4a16_gemm_noalloc(const uint16_t* x, const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
                       const int32_t* g_idx, int group_size, int M, int N, int K, uint16_t* y, void* stream) {
  begin_call();
  void* unused = nullptr;
  if (int rc = static_scratch_setup(&unused)) return rc;
  return gemm4(x, qweight, scales, qzeros, g_idx, group_size, M, N, K, y, stream, static_scratch);
}

int w4a16_reload_env(void) {
  g_knobs = read_knobs();
  return W4A16_OK;
}

int w4a16_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros, const int32_t* g_idx,
                  int group_size, int N, int K, uint16_t* w_out, void* stream) {
  begin_call();
  const void* ptrs[] = {qweight, scales, w_out, qzeros};   // qzeros may be NULL: symmetric
  if (int st = check_device_args(ptrs, qzeros ? 4 : 3, N, K, group_size)) return st;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool act = g_idx != nullptr;
  if (act)
    if (int s = debug_check_gidx(g_idx, qweight + qweight_words(N, K, false), K, group_size, st)) return s;
  const size_t words = static_cast<size_t>(N) * (K / 8);
  const dim3 grid(static_cast<unsigned>((words + 255) / 256));
  const auto* hq = reinterpret_cast<const uint32_t*>(qweight);
  const auto* hs = reinterpret_cast<const half_t*>(scales);
  const Zeros hz = layer_zeros(qzeros, scales);
  auto* hw = reinterpret_cast<half_t*>(w_out);
  const int gshift = log2_group(group_size);
  if (act)
    hipLaunchKernelGGL(dequant_kernel<true>, grid, dim3(256), 0, st, hq, hs, hz, hw, N, K, gshift);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, grid, dim3(256), 0, st, hq, hs, hz, hw, N, K, gshift);
  return check_launch("dequant launch");
}

// 8-bit weights ("AWQ + GPTQ Quantization, in depth", 4-bit bigger or 8-bit smaller):
// M == 1 on the GEMV, up to 32 rows on the skinny kernel, larger batches on the
// large-tile kernel (the tiled MFMA kernel where its conditions do not hold).
int w8a16_gemm(const uint16_t* x, const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros,
               const int32_t* g_idx, int group_size, int M, int N, int K, uint16_t* y, void* stream) {
  begin_call();
  if (M <= 0) return fail(W4A16_ERR_INVALID_ARG, "M must be positive (M=%d)", M);
  const void* ptrs[] = {x, qweight, scales, y, qzeros};   // qzeros may be NULL: symmetric
  if (int st = check_device_args(ptrs, qzeros ? 5 : 4, N, K, group_size)) return st;
  const bool act = g_idx != nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act)
    if (int s = debug_check_gidx(g_idx, qweight + qweight8_words(N, K, false), K, group_size, st)) return s;
  const int gshift = log2_group(group_size);
  const auto* hx = reinterpret_cast<const half_t*>(x);
  const auto* hq = reinterpret_cast<const uint32_t*>(qweight);
  const auto* hs = reinterpret_cast<const half_t*>(scales);
  const Zeros hz = layer_zeros(qzeros, scales);
  auto* hy = reinterpret_cast<half_t*>(y);

  const Path forced = knobs().force_path;
  const GemvPlan gp = M == 1 ? plan_gemv(N, K, gshift, act, 8) : GemvPlan{};
  if (forced == Path::kGemv && !gp.ok)
    return fail(W4A16_ERR_UNSUPPORTED,
                "the 8-bit GEMV path needs M == 1, K <= 32768, N*K < 2^31 and at most 512 groups per row "
                "(M=%d N=%d K=%d group_size=%d)",
                M, N, K, group_size);
  if (gp.ok && forced != Path::kGemm)
    return run_gemv<8>(gp, act, hx, hq, reinterpret_cast<const uint16_t*>(scales), hz, hy, N, K, gshift, st);
  // up to kSkinnyChunkMaxM rows: the skinny kernel (32-bit byte offsets into the codes)
  const SkinnyShape sk = pick_skinny_shape(std::min(M, kSkinnyMaxM), K, gshift, 8);
  if (sk.waves != 0 && static_cast<long long>(N) * K < (1LL << 31) && M <= kSkinnyChunkMaxM &&
      knobs().gemm_skinny != 0)
    return run_skinny<8>(sk, act, st, hx, hq, hs, hz, hy, M, N, K, gshift, workspace_scratch);
  if (static_cast<long long>(M) * K >= (1LL << 31) || static_cast<long long>(N) * (K / 4) >= (1LL << 31))
    return fail(W4A16_ERR_UNSUPPORTED, "8-bit layer too large for 32-bit element offsets (M=%d N=%d K=%d)", M, N, K);
  if (!act) return run_gemm<8>(st, hx, hq, hs, hz, hy, M, N, K, gshift);
  return run_gemm_act<8>(st, hx, hq, qweight + qweight8_words(N, K, false), hs, hz, hy, M, N, K, gshift,
                         workspace_scratch);
}

int w8a16_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros, const int32_t* g_idx,
                  int group_size, int N, int K, uint16_t* w_out, void* stream) {
  begin_call();
  const void* ptrs[] = {qweight, scales, w_out, qzeros};   // qzeros may be NULL: symmetric
  if (int st = check_device_args(ptrs, qzeros ? 4 : 3, N, K, group_size)) return st;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool act = g_idx != nullptr;
  if (act)
    if (int s = debug_check_gidx(g_idx, qweight + qweight8_words(N, K, false), K, group_size, st)) return s;
  const size_t words = static_cast<size_t>(N) * (K / 4);
  const dim3 grid(static_cast<unsigned>((words + 255) / 256));
  const auto* hq = reinterpret_cast<const uint32_t*>(qweight);
  const auto* hs = reinterpret_cast<const half_t*>(scales);
  const Zeros hz = layer_zeros(qzeros, scales);
  auto* hw = reinterpret_cast<half_t*>(w_out);
  const int gshift = log2_group(group_size);
  if (act)
    hipLaunchKernelGGL(dequant8_kernel<true>, grid, dim3(256), 0, st, hq, hs, hz, hw, N, K, gshift);
  else
    hipLaunchKernelGGL(dequant8_kernel<false>, grid, dim3(256), 0, st, hq, hs, hz, hw, N, K, gshift);
  return check_launch("dequant launch");
}

int w4a16_quantize_device(const uint16_t* w, int N, int K, int group_size, const double* in_scale, int sym,
                          int32_t* qweight, uint16_t* scales, int32_t* qzeros, void* stream) {
  begin_call();
  if (!w || !qweight || !scales || (!sym && !qzeros)) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (int rc = check_shape(N, K, group_size)) return rc;
  const long long threads = static_cast<long long>(N) * (K / group_size);
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto* qw = reinterpret_cast<uint32_t*>(qweight);
  auto* qz = reinterpret_cast<uint32_t*>(qzeros);
  if (sym)
    hipLaunchKernelGGL(quantize_rtn_kernel<true>, grid, dim3(256), 0, st, w, in_scale, N, K, group_size, qw, scales, qz);
  else
    hipLaunchKernelGGL(quantize_rtn_kernel<false>, grid, dim3(256), 0, st, w, in_scale, N, K, group_size, qw, scales,
                       qz);
  return check_launch("quantize launch");
}

// AWQ alpha search: the W4A16 GEMM of every candidate against the binary16 product of
// the unquantised layer, on the calibration activations.  Host inputs, device work on
// `stream`, returns when the losses are on the host.
int w4a16_awq_search(const uint16_t* w, const uint16_t* xcal, int N, int K, int T, int group_size,
                     const double* alphas, int n_alpha, double* losses, int* best, void* stream) {
  begin_call();
  if (!w || !xcal || !alphas || !losses || !best) return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (T <= 0 || n_alpha <= 0) return fail(W4A16_ERR_INVALID_ARG, "T and the grid size must be positive");
  if (int rc = check_shape(N, K, group_size)) return rc;
  for (int i = 0; i < n_alpha; ++i)
    if (!(alphas[i] >= 0.0) || !std::isfinite(alphas[i]))
      return fail(W4A16_ERR_INVALID_ARG, "alpha[%d] is not a finite number >= 0", i);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = K / group_size;
  const size_t nk = static_cast<size_t>(N) * K, tk = static_cast<size_t>(T) * K, tn = static_cast<size_t>(T) * N;
  const int parts = static_cast<int>(std::min<size_t>(1024, (tn + 255) / 256));

  std::vector<void*> dev;
  auto release = [&](int rc) {
    for (void* p : dev) (void)hipFree(p);
    return rc;
  };
  auto alloc = [&](size_t bytes) -> void* {
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
    dev.push_back(p);
    return p;
  };
  auto* dw = static_cast<half_t*>(alloc(nk * 2));
  auto* dx = static_cast<half_t*>(alloc(tk * 2));
  auto* dxs = static_cast<uint16_t*>(alloc(tk * 2));
  auto* dq = static_cast<int32_t*>(alloc(nk / 2));
  auto* ds = static_cast<uint16_t*>(alloc(static_cast<size_t>(G) * N * 2));
  auto* dz = static_cast<int32_t*>(alloc(static_cast<size_t>(G) * N / 2));
  auto* dyref = static_cast<half_t*>(alloc(tn * 2));
  auto* dy = static_cast<uint16_t*>(alloc(tn * 2));
  auto* dpart = static_cast<float*>(alloc(static_cast<size_t>(parts) * sizeof(float)));
  auto* dsc = static_cast<double*>(alloc(static_cast<size_t>(K) * sizeof(double)));
  if (dev.size() != 10) return release(fail(W4A16_ERR_HIP, "hipMalloc failed for the search buffers"));
  if (int rc = hip_status(hipMemcpyAsync(dw, w, nk * 2, hipMemcpyHostToDevice, st), "hipMemcpyAsync")) return release(rc);
  if (int rc = hip_status(hipMemcpyAsync(dx, xcal, tk * 2, hipMemcpyHostToDevice, st), "hipMemcpyAsync"))
    return release(rc);
  // the unquantised layer's outputs: binary16 weights on the tiled MFMA kernel
  if (int rc = run_gemm_tiled<16>(st, dx, reinterpret_cast<const uint32_t*>(dw), nullptr, Zeros{nullptr, 0}, dyref,
                                  T, N, K, 0))
    return release(rc);

  std::vector<double> s(K);
  std::vector<float> part(parts);
  for (int i = 0; i < n_alpha; ++i) {
    // the candidate's scale on the host (exact mean), quantisation and fold on the device
    int rc = w4a16_awq_scales(xcal, T, K, alphas[i], s.data());
    if (rc != W4A16_OK) return release(rc);
    if (int r = hip_status(hipMemcpyAsync(dsc, s.data(), K * sizeof(double), hipMemcpyHostToDevice, st),
                           "hipMemcpyAsync"))
      return release(r);
    rc = w4a16_quantize_device(reinterpret_cast<const uint16_t*>(dw), N, K, group_size, dsc, 0, dq, ds, dz, st);
    if (rc != W4A16_OK) return release(rc);
    hipLaunchKernelGGL(fold_activations_kernel, dim3(static_cast<unsigned>((tk + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const uint16_t*>(dx), dsc, tk, K, dxs);
    if (int r = check_launch("fold launch")) return release(r);
    rc = w4a16_gemm(dxs, dq, ds, dz, nullptr, group_size, T, N, K, dy, st);
    if (rc != W4A16_OK) return release(rc);
    hipLaunchKernelGGL(sq_diff_kernel, dim3(parts), dim3(256), 0, st, dyref, reinterpret_cast<const half_t*>(dy), tn,
                       dpart);
    if (int r = check_launch("squared-difference launch")) return release(r);
    if (int r = hip_status(hipMemcpyAsync(part.data(), dpart, parts * sizeof(float), hipMemcpyDeviceToHost, st),
                           "hipMemcpyAsync"))
      return release(r);
    if (int r = hip_status(hipStreamSynchronize(st), "hipStreamSynchronize")) return release(r);
    double total = 0.0;
    for (int p = 0; p < parts; ++p) total += part[p];
    losses[i] = std::sqrt(total);
  }
  int b = 0;
  for (int i = 1; i < n_alpha; ++i)
    if (losses[i] < losses[b]) b = i;
  *best = b;
  return release(W4A16_OK);
}

// GPTQ ("AWQ + GPTQ Quantization, in depth", The two algorithms, compactly): host
// inputs and outputs, binary64 device work on `stream`, returns when the outputs are on
// the host.
int w4a16_gptq(const uint16_t* w, const uint16_t* xcal, int N, int K, int T, int group_size, int act_order,
               double damp, uint8_t* codes, uint16_t* scales, uint8_t* zeros, int32_t* g_idx, void* stream) {
  begin_call();
  if (!w || !xcal || !codes || !scales || !zeros || (act_order && !g_idx))
    return fail(W4A16_ERR_INVALID_ARG, "NULL buffer");
  if (T <= 0) return fail(W4A16_ERR_INVALID_ARG, "T must be positive (T=%d)", T);
  if (!(damp >= 0.0) || !std::isfinite(damp)) return fail(W4A16_ERR_INVALID_ARG, "damp must be a finite number >= 0");
  if (int rc = check_shape(N, K, group_size)) return rc;
  const size_t nk = static_cast<size_t>(N) * K, tk = static_cast<size_t>(T) * K, kk = static_cast<size_t>(K) * K;
  for (size_t i = 0; i < nk; ++i)
    if (((w[i] >> 10) & 0x1F) == 0x1F) return fail(W4A16_ERR_INVALID_ARG, "weight %zu is not finite", i);
  // visiting order: act order (descending diag(H), exact) or the channels in order
  std::vector<int32_t> order;
  if (int rc = act_order_rank(xcal, T, K, order)) return rc;   // also checks xcal is finite
  if (act_order) {
    for (int i = 0; i < K; ++i) g_idx[order[i]] = i / group_size;
  } else {
    for (int k = 0; k < K; ++k) order[k] = k;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int G = K / group_size;

  std::vector<void*> dev;
  auto release = [&](int rc) {
    for (void* p : dev) (void)hipFree(p);
    return rc;
  };
  auto alloc = [&](size_t bytes) -> void* {
    void* p = nullptr;
    if (hipMalloc(&p, bytes) != hipSuccess) return nullptr;
    dev.push_back(p);
    return p;
  };
  auto* dw = static_cast<uint16_t*>(alloc(nk * 2));
  auto* dx = static_cast<uint16_t*>(alloc(tk * 2));
  auto* dperm = static_cast<int32_t*>(alloc(static_cast<size_t>(K) * 4));
  auto* dwp = static_cast<double*>(alloc(nk * 8));
  auto* dxp = static_cast<double*>(alloc(tk * 8));
  auto* dH = static_cast<double*>(alloc(kk * 8));
  auto* dU = static_cast<double*>(alloc(kk * 8));
  auto* derr = static_cast<double*>(alloc(static_cast<size_t>(N) * kGptqBatch * 8));
  auto* dsz = static_cast<double2*>(alloc(static_cast<size_t>(N) * sizeof(double2)));
  auto* dcp = static_cast<uint8_t*>(alloc(nk));
  auto* dc = static_cast<uint8_t*>(alloc(nk));
  auto* ds = static_cast<uint16_t*>(alloc(static_cast<size_t>(G) * N * 2));
  auto* dz = static_cast<uint8_t*>(alloc(static_cast<size_t>(G) * N));
  auto* dflag = static_cast<int*>(alloc(sizeof(int)));
  auto* ddg = static_cast<double*>(alloc(static_cast<size_t>(kGptqPivots) * kGptqPivots * 8));
  if (dev.size() != 15) return release(fail(W4A16_ERR_HIP, "hipMalloc failed for the GPTQ buffers"));
  const int zero = 0;
  int flag = 0;
  auto copy = [&](void* dst, const void* src, size_t bytes, hipMemcpyKind kind) {
    return hip_status(hipMemcpyAsync(dst, src, bytes, kind, st), "hipMemcpyAsync");
  };
  if (int rc = copy(dw, w, nk * 2, hipMemcpyHostToDevice)) return release(rc);
  if (int rc = copy(dx, xcal, tk * 2, hipMemcpyHostToDevice)) return release(rc);
  if (int rc = copy(dperm, order.data(), static_cast<size_t>(K) * 4, hipMemcpyHostToDevice)) return release(rc);
  if (int rc = copy(dflag, &zero, sizeof(int), hipMemcpyHostToDevice)) return release(rc);
  auto blocks = [](size_t n) { return dim3(static_cast<unsigned>((n + 255) / 256)); };

  // weights and calibration rows in visiting order, H = 2 X X^T, damping
  hipLaunchKernelGGL(gptq_gather_kernel, blocks(nk), dim3(256), 0, st, dw, dperm, static_cast<size_t>(N), K, dwp);
  hipLaunchKernelGGL(gptq_gather_kernel, blocks(tk), dim3(256), 0, st, dx, dperm, static_cast<size_t>(T), K, dxp);
  const unsigned kt = static_cast<unsigned>((K + 63) / 64);
  hipLaunchKernelGGL(gptq_gram_kernel, dim3(kt, kt), dim3(256), 0, st, dxp, T, K, dH);
  hipLaunchKernelGGL(gptq_damp_kernel, dim3(1), dim3(256), 0, st, dH, K, damp);
  if (int rc = check_launch("GPTQ Hessian launch")) return release(rc);
  // H = Ut^T Ut from the bottom-right corner, then U = (Ut^T)^-1; pivots in blocks of 64
  // from the bottom (the same operations, in the same order per element, as one pivot
  // at a time)
  auto tiles = [](int n) { return (n + kGptqPivots - 1) / kGptqPivots; };
  for (int p1 = K; p1 > 0;) {
    const int p0 = std::max(0, p1 - kGptqPivots), bs = p1 - p0;
    hipLaunchKernelGGL(gptq_chol_panel_kernel, dim3(static_cast<unsigned>(tiles(p0) + 1)), dim3(256), 0, st, dH, K, p0,
                       bs, ddg);
    const int nt = tiles(p0);
    hipLaunchKernelGGL(gptq_chol_trail_kernel, dim3(static_cast<unsigned>(std::max(1, nt * (nt + 1) / 2))), dim3(256), 0,
                       st, dH, K, p0, bs, ddg);
    p1 = p0;
  }
  hipLaunchKernelGGL(gptq_chol_finish_kernel, dim3(K), dim3(256), 0, st, dH, K, dflag);
  hipLaunchKernelGGL(gptq_eye_kernel, blocks(kk), dim3(256), 0, st, dU, K);
  for (int p1 = K; p1 > 0;) {
    const int p0 = std::max(0, p1 - kGptqPivots), bs = p1 - p0;
    const unsigned ct = static_cast<unsigned>(tiles(K - p0));
    hipLaunchKernelGGL(gptq_trinv_panel_kernel, dim3(ct), dim3(256), 0, st, dH, dU, K, p0, bs);
    if (p0 > 0)
      hipLaunchKernelGGL(gptq_trinv_trail_kernel, dim3(ct, static_cast<unsigned>(tiles(p0))), dim3(256), 0, st, dH,
                         dU, K, p0, bs);
    p1 = p0;
  }
  hipLaunchKernelGGL(gptq_trinv_finish_kernel, dim3(K), dim3(256), 0, st, dH, dU, K);
  if (int rc = check_launch("GPTQ factorisation launch")) return release(rc);
  // rounding with error feedback, 32 visited columns at a time, 128 to a batch: the
  // block's errors go to the batch's later columns, the batch's to every column after it
  auto update = [&](const double* e, int i0, int rank, int k_begin, int k_end) {
    hipLaunchKernelGGL(gptq_update_kernel, dim3(static_cast<unsigned>((k_end - k_begin + 63) / 64),
                                                static_cast<unsigned>((N + 63) / 64)),
                       dim3(256), 0, st, dwp, dU, e, kGptqBatch, N, K, i0, rank, k_begin, k_end);
  };
  for (int b0 = 0; b0 < K; b0 += kGptqBatch) {
    const int bend = std::min(b0 + kGptqBatch, K);
    for (int i0 = b0; i0 < bend; i0 += kGptqBlock) {
      hipLaunchKernelGGL(gptq_block_kernel, dim3(static_cast<unsigned>((N + 127) / 128)), dim3(128), 0, st, dwp, dU,
                         N, K, i0, group_size, dsz, derr + (i0 - b0), kGptqBatch, dcp, ds, dz);
      if (i0 + kGptqBlock < bend) update(derr + (i0 - b0), i0, kGptqBlock, i0 + kGptqBlock, bend);
    }
    if (bend < K) update(derr, b0, bend - b0, bend, K);
  }
  hipLaunchKernelGGL(gptq_scatter_codes_kernel, blocks(nk), dim3(256), 0, st, dcp, dperm, N, K, dc);
  if (int rc = check_launch("GPTQ rounding launch")) return release(rc);
  if (int rc = copy(codes, dc, nk, hipMemcpyDeviceToHost)) return release(rc);
  if (int rc = copy(scales, ds, static_cast<size_t>(G) * N * 2, hipMemcpyDeviceToHost)) return release(rc);
  if (int rc = copy(zeros, dz, static_cast<size_t>(G) * N, hipMemcpyDeviceToHost)) return release(rc);
  if (int rc = copy(&flag, dflag, sizeof(int), hipMemcpyDeviceToHost)) return release(rc);
  if (int rc = hip_status(hipStreamSynchronize(st), "hipStreamSynchronize")) return release(rc);
  if (flag) return release(fail(W4A16_ERR_INVALID_ARG, "the damped Hessian is not positive definite (raise damp)"));
  return release(W4A16_OK);
}

}  // extern "C"
