// C-ABI entry points: argument validation, the dispatcher's plan, split-K
// workspace handling and kernel launch.  See include/fp8bg.h for the
// contract of each function.
#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp8bg.h"
#include "fp8bg_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];  // 0 = not yet queried

int device_cu_count(int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    *status = FBG_ERROR_HIP;
    return 0;
  }
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) {
    *status = FBG_ERROR_HIP;
    return 0;
  }
  if (dev < kMaxDevices) g_cu_count[dev].store(cu, std::memory_order_relaxed);
  return cu;
}

bool env_flag(const char* name) {
  const char* v = getenv(name);
  return v && v[0] && strcmp(v, "0") != 0;
}

int elem_size(int out_dtype) { return out_dtype == FBG_OUT_FP32 ? 4 : 2; }

// Largest K: the kernels address a tile's rows (up to 256 of K bytes each)
// through a buffer resource based at the tile's first row, whose 32-bit
// record count reaches 2^32 - 1 bytes: 256 rows of K bytes must end before
// that, so K <= 2^24 - 128 (at K = 2^24 the last dword of a 256-row tile
// read as zero).
constexpr int64_t kMaxK = ((int64_t)1 << 24) - 128;

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// FBG_FORCE_CONFIG=<index>: tests and benchmarks pin the tile configuration
// of the chosen variant (read on every call so a test can change it).
int forced_config() {
  const char* v = getenv("FBG_FORCE_CONFIG");
  return (v && v[0]) ? atoi(v) : -1;
}

// Pure host checks, made before any HIP call.
int validate(const void* A, const float* a_s, const void* B, const float* b_s, const void* C, int64_t M,
             int64_t N, int64_t K, int out_dtype) {
  if (M < 0 || N < 0 || K < 0) return FBG_ERROR_INVALID_VALUE;
  if (out_dtype != FBG_OUT_BF16 && out_dtype != FBG_OUT_FP16 && out_dtype != FBG_OUT_FP32)
    return FBG_ERROR_INVALID_VALUE;
  if (K % 128 != 0) return FBG_ERROR_UNSUPPORTED;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return FBG_ERROR_UNSUPPORTED;
  // The kernels address a tile's rows (up to 256 of them) with 32-bit offsets.
  if (K > kMaxK) return FBG_ERROR_UNSUPPORTED;
  const int64_t G = K / 128, NB = (N + 127) / 128;
  const int64_t bytesA = M * K, bytesB = N * K, bytesAs = M * G * 4, bytesBs = NB * G * 4;
  const int64_t bytesC = M * N * elem_size(out_dtype);
  // The generic kernel addresses the scale arrays with 32-bit buffer offsets.
  if (bytesAs > (int64_t)UINT32_MAX || bytesBs > (int64_t)UINT32_MAX) return FBG_ERROR_UNSUPPORTED;
  if ((bytesA > 0 && !A) || (bytesB > 0 && !B) || (bytesAs > 0 && !a_s) || (bytesBs > 0 && !b_s) ||
      (bytesC > 0 && !C))
    return FBG_ERROR_INVALID_VALUE;
  if (overlaps(C, bytesC, A, bytesA) || overlaps(C, bytesC, B, bytesB) || overlaps(C, bytesC, a_s, bytesAs) ||
      overlaps(C, bytesC, b_s, bytesBs))
    return FBG_ERROR_INVALID_VALUE;
  if ((bytesA > 0 && !aligned(A, 16)) || (bytesB > 0 && !aligned(B, 16)) || (bytesAs > 0 && !aligned(a_s, 4)) ||
      (bytesBs > 0 && !aligned(b_s, 4)) || (bytesC > 0 && !aligned(C, (uintptr_t)elem_size(out_dtype))))
    return FBG_ERROR_UNSUPPORTED;
  return FBG_SUCCESS;
}

// FBG_RASTER_BAND=<rows>: benchmarks try other raster band heights for the
// generic kernel (default 8 tile-rows).
int raster_band() {
  const char* v = getenv("FBG_RASTER_BAND");
  const int b = (v && v[0]) ? atoi(v) : 0;
  return b > 0 ? b : 8;
}

// Launches the plan's kernel.  partial / counters: the split-K workspace's
// FP32 partials and arrival counters (unused unless the plan splits K).
int launch_plan(const fbg_plan& p, const fbg::GemmArgs& args, float* partial, unsigned* counters) {
  hipError_t e = hipSuccess;
  switch (p.variant) {
    case FBG_VARIANT_GENERIC:
      e = fbg::launch_generic(args, p.config, p.grid, raster_band());
      break;
    case FBG_VARIANT_SHORT_K256:
      e = fbg::launch_short_k256(args, p.config, p.grid);
      break;
    case FBG_VARIANT_SWAP_AB:
    case FBG_VARIANT_SWAP_AB_SPLITK:
      if (p.split_k <= 1) partial = nullptr, counters = nullptr;
      e = fbg::launch_swap(args, p.config, p.grid, p.split_k, partial, counters);
      break;
    default:
      return FBG_ERROR_INVALID_VALUE;
  }
  return e == hipSuccess ? FBG_SUCCESS : FBG_ERROR_HIP;
}

// A workspace laid out as fp8_block_gemm_workspace_size describes: the
// partials first, the counters at workspace_counter_offset.
int launch_with_workspace(const fbg_plan& p, const fbg::GemmArgs& args, void* ws, int64_t M, int64_t N) {
  return launch_plan(p, args, static_cast<float*>(ws),
                     reinterpret_cast<unsigned*>(static_cast<char*>(ws) + fbg::workspace_counter_offset(p, M, N)));
}

// ---------------------------------------------------------------------------
// The no-allocation entry point's scratch: split-K arrival counters in the
// first kScratchCounterBytes, FP32 partials after them.  Every GPU the library
// runs on holds its own copy for the life of the process.  In host code the
// array's name is not a device address: the kernels get the per-device address
// that hipGetSymbolAddress returns (scratch_address).  The counters are zero
// when the code object is loaded, are cleared once more by the first call on
// each device, and every completed call leaves them zero.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = (int64_t)4 << 20;
constexpr int64_t kScratchCounterBytes = (int64_t)16 << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// This device's scratch address (set up on the device's first call: the
// symbol's address, then a kernel on `stream` clearing the counters), or
// nullptr with *status set.
void* scratch_address(hipStream_t stream, int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = FBG_ERROR_HIP;
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
    (void)hipGetLastError();
    *status = FBG_ERROR_HIP;
    return nullptr;
  }
  if (fbg::launch_zero_words(ptr, kScratchCounterBytes / 4, stream) != hipSuccess) {
    *status = FBG_ERROR_HIP;
    return nullptr;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

enum WorkspaceMode { kCallerOrLibrary, kStaticScratch };

int gemm_call(const void* A, const float* a_s, const void* B, const float* b_s, void* C, int64_t M, int64_t N,
              int64_t K, int out_dtype, void* stream_, int variant, int split_k, void* workspace,
              size_t workspace_size, WorkspaceMode mode) {
  int st = validate(A, a_s, B, b_s, C, M, N, K, out_dtype);
  if (st != FBG_SUCCESS) return st;
  if (variant < FBG_VARIANT_AUTO || variant > FBG_VARIANT_SWAP_AB_SPLITK || split_k < 0)
    return FBG_ERROR_INVALID_VALUE;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  // No caller workspace and the dispatcher's choice: plan without a K split,
  // so the call never allocates (a stream-ordered allocation and free cost
  // more than splitting saves).  A split forced without a workspace still
  // gets a stream-ordered one below.  The static scratch keeps the split.
  if (mode == kCallerOrLibrary && !workspace && variant == FBG_VARIANT_AUTO && split_k == 0) split_k = 1;
  if (M == 0 || N == 0) return FBG_SUCCESS;
  if (K == 0) {
    // Still honour a forced variant's guard before filling.
    fbg_plan p;
    st = fbg::make_plan(M, N, K, out_dtype, 256, variant, split_k, &p, -1);
    if (st != FBG_SUCCESS) return st;
    return fbg::launch_fill_zero(C, M * N, out_dtype, stream) == hipSuccess ? FBG_SUCCESS : FBG_ERROR_HIP;
  }
  const int cu = device_cu_count(&st);
  if (st != FBG_SUCCESS) return st;
  fbg_plan p;
  st = fbg::make_plan(M, N, K, out_dtype, cu, variant, split_k, &p, forced_config());
  if (st != FBG_SUCCESS) return st;

  fbg::GemmArgs args;
  args.A = static_cast<const uint8_t*>(A);
  args.a_s = a_s;
  args.B = static_cast<const uint8_t*>(B);
  args.b_s = b_s;
  args.C = C;
  args.M = (int)M;
  args.N = (int)N;
  args.K = (int)K;
  args.out = out_dtype;
  args.vec = (N % 4 == 0) && aligned(C, (uintptr_t)(4 * elem_size(out_dtype)));
  if (args.vec && (N * elem_size(out_dtype)) % 16 == 0 && aligned(C, 16)) args.vec |= 2;  // 16-byte rows
  args.stream = stream;

  if (env_flag("FBG_LOG"))
    fprintf(stderr, "fp8bg: M=%lld N=%lld K=%lld out=%d -> variant=%d cfg=%d tile=%dx%d S=%d grid=%lld ws=%lld\n",
            (long long)M, (long long)N, (long long)K, out_dtype, p.variant, p.config, p.tile_m, p.tile_n, p.split_k,
            (long long)p.grid, (long long)p.workspace_bytes);

  if (p.workspace_bytes == 0) return launch_plan(p, args, nullptr, nullptr);

  if (mode == kStaticScratch) {
    const int64_t tiles = p.grid / p.split_k;
    const int64_t partial = fbg::workspace_counter_offset(p, M, N);
    if (tiles * 4 > kScratchCounterBytes || partial > kScratchBytes - kScratchCounterBytes)
      return FBG_ERROR_SCRATCH_LIMIT;
    char* base = static_cast<char*>(scratch_address(stream, &st));
    if (!base) return st;
    return launch_plan(p, args, reinterpret_cast<float*>(base + kScratchCounterBytes),
                       reinterpret_cast<unsigned*>(base));
  }
  if (workspace) {
    if (workspace_size < (size_t)p.workspace_bytes) return FBG_ERROR_OUT_OF_MEMORY;
    if (!aligned(workspace, 16)) return FBG_ERROR_UNSUPPORTED;
    return launch_with_workspace(p, args, workspace, M, N);
  }
  // Library-owned workspace: stream-ordered, so concurrent streams never share one.
  if (env_flag("FBG_TEST_FAIL_ALLOC")) return FBG_ERROR_OUT_OF_MEMORY;
  void* ws = nullptr;
  if (hipMallocAsync(&ws, (size_t)p.workspace_bytes, stream) != hipSuccess || !ws) {
    (void)hipGetLastError();
    return FBG_ERROR_OUT_OF_MEMORY;
  }
  const int64_t coff = fbg::workspace_counter_offset(p, M, N);
  if (fbg::launch_zero_words(static_cast<char*>(ws) + coff, (p.workspace_bytes - coff) / 4, stream) != hipSuccess) {
    (void)hipFreeAsync(ws, stream);
    return FBG_ERROR_HIP;
  }
  st = launch_with_workspace(p, args, ws, M, N);
  if (hipFreeAsync(ws, stream) != hipSuccess && st == FBG_SUCCESS) st = FBG_ERROR_HIP;
  return st;
}

}  // namespace

extern "C" int fp8_block_gemm_ex(const void* A, const float* a_s, const void* B, const float* b_s, void* C, int64_t M,
                                 int64_t N, int64_t K, int out_dtype, void* stream, int variant, int split_k,
                                 void* workspace, size_t workspace_size) {
  return gemm_call(A, a_s, B, b_s, C, M, N, K, out_dtype, stream, variant, split_k, workspace, workspace_size,
                   kCallerOrLibrary);
}

extern "C" int fp8_block_gemm(const void* A, const float* a_s, const void* B, const float* b_s, void* C, int64_t M,
                              int64_t N, int64_t K, int out_dtype, void* stream) {
  return fp8_block_gemm_ex(A, a_s, B, b_s, C, M, N, K, out_dtype, stream, FBG_VARIANT_AUTO, 0, nullptr, 0);
}

extern "C" int fp8_block_gemm_noalloc(const void* A, const float* a_s, const void* B, const float* b_s, void* C,
                                      int64_t M, int64_t N, int64_t K, int out_dtype, void* stream, int variant,
                                      int split_k) {
  return gemm_call(A, a_s, B, b_s, C, M, N, K, out_dtype, stream, variant, split_k, nullptr, 0, kStaticScratch);
}

extern "C" size_t fp8_block_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int variant, int split_k) {
  int cu = 256;
  if (variant == FBG_VARIANT_AUTO || split_k == 0) {
    int st = FBG_SUCCESS;
    cu = device_cu_count(&st);
    if (st != FBG_SUCCESS) return (size_t)-1;
  }
  fbg_plan p;
  if (fbg::make_plan(M, N, K, FBG_OUT_BF16, cu, variant, split_k, &p, forced_config()) != FBG_SUCCESS)
    return (size_t)-1;
  return (size_t)p.workspace_bytes;
}

extern "C" int fp8_block_gemm_quantize_rows(const void* x, int64_t M, int64_t K, void* A, float* a_s, void* stream_) {
  if (M < 0 || K < 0) return FBG_ERROR_INVALID_VALUE;
  if (K % 128 != 0) return FBG_ERROR_UNSUPPORTED;
  if (M > INT32_MAX || K > INT32_MAX) return FBG_ERROR_UNSUPPORTED;
  const int64_t G = K / 128, bytesX = M * K * 2, bytesA = M * K, bytesAs = M * G * 4;
  if ((bytesX > 0 && !x) || (bytesA > 0 && !A) || (bytesAs > 0 && !a_s)) return FBG_ERROR_INVALID_VALUE;
  if (overlaps(A, bytesA, x, bytesX) || overlaps(a_s, bytesAs, x, bytesX) || overlaps(A, bytesA, a_s, bytesAs))
    return FBG_ERROR_INVALID_VALUE;
  if ((bytesX > 0 && !aligned(x, 16)) || (bytesA > 0 && !aligned(A, 8)) || (bytesAs > 0 && !aligned(a_s, 4)))
    return FBG_ERROR_UNSUPPORTED;
  if (M == 0 || K == 0) return FBG_SUCCESS;
  const hipError_t e = fbg::launch_quantize_rows(static_cast<const uint16_t*>(x), static_cast<uint8_t*>(A), a_s,
                                                 M * G, static_cast<hipStream_t>(stream_));
  return e == hipSuccess ? FBG_SUCCESS : FBG_ERROR_HIP;
}

extern "C" int fp8_block_gemm_quantize_blocks(const void* w, int64_t N, int64_t K, void* B, float* b_s,
                                              void* stream_) {
  if (N < 0 || K < 0) return FBG_ERROR_INVALID_VALUE;
  if (K % 128 != 0) return FBG_ERROR_UNSUPPORTED;
  if (N > INT32_MAX || K > INT32_MAX) return FBG_ERROR_UNSUPPORTED;
  const int64_t G = K / 128, NB = (N + 127) / 128;
  const int64_t bytesW = N * K * 2, bytesB = N * K, bytesBs = NB * G * 4;
  if ((bytesW > 0 && !w) || (bytesB > 0 && !B) || (bytesBs > 0 && !b_s)) return FBG_ERROR_INVALID_VALUE;
  if (overlaps(B, bytesB, w, bytesW) || overlaps(b_s, bytesBs, w, bytesW) || overlaps(B, bytesB, b_s, bytesBs))
    return FBG_ERROR_INVALID_VALUE;
  if ((bytesW > 0 && !aligned(w, 16)) || (bytesB > 0 && !aligned(B, 8)) || (bytesBs > 0 && !aligned(b_s, 4)))
    return FBG_ERROR_UNSUPPORTED;
  if (N == 0 || K == 0) return FBG_SUCCESS;
  const hipError_t e = fbg::launch_quantize_blocks(static_cast<const uint16_t*>(w), static_cast<uint8_t*>(B), b_s,
                                                   (int)N, (int)K, static_cast<hipStream_t>(stream_));
  return e == hipSuccess ? FBG_SUCCESS : FBG_ERROR_HIP;
}

extern "C" int fp8_block_gemm_grouped(const void* A, const float* a_s, const void* B, const float* b_s, void* C,
                                      const int32_t* offsets, int64_t E, int64_t M, int64_t N, int64_t K,
                                      int out_dtype, void* stream_) {
  if (E < 0 || M < 0 || N < 0 || K < 0) return FBG_ERROR_INVALID_VALUE;
  if (out_dtype != FBG_OUT_BF16 && out_dtype != FBG_OUT_FP16 && out_dtype != FBG_OUT_FP32)
    return FBG_ERROR_INVALID_VALUE;
  if (K % 128 != 0) return FBG_ERROR_UNSUPPORTED;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || E > INT32_MAX - 1) return FBG_ERROR_UNSUPPORTED;
  if (K > kMaxK) return FBG_ERROR_UNSUPPORTED;  // 32-bit offsets inside a tile's rows
  const int64_t G = K / 128, NB = (N + 127) / 128;
  int64_t bytesB = 0, bytesBs = 0;
  if (__builtin_mul_overflow(E, N * K, &bytesB) || __builtin_mul_overflow(E, NB * G * 4, &bytesBs))
    return FBG_ERROR_UNSUPPORTED;  // B or b_s larger than any address space
  const int64_t bytesA = M * K, bytesAs = M * G * 4;
  const int64_t bytesC = M * N * elem_size(out_dtype), bytesOff = (E + 1) * 4;
  // The generic kernel addresses the scale arrays (one expert's b_s) with 32-bit buffer offsets.
  if (bytesAs > (int64_t)UINT32_MAX || NB * G * 4 > (int64_t)UINT32_MAX) return FBG_ERROR_UNSUPPORTED;
  if ((bytesA > 0 && !A) || (bytesAs > 0 && !a_s) || (bytesB > 0 && !B) || (bytesBs > 0 && !b_s) ||
      (bytesC > 0 && !C) || (E > 0 && !offsets))
    return FBG_ERROR_INVALID_VALUE;
  if (overlaps(C, bytesC, A, bytesA) || overlaps(C, bytesC, B, bytesB) || overlaps(C, bytesC, a_s, bytesAs) ||
      overlaps(C, bytesC, b_s, bytesBs) || overlaps(C, bytesC, offsets, bytesOff))
    return FBG_ERROR_INVALID_VALUE;
  if ((bytesA > 0 && !aligned(A, 16)) || (bytesB > 0 && !aligned(B, 16)) || (bytesAs > 0 && !aligned(a_s, 4)) ||
      (bytesBs > 0 && !aligned(b_s, 4)) || (bytesC > 0 && !aligned(C, (uintptr_t)elem_size(out_dtype))) ||
      (E > 0 && !aligned(offsets, 4)))
    return FBG_ERROR_UNSUPPORTED;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  if (M == 0 || N == 0) return FBG_SUCCESS;
  if (K == 0 || E == 0)  // the empty sum (no groups, or no expert to hold a row)
    return fbg::launch_fill_zero(C, M * N, out_dtype, stream) == hipSuccess ? FBG_SUCCESS : FBG_ERROR_HIP;
  const int cfg = fbg::grouped_cfg_for(M, E, N, K, forced_config());
  if (cfg < 0) return FBG_ERROR_UNSUPPORTED;
  const int64_t grid = fbg::grouped_grid(cfg, E, M, N);
  if (grid > INT32_MAX) return FBG_ERROR_UNSUPPORTED;

  fbg::GemmArgs args;
  args.A = static_cast<const uint8_t*>(A);
  args.a_s = a_s;
  args.B = static_cast<const uint8_t*>(B);
  args.b_s = b_s;
  args.C = C;
  args.M = (int)M;
  args.N = (int)N;
  args.K = (int)K;
  args.out = out_dtype;
  args.vec = (N % 4 == 0) && aligned(C, (uintptr_t)(4 * elem_size(out_dtype)));
  if (args.vec && (N * elem_size(out_dtype)) % 16 == 0 && aligned(C, 16)) args.vec |= 2;  // 16-byte rows
  args.stream = stream;
  if (env_flag("FBG_LOG"))
    fprintf(stderr, "fp8bg grouped: E=%lld M=%lld N=%lld K=%lld out=%d -> cfg=%d grid=%lld\n", (long long)E,
            (long long)M, (long long)N, (long long)K, out_dtype, cfg, (long long)grid);
  const hipError_t e = cfg < fbg::grouped_num_skinny_cfgs()
                           ? fbg::launch_grouped(args, cfg, grid, offsets, (int)E)
                           : fbg::launch_generic_grouped(args, cfg - fbg::grouped_num_skinny_cfgs(), grid, offsets,
                                                         (int)E);
  return e == hipSuccess ? FBG_SUCCESS : FBG_ERROR_HIP;
}
