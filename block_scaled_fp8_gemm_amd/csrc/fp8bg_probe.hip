// Load-path probe: measures how fast one workgroup per CU can stream bytes
// from memory, through direct-to-LDS loads or loads into registers, with a
// fixed number of 1 KB wave loads in flight.  It is a measuring tool for the
// design notes (built into libfp8bg_probe.so, not into the GEMM library) and
// computes nothing of the GEMM.
//
// Workgroup w reads its region src + w * wg_stride at offsets
// ((i * NW + wave) * 1024 + 16 * lane) & region_mask for load i of the wave:
// region_mask + 1 bytes per region (a power of two), so a small region read
// by every workgroup (wg_stride 0) streams from L2, and disjoint regions
// larger than the caches stream from HBM.  The host call checks that every
// offset stays inside the caller's buffer.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "fp8bg_device.hpp"

namespace fbg {
namespace {

constexpr int kDepth = 8;  // 1 KB loads in flight per wave

template <int NW, int DMA>
__global__ __launch_bounds__(64 * NW) void k_probe_stream(const uint8_t* __restrict__ src, int64_t wg_stride,
                                                          uint32_t region_mask, int loads_per_wave,
                                                          uint32_t* __restrict__ sink, int sink_flag) {
  // 96 KB of LDS: no second workgroup fits on a CU (160 KB), so the grid
  // spreads one workgroup per CU.
  __shared__ __attribute__((aligned(16))) uint8_t ring[96 * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint8_t* base = src + (int64_t)blockIdx.x * wg_stride;
  auto off = [&](int i) { return ((uint32_t)(i * NW + wave) * 1024u + 16u * (uint32_t)lane) & region_mask; };
  if constexpr (DMA) {
    const buf_rsrc r = make_rsrc(base);
    lds_u8* const lds = (lds_u8*)ring;
    auto issue = [&](int i) { lds_dma16(r, off(i), 0, lds + ((i % kDepth) * NW + wave) * 1024); };
    const int pro = loads_per_wave < kDepth ? loads_per_wave : kDepth;
    for (int i = 0; i < pro; ++i) issue(i);
    for (int i = kDepth; i < loads_per_wave; ++i) {
      __builtin_amdgcn_s_waitcnt(vmcnt_only(kDepth - 1));
      issue(i);
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  } else {
    uint32_t acc = 0;
    for (int i0 = 0; i0 < loads_per_wave; i0 += kDepth) {
      v4i v[kDepth];
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        const int i = i0 + d < loads_per_wave ? i0 + d : loads_per_wave - 1;
        v[d] = *reinterpret_cast<const v4i*>(base + off(i));
      }
#pragma unroll
      for (int d = 0; d < kDepth; ++d) acc ^= (uint32_t)(v[d][0] ^ v[d][1] ^ v[d][2] ^ v[d][3]);
    }
    // Never true for the flag the host passes: keeps the loads live, and the
    // LDS allocation that holds the grid to one workgroup per CU.
    if (sink_flag == 0x5eed && acc == 0x9e3779b9u) {
      ring[threadIdx.x] = (uint8_t)acc;
      sink[blockIdx.x * 64 * NW + threadIdx.x] = acc + ring[(threadIdx.x + 1) & 255];
    }
  }
}

}  // namespace
}  // namespace fbg

// Streams loads_per_wave 1 KB loads per wave through `grid` workgroups of
// `waves` waves (4 or 8), direct-to-LDS (dma != 0) or into registers.
// src: device buffer of src_bytes; region_bytes a power of two between 1 KB
// and 1 GiB; every workgroup's region must lie inside the buffer.  sink: a
// device buffer of grid * 64 * waves words, never written in practice.
// Returns 0, or 1 for invalid arguments (nothing launched), or 2 for a
// launch error.
extern "C" int fbg_probe_stream(const void* src, int64_t src_bytes, int64_t wg_stride, int64_t region_bytes,
                                int grid, int waves, int dma, int loads_per_wave, void* sink,
                                hipStream_t stream) {
  if (!src || !sink || grid <= 0 || loads_per_wave <= 0 || wg_stride < 0) return 1;
  if (region_bytes < 1024 || region_bytes > ((int64_t)1 << 30) || (region_bytes & (region_bytes - 1))) return 1;
  if ((int64_t)(grid - 1) * wg_stride + region_bytes > src_bytes) return 1;
  const uint32_t mask = (uint32_t)(region_bytes - 1);
  const dim3 blk(64 * waves);
  using namespace fbg;
  const uint8_t* s = static_cast<const uint8_t*>(src);
  uint32_t* k = static_cast<uint32_t*>(sink);
  if (waves == 4 && dma) hipLaunchKernelGGL((k_probe_stream<4, 1>), dim3(grid), blk, 0, stream, s, wg_stride, mask, loads_per_wave, k, 0);
  else if (waves == 4) hipLaunchKernelGGL((k_probe_stream<4, 0>), dim3(grid), blk, 0, stream, s, wg_stride, mask, loads_per_wave, k, 0);
  else if (waves == 8 && dma) hipLaunchKernelGGL((k_probe_stream<8, 1>), dim3(grid), blk, 0, stream, s, wg_stride, mask, loads_per_wave, k, 0);
  else if (waves == 8) hipLaunchKernelGGL((k_probe_stream<8, 0>), dim3(grid), blk, 0, stream, s, wg_stride, mask, loads_per_wave, k, 0);
  else return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
