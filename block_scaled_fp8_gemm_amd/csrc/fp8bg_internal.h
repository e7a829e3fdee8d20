// Internal interfaces between the C-ABI layer, the planner and the kernel
// launchers.  Not installed; the public interface is include/fp8bg.h.
#pragma once

#include <stdint.h>

#include "fp8bg.h"

#ifdef __HIPCC__
#include <hip/hip_runtime.h>
#endif

namespace fbg {

// Planner (pure host code, fp8bg_plan.cpp).  Fills *out for a validated shape.
// force_cfg >= 0 overrides the tile configuration within the chosen variant.
int make_plan(int64_t M, int64_t N, int64_t K, int out_dtype, int cu_count, int variant, int split_k,
              fbg_plan* out, int force_cfg);

// Grouped GEMM: the tile configuration for E experts holding M token rows in
// total (force_cfg >= 0 overrides it; -1 if no such configuration) and the
// launch grid.  Configurations 0 .. kNumGroupedCfgs-1 are the skinny grouped
// kernel's (grid E x n-tiles); kNumGroupedCfgs + c is the generic kernel's
// configuration c in grouped mode (grid (ceil(M/BM) + E) x n-tiles, an upper
// bound on the experts' row tiles).  Pure host code.
int grouped_cfg_for(int64_t M, int64_t E, int64_t N, int64_t K, int force_cfg);
int64_t grouped_grid(int cfg, int64_t E, int64_t M, int64_t N);
int grouped_num_cfgs();
int grouped_num_skinny_cfgs();

// Bytes of split-K workspace for a plan: FP32 partials, then one counter per tile.
int64_t workspace_bytes(const fbg_plan& p, int64_t M, int64_t N);
int64_t workspace_counter_offset(const fbg_plan& p, int64_t M, int64_t N);

#ifdef __HIPCC__
struct GemmArgs {
  const uint8_t* A;
  const float* a_s;
  const uint8_t* B;
  const float* b_s;
  void* C;
  int M, N, K;
  int out;
  int vec;  // bit 0: N % 4 == 0 and C aligned for 4-element vector stores;
            // bit 1: C rows 16-byte aligned (row pitch and base)
  hipStream_t stream;
};

hipError_t launch_generic(const GemmArgs& a, int cfg, int64_t grid, int band);
hipError_t launch_swap(const GemmArgs& a, int cfg, int64_t grid, int S, float* ws, unsigned* counters);
hipError_t launch_short_k256(const GemmArgs& a, int cfg, int64_t grid);
hipError_t launch_zero_words(void* p, int64_t count, hipStream_t stream);
hipError_t launch_fill_zero(void* C, int64_t count, int out, hipStream_t stream);
hipError_t launch_grouped(const GemmArgs& a, int cfg, int64_t grid, const int* offsets, int E);
hipError_t launch_generic_grouped(const GemmArgs& a, int cfg, int64_t grid, const int* offsets, int E);
hipError_t launch_quantize_rows(const uint16_t* x, uint8_t* q, float* a_s, int64_t groups, hipStream_t stream);
hipError_t launch_quantize_blocks(const uint16_t* w, uint8_t* q, float* b_s, int N, int K, hipStream_t stream);
#endif

}  // namespace fbg
