// The (M, N, K) dispatcher: pure host code, no HIP calls, so it runs and is
// tested without a GPU.
//
// The pages' dispatch routes each shape by (M, N, K) to the best-fit kernel,
// every special path behind its own shape guard, with the generic kernel as
// the fallback for everything else (FlagGems-vllm PR #693, "feat: optimize
// w8a8 block fp8 matmul for Hopper", sections "Description" and "Numerical
// safety").  The per-shape meta-parameters the pages tune offline (block
// sizes, warps, stages, split-K; section "Specialized kernels and the
// optimization idea") become, here, a configuration index and a split count
// chosen from the shape and the device's compute-unit count.
#include <limits.h>
#include <string.h>

#include "fp8bg.h"
#include "fp8bg_configs.h"
#include "fp8bg_internal.h"

namespace fbg {

namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t skinny_tiles(const SkinnyCfg& c, int64_t M, int64_t N) {
  return cdiv(N, skinny_tile_n(c)) * cdiv(M, skinny_tile_m(c));
}

// Tile configurations, from on-device configuration sweeps of every
// workload shape and sweep point (bench.py with forced variant, split and
// configuration; the results are kept in profiles/).  The small shapes are
// bound by how many bytes each compute unit must pull (each CU sustains
// ~25-28 GB/s at these sizes) plus the split-K handshake, so the rules
// pick the tile that fills the device with the fewest bytes per CU.
//
// Swap-AB: 32 n x 64 m tiles (config 4) read every weight row once for
// M <= 64 and are used when they alone give every CU a workgroup (M > 16);
// otherwise 32 n x 16 m tiles (config 7), split over K below until the
// grid covers the device.
int swap_cfg_for(int64_t M, int64_t N, int cu) {
  if (M > 16 && cdiv(N, 32) * cdiv(M, 64) >= (int64_t)cu) return 4;
  return 7;
}

// Short-K (two groups, one per wave): 16 n x 16 m up to M = 48 (config 12),
// 32 n x 32 m up to M = 200 (config 15), 32 n x 64 m up to M = 256
// (config 10); above, 32 n x 32 m with one wave taking both groups
// (config 6).
int short_cfg_for(int64_t M) {
  if (M <= 48) return 12;
  if (M <= 200) return 15;
  if (M <= 256) return 10;
  return 6;
}

// Generic: the largest tile that still gives every compute unit a
// workgroup -- 256 x 256 (8 waves, the highest MFMA work per LDS byte),
// then 256 x 128, then 128 x 128 -- else 64 x 128 (the most workgroups).
int generic_cfg_for(int64_t M, int64_t N, int cu) {
  if (M <= 64) return 2;
  if (cdiv(M, 256) * cdiv(N, 256) >= (int64_t)cu) return 3;
  if (cdiv(M, 256) * cdiv(N, 128) >= (int64_t)cu) return 1;
  if (cdiv(M, 128) * cdiv(N, 128) >= (int64_t)cu) return 0;
  return 2;
}

}  // namespace

int make_plan(int64_t M, int64_t N, int64_t K, int out_dtype, int cu_count, int variant, int split_k,
              fbg_plan* out, int force_cfg) {
  if (!out) return FBG_ERROR_INVALID_VALUE;
  memset(out, 0, sizeof *out);
  out->split_k = 1;
  out->config = -1;
  if (M < 0 || N < 0 || K < 0 || split_k < 0) return FBG_ERROR_INVALID_VALUE;
  if (out_dtype != FBG_OUT_BF16 && out_dtype != FBG_OUT_FP16 && out_dtype != FBG_OUT_FP32)
    return FBG_ERROR_INVALID_VALUE;
  if (variant < FBG_VARIANT_AUTO || variant > FBG_VARIANT_SWAP_AB_SPLITK) return FBG_ERROR_INVALID_VALUE;
  if (K % 128 != 0) return FBG_ERROR_UNSUPPORTED;
  if (M > INT_MAX || N > INT_MAX || K > INT_MAX) return FBG_ERROR_UNSUPPORTED;
  const int cu = cu_count > 0 ? cu_count : 256;
  const int64_t G = K / 128;

  // Guards of forced variants: a forced path whose guard fails is an error,
  // never a silent fallback.
  if (variant == FBG_VARIANT_SHORT_K256 && K != 256) return FBG_ERROR_UNSUPPORTED;
  if (split_k > 1 && variant != FBG_VARIANT_SWAP_AB_SPLITK) return FBG_ERROR_UNSUPPORTED;
  if (split_k > G && G > 0) return FBG_ERROR_UNSUPPORTED;

  if (M == 0 || N == 0 || K == 0) {  // nothing to multiply: no GEMM kernel
    out->variant = variant;
    return FBG_SUCCESS;
  }

  int v = variant;
  if (v == FBG_VARIANT_AUTO) {
    // Swap-AB (maybe split over K below) for M <= 64, and up to M = 128 when
    // the generic kernel's smallest tile would leave over half the device idle.
    if (K == 256 && M <= 1024)
      v = FBG_VARIANT_SHORT_K256;
    else if (M <= 64 || (M <= 128 && cdiv(M, 64) * cdiv(N, 128) < (int64_t)cu / 2))
      v = FBG_VARIANT_SWAP_AB;
    else
      v = FBG_VARIANT_GENERIC;
  }

  out->variant = v;
  if (force_cfg >= 0) {  // test / benchmark override of the tile configuration
    const int n = v == FBG_VARIANT_GENERIC ? kNumGenericCfgs
                                           : (v == FBG_VARIANT_SHORT_K256 ? kNumShortCfgs : kNumSwapCfgs);
    if (force_cfg >= n) return FBG_ERROR_UNSUPPORTED;
  }
  if (v == FBG_VARIANT_GENERIC) {
    const int c = force_cfg >= 0 ? force_cfg : generic_cfg_for(M, N, cu);
    const GenericCfg& g = kGenericCfgs[c];
    out->config = c;
    out->tile_m = g.bm;
    out->tile_n = g.bn;
    out->waves = g.waves_m * g.waves_n;
    out->grid = cdiv(M, g.bm) * cdiv(N, g.bn);
  } else if (v == FBG_VARIANT_SHORT_K256) {
    const int c = force_cfg >= 0 ? force_cfg : short_cfg_for(M);
    const SkinnyCfg& k = kShortCfgs[c];
    out->config = c;
    out->tile_m = skinny_tile_m(k);
    out->tile_n = skinny_tile_n(k);
    out->waves = k.kw;
    out->grid = skinny_tiles(k, M, N);
  } else {  // SWAP_AB or SWAP_AB_SPLITK
    const int c = force_cfg >= 0 ? force_cfg : swap_cfg_for(M, N, cu);
    const SkinnyCfg& k = kSwapCfgs[c];
    const int64_t tiles = skinny_tiles(k, M, N);
    int64_t S = 1;
    if (split_k > 0) {
      S = split_k;
    } else if (variant == FBG_VARIANT_AUTO || variant == FBG_VARIANT_SWAP_AB_SPLITK) {
      // Split K until the grid covers the device once, keeping at least one
      // group per wave in every split.
      const int64_t want = cdiv(cu, tiles);
      const int64_t cap = G / k.kw > 1 ? G / k.kw : 1;
      S = want < cap ? want : cap;
      if (S < 1) S = 1;
    }
    if (variant == FBG_VARIANT_AUTO) v = S > 1 ? FBG_VARIANT_SWAP_AB_SPLITK : FBG_VARIANT_SWAP_AB;
    out->variant = v;
    out->config = c;
    out->tile_m = skinny_tile_m(k);
    out->tile_n = skinny_tile_n(k);
    out->waves = k.kw;
    out->split_k = (int32_t)S;
    out->grid = tiles * S;
  }
  if (out->grid > INT_MAX) return FBG_ERROR_UNSUPPORTED;
  out->workspace_bytes = workspace_bytes(*out, M, N);
  return FBG_SUCCESS;
}

int64_t workspace_counter_offset(const fbg_plan& p, int64_t M, int64_t N) {
  if (p.split_k <= 1 || p.tile_m <= 0 || p.tile_n <= 0) return 0;
  const int64_t T = cdiv(M, p.tile_m) * cdiv(N, p.tile_n);
  const int64_t partial = (int64_t)p.split_k * T * p.tile_m * p.tile_n * 4;
  return cdiv(partial, 256) * 256;
}

int64_t workspace_bytes(const fbg_plan& p, int64_t M, int64_t N) {
  if (p.split_k <= 1 || p.tile_m <= 0 || p.tile_n <= 0) return 0;
  const int64_t T = cdiv(M, p.tile_m) * cdiv(N, p.tile_n);
  return workspace_counter_offset(p, M, N) + T * 4;
}

// Grouped: by the mean number of tokens per expert -- 32 n x 16 m tiles
// (config 0) for decode-sized groups, 32 n x 32 m (config 1) up to 32, and
// 32 n x 64 m (config 2) above, so each expert's weight rows are streamed
// once per few token tiles.  force_cfg >= 0 picks a configuration; -1 is
// returned for one that does not exist.
int grouped_cfg_for(int64_t M, int64_t E, int64_t N, int64_t K, int force_cfg) {
  (void)N;
  (void)K;
  if (force_cfg >= 0) return force_cfg < kNumGroupedCfgs ? force_cfg : -1;
  const int64_t per = E > 0 ? cdiv(M, E) : M;
  if (per <= 16) return 0;
  if (per <= 32) return 1;
  return 2;
}

int64_t grouped_grid(int cfg, int64_t E, int64_t N) {
  return E * cdiv(N, skinny_tile_n(kGroupedCfgs[cfg]));
}

}  // namespace fbg

extern "C" int fp8_block_gemm_plan(int64_t M, int64_t N, int64_t K, int out_dtype, int cu_count, int variant,
                                   int split_k, fbg_plan* out) {
  return fbg::make_plan(M, N, K, out_dtype, cu_count, variant, split_k, out, -1);
}

extern "C" const char* fp8_block_gemm_status_string(int status) {
  switch (status) {
    case FBG_SUCCESS: return "success";
    case FBG_ERROR_INVALID_VALUE: return "invalid value (null pointer, negative size, bad dtype or overlapping output)";
    case FBG_ERROR_UNSUPPORTED: return "unsupported (K % 128 != 0, misaligned pointer, or a forced variant's guard failed)";
    case FBG_ERROR_OUT_OF_MEMORY: return "out of memory (split-K workspace unavailable or too small)";
    case FBG_ERROR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" int fp8_block_gemm_version(void) { return 100; }
