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

// Tile configurations and variant choice, from on-device sweeps (bench.py
// --sweep over the workloads, and --dispatch-sweep: every forced alternative
// on 108 shapes of the pages' sets N in {512, 1536, 4096, 8192}, K in {256,
// 1024, 4096}, M = 1 .. 4096).  What those sweeps show: each compute unit
// pulls its tiles' rows at a roughly fixed rate, so a launch costs about its
// busiest CU's rows x K; the split-K handshake (three memory round trips)
// costs ~1.5-2 us, more than splitting saves unless K is long and the
// unsplit grid fills at most half the device.
//
// Swap-AB (small M), its fragments staged through LDS: 16 n x 16 m tiles
// (config 2) up to three workgroups per CU, else 32 n x 16 m (config 7) up to
// two, else, for long K and M <= 64, 32 n x 64 m (config 19) where its grid
// leaves room to split K in two; none fits -> the generic kernel.  Measured
// (K = 4096): 16 x 16 beats 32 x 16 up to three workgroups per CU (N = 8192,
// M = 16: 9.7 us against 10.2 us) and loses past it (N = 4096, M = 64: 13.3
// us against 10.6 us); at two workgroups per CU the 32 x 16 tiles beat the
// generic kernel (N = 512, M = 512: 9.7 us against 12.2 us), at three they
// lose (N = 1536, M = 256: 15.8 us against 12.6 us).  Split over K only for
// K >= 2048, M > 1 and a grid of at most three quarters of the device, into
// enough splits for two workgroups per CU but at most 4 (decode N = 512,
// M = 64: 6.13 us in 4 splits, 6.17 us in 2, 6.78 us unsplit; M = 32:
// 5.74 us in 4 splits, 6.83 us unsplit; N = 512, M = 128, one workgroup per
// CU unsplit: 6.79 us against 6.89 us in 2; the benchmark's back-to-back
// replays over inputs rotated past the MALL).
//
// 12-64 groups with a 16 n x 8 m grid of at most one workgroup per CU: the
// single-stage tile with 8 activation rows (config 23, unsplit; a wave
// stages 4 groups at a time, so past 32 groups it reloads its area).  A
// single-stage workgroup's time follows its own bytes, not the grid's (K =
// 4096, 8 waves, cold: 5.62-5.75 us at 128 KB per workgroup for 32 to 256
// workgroups, 5.14 us at 96 KB, 4.37-4.42 us at 64 KB), and the 8-row tile
// moves 96 KB where the 16 x 16 one moves 128: N = 512, M = 64: 4.98 us
// against 5.64; M = 32: 4.91 against 5.75 (16 x 16 in 4 splits); M = 16:
// 4.96 against 5.31.  Up to 4 tokens it needs a grid of at most half the
// device (N = 512, M = 1 and 4: 4.40 and 4.73 against 4.63 and 4.93; N =
// 1536: 4.66 and 4.98 against 5.03 and 5.72 for config 11); a full-device
// grid of a few tokens loses (N = 4096, M = 1: 5.97 against 5.57 for config
// 11), and so does a grid past one workgroup per CU (N = 512, M = 128: 8.37
// against 5.66).
// Other K (N = 512, M = 64): 1536: 3.76 against 3.97 us; 2048: 4.05 against
// 4.59 unsplit and 5.87 in 4 splits; 6144: 6.12 against 7.00 in 4 splits;
// 8192: 6.96 against 7.45; 1024: 3.57 against 3.32 (not taken).  Past 32
// groups a grid of at most a quarter of the device splits better when a
// workspace is given (N = 512, K = 8192, M = 16: 6.47 us in 4 splits against
// 7.08).
// Else, with a 16 x 16 grid of at most one workgroup per CU:
// the single-stage tile (config 22: 8 waves x 4 groups, the workgroup's whole
// K range -- up to 128 KB -- in flight at once, one wait), unsplit.  Measured
// (K = 4096, cold): N = 512, M = 64: 5.67 us against 6.15 us for 16 x 16 in
// 4 splits; M = 128: 5.69 against 6.79 unsplit; N = 4096, M = 16: 6.93
// against 7.78.  Where that grid fills at most a quarter of the device and
// a workspace is available, splitting K over more workgroups still wins
// (N = 512, M = 16: 5.31 us in 4 splits against 5.77); a single token keeps
// the 8-wave register tile (config 11) unless its grid is that small
// (N = 4096, M = 1: 5.53 against 6.07; N = 512: 4.68 with config 22 against
// 4.92).
struct SwapPick {
  int cfg;
  int64_t S;
};

bool swap_pick(int64_t M, int64_t N, int64_t G, int cu, bool allow_split, SwapPick* out) {
  const int64_t W2 = cdiv(N, 16) * cdiv(M, 16), W7 = cdiv(N, 32) * cdiv(M, 16), W19 = cdiv(N, 32) * cdiv(M, 64);
  const int64_t W23 = cdiv(N, 16) * cdiv(M, 8);
  int64_t W;
  if (G >= 12 && G <= 64) {
    const bool small = 4 * W2 <= (int64_t)cu;
    const bool split_wins = G > 32 && M > 4 && 4 * W23 <= (int64_t)cu && allow_split;
    if (W23 <= (int64_t)cu && (M > 4 || 2 * W23 <= (int64_t)cu) && !split_wins) {
      out->cfg = 23;
      out->S = 1;
      return true;
    }
    if (G > 16 && G <= 32 && W2 <= (int64_t)cu && (M <= 4 ? small : !(small && allow_split))) {
      out->cfg = 22;
      out->S = 1;
      return true;
    }
  }
  if (W2 <= 3 * (int64_t)cu) {
    out->cfg = 2;
    W = W2;
  } else if (W7 <= 2 * (int64_t)cu) {
    out->cfg = 7;
    W = W7;
  } else if (G >= 16 && M <= 64 && 2 * W19 <= cu) {
    out->cfg = 19;
    W = W19;
  } else {
    return false;
  }
  out->S = 1;
  if (out->cfg == 2 && G >= 16 && M <= 4) {
    // A few tokens and long K: the same 16 x 16 tile with 8 waves, two groups
    // per chunk (config 11), unsplit -- more loads in flight per workgroup
    // (N = 4096, K = 4096, M = 1: 5.5-5.7 us against 6.5-6.6 us).
    out->cfg = 11;
    return true;
  }
  if (allow_split && G >= 16 && M > 1 && 4 * W <= 3 * (int64_t)cu) {
    const int64_t cap = G / kSwapCfgs[out->cfg].kw < 4 ? G / kSwapCfgs[out->cfg].kw : 4;
    const int64_t want = cdiv(2 * (int64_t)cu, W);
    out->S = want < cap ? want : cap;
    if (out->S < 1) out->S = 1;
  }
  return true;
}

// The configuration with the same tile as an 8-row one, with 16 activation
// rows (the single-stage tile 23 -> 22).
int sixteen_row_twin(int c) {
  const SkinnyCfg& k = kSwapCfgs[c];
  for (int i = 0; i < kNumSwapCfgs; ++i) {
    const SkinnyCfg& t = kSwapCfgs[i];
    if (t.one == 1 && t.nb16 == k.nb16 && t.mb16 == k.mb16 && t.kw == k.kw && t.gpw == k.gpw) return i;
  }
  return 2;
}

// Forced split-K without a split count: split until the grid covers the
// device once, keeping at least one group per wave in every split.
int64_t swap_split(const SkinnyCfg& k, int64_t tiles, int64_t G, int cu) {
  const int64_t want = cdiv(cu, tiles);
  const int64_t cap = G / k.kw > 1 ? G / k.kw : 1;
  const int64_t S = want < cap ? want : cap;
  return S < 1 ? 1 : S;
}

// The swap-AB tile when a variant is forced without a configuration and
// swap_pick finds none: 32 n x 64 m tiles (config 4) when they alone give
// every CU a workgroup, else 32 n x 16 m (config 7).
int swap_cfg_for(int64_t M, int64_t N, int64_t G, int cu) {
  SwapPick p;
  if (swap_pick(M, N, G, cu, true, &p)) return p.cfg;
  if (M > 16 && cdiv(N, 32) * cdiv(M, 64) >= (int64_t)cu) return 4;
  return 7;
}

// Short-K (K == 256, two groups, staged through LDS): 16 n x 16 m tiles with
// one group per wave (config 12) while their grid fits four workgroups per
// CU, else 32 n x 16 m (config 13) while that grid fits three; the
// automatic dispatch sends larger shapes to the generic kernel.  Measured
// (dispatch sweep, cold): 16 x 16 at four per CU beats the generic kernel
// (M = 32, N = 8192: 3.42 against 3.72 us; M = 64, N = 4096: 3.52 against
// 3.77; M = 512, N = 512: 3.38 against 3.69), 32 x 16 at three per CU too
// (M = 256, N = 1536: 3.57 against 3.78), and both lose past that (M = 128,
// N = 4096: 3.82 at best against 3.78; M = 1024, N = 512: 3.75 against
// 3.66; N = 8192, M = 512: 8.5 against 7.6).  A forced short-K launch of a
// larger shape takes 32 n x 32 m (config 15) up to M = 200, 32 n x 64 m
// (config 10) up to M = 256, else 32 n x 32 m with one wave taking both
// groups (config 6).
bool short_fits16(int64_t M, int64_t N, int cu) { return cdiv(N, 16) * cdiv(M, 16) <= 4 * (int64_t)cu; }
bool short_fits32(int64_t M, int64_t N, int cu) { return cdiv(N, 32) * cdiv(M, 16) <= 3 * (int64_t)cu; }
bool short_fits(int64_t M, int64_t N, int cu) { return short_fits16(M, N, cu) || short_fits32(M, N, cu); }

int short_cfg_for(int64_t M, int64_t N, int cu) {
  if (short_fits16(M, N, cu) || M <= 48) return 12;
  if (short_fits32(M, N, cu)) return 13;
  if (M <= 200) return 15;
  if (M <= 256) return 10;
  return 6;
}

// Generic: a launch costs about (workgroups per CU) x (BM + BN) x K bytes
// per CU, so the planner takes the configuration with the fewest such bytes;
// on a tie, the larger tile (more MFMA work per LDS byte, fewer workgroups),
// then, for K >= 2048, the deeper LDS ring (64 x 128 with 4 stages over
// 128 x 64 with 3: K = 4096, N = 4096, M = 512 in 25.0 us against 26.9 us),
// else more waves.  For large M this is the 256 x 256 tile; in the mid-M
// band it picks the small tiles that put a workgroup on every CU (measured:
// M = 128, N = 8192, K = 1024 runs in 6.8 us with 64 x 64 tiles against
// 9.3 us with 64 x 128).  Where the 128 x 256 tile (8 waves, 3-slot ring)
// ties with 256 x 128 (4 waves) it wins on the waves (dispatch sweep, cold:
// M = 4096, N = 1536, K = 1024: 15.8 against 18.5 us; M = 1024, N = 8192,
// K = 1024: 17.7 against 19.3 us; K = 4096: 45.3 against 49.1 and 50.2
// against 50.4 us).
int64_t generic_cost(const GenericCfg& g, int64_t M, int64_t N, int cu) {
  const int64_t wgs = cdiv(M, g.bm) * cdiv(N, g.bn);
  return cdiv(wgs, cu) * (g.bm + g.bn);
}

// The configurations the dense planner weighs (0-7; configurations 8-11
// replace 3, 4, 2 and 0 where they measured faster).
constexpr int kNumDenseGenericCfgs = 8;

int generic_cfg_for(int64_t M, int64_t N, int64_t G, int cu) {
  int best = 0;
  for (int c = 1; c < kNumDenseGenericCfgs; ++c) {
    const GenericCfg& g = kGenericCfgs[c];
    const GenericCfg& b = kGenericCfgs[best];
    const int64_t cg = generic_cost(g, M, N, cu), cb = generic_cost(b, M, N, cu);
    bool better = cg < cb;
    if (cg == cb) {
      if (g.bm * g.bn != b.bm * b.bn)
        better = g.bm * g.bn > b.bm * b.bn;
      else if (G >= 16 && g.stages != b.stages)
        better = g.stages > b.stages;
      else
        better = g.waves_m * g.waves_n > b.waves_m * b.waves_n;
    }
    if (better) best = c;
  }
  // The 256 x 256 tile with its refill split at mid-group (configuration 8):
  // prefill 16384 x 4096 x 4096 in 276 against 288 us (bf16), 294 against
  // 305 us (fp32), interleaved runs on one box.  The 64 x 64 tile with 2 x 2
  // waves (configuration 9) where the 2-wave one wins the cost: 1.6-3.9%
  // faster at every such shape of the dispatch sweep (cold: 128 x 8192 x
  // 1024 6.22 against 6.42 us; 184 x 4096 x 256 3.93 against 4.06; 512 x
  // 1536 x 4096 14.56 against 15.15; 256 x 4096 x 1024 5.99 against 6.24).
  // The 64 x 128 tile with 2 x 2 waves (configuration 10) where the 2-wave
  // one wins: 4-7% faster at every such shape (K = 4096: 1024 x 1536 20.6
  // against 22.0 us; 512 x 4096 21.7 against 23.0; 4096 x 512 21.4 against
  // 22.9).  The 128 x 128 tile with 8 waves (configuration 11) for K of at
  // most 1024 (1024 x 4096 x 256 7.09 against 7.53 us; 512 x 8192 x 1024
  // 11.58 against 11.98); at K = 4096 it loses (33.4 against 30.5 us).
  if (best == 3) return 8;
  if (best == 4) return 9;
  if (best == 2) return 10;
  if (best == 0 && G <= 8) return 11;
  return best;
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
  SwapPick pick{7, 1};
  // split_k = 1 under AUTO: the best plan without a K split (no workspace).
  const bool allow_split = !(variant == FBG_VARIANT_AUTO && split_k == 1);
  const bool picked = swap_pick(M, N, G, cu, allow_split, &pick);
  if (v == FBG_VARIANT_AUTO) {
    // K == 256: the swap-AB 16x16 tile (configuration 2, the two groups on
    // two of its four waves) while its grid is at most one workgroup per CU
    // (for M = 1 only up to 512 columns), then short-K while its 16x16 or
    // 32x16 grid fits, else generic.  The swap-AB tile measured 1-4% faster
    // there (interleaved runs, cold: 16x512x256 3.00 against 3.11 us for
    // short-K, 32x512 3.00 / 3.09, 64x512 3.02 / 3.07, 16x1536 3.05 / 3.09;
    // dispatch sweeps: 128x512, 32x1536, 16x4096 likewise, 1x512 2.87-2.89
    // against 2.96-2.99 in three runs), and not at M = 1 with 1536 or 4096
    // columns (0.6-0.8% slower) or past one workgroup per CU (32x4096 3.35
    // against 3.21).  Otherwise swap-AB for M <= 16 and, up to M = 512, when
    // swap_pick finds a tile; the generic kernel for the rest.
    if (K == 256 && M <= 1024)
      v = ((M > 1 || N <= 512) && cdiv(N, 16) * cdiv(M, 16) <= (int64_t)cu) ? FBG_VARIANT_SWAP_AB
          : short_fits(M, N, cu)                             ? FBG_VARIANT_SHORT_K256
                                                             : FBG_VARIANT_GENERIC;
    else if (M <= 16 || (M <= 512 && picked))
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
    const int c = force_cfg >= 0 ? force_cfg : generic_cfg_for(M, N, G, cu);
    const GenericCfg& g = kGenericCfgs[c];
    out->config = c;
    out->tile_m = g.bm;
    out->tile_n = g.bn;
    out->waves = g.waves_m * g.waves_n;
    out->grid = cdiv(M, g.bm) * cdiv(N, g.bn);
  } else if (v == FBG_VARIANT_SHORT_K256) {
    const int c = force_cfg >= 0 ? force_cfg : short_cfg_for(M, N, cu);
    const SkinnyCfg& k = kShortCfgs[c];
    out->config = c;
    out->tile_m = skinny_tile_m(k);
    out->tile_n = skinny_tile_n(k);
    out->waves = k.kw;
    out->grid = skinny_tiles(k, M, N);
  } else {  // SWAP_AB or SWAP_AB_SPLITK
    int c = force_cfg >= 0 ? force_cfg : (picked ? pick.cfg : swap_cfg_for(M, N, G, cu));
    // A split asked for without a configuration: the 8-row tile's 16-row
    // counterpart, whose partials the split-K workspace holds.
    if (force_cfg < 0 && kSwapCfgs[c].one == 2 && (split_k > 1 || variant == FBG_VARIANT_SWAP_AB_SPLITK))
      c = sixteen_row_twin(c);
    const SkinnyCfg& k = kSwapCfgs[c];
    const int64_t tiles = skinny_tiles(k, M, N);
    int64_t S = 1;
    if (split_k > 0) {
      S = split_k;
    } else if (variant == FBG_VARIANT_AUTO) {
      // The picked split (or none) when the picked tile is used.
      S = (picked && c == pick.cfg) ? pick.S : 1;
    } else if (variant == FBG_VARIANT_SWAP_AB_SPLITK) {
      S = swap_split(k, tiles, G, cu);  // forced split-K: fill the device
    }
    // Tiles of 8 activation rows keep their partials in 16-row blocks: they
    // never split over K.
    if (k.one == 2 && S > 1) return FBG_ERROR_UNSUPPORTED;
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

// Grouped: by the mean number of tokens per expert (measured on 256 experts
// of 512 x 4096, 16 .. 4096 tokens routed top-8).  Up to 12: 32-column tiles
// of one 16-row block with the K range split over 8 waves (config 5: the
// weight stream is the whole cost, and 8 waves keep the most loads in
// flight); up to 20: 32 x 32 tiles (config 1); up to 48: 64-column tiles of
// up to 64 rows (config 6), which cut the activation re-reads (one per
// column tile) 2x and stream each weight tile once for experts of up to 64
// tokens.  Skinny tiles compute only their 16-row blocks that hold tokens.
// Up to 96: the generic kernel's 128 x 256 tiles (8 waves, 3-slot ring) in
// grouped mode, one row tile per expert (2048 tokens, 47-87 per expert:
// 209.6 us against 222.7 us in config 6 and 231 us in 256 x 256); above
// (prefill-sized experts), its 256 x 256 tiles: 4096 tokens run in 242 us
// against 275 us in 128 x 256 (a second row tile re-reads the weight) and
// 353-511 us in every other tile.
int grouped_num_cfgs() { return kNumGroupedCfgs + kNumGroupedGenericCfgs; }
int grouped_num_skinny_cfgs() { return kNumGroupedCfgs; }

int grouped_cfg_for(int64_t M, int64_t E, int64_t N, int64_t K, int force_cfg) {
  (void)N;
  (void)K;
  if (force_cfg >= 0) return force_cfg < grouped_num_cfgs() ? force_cfg : -1;
  const int64_t per = E > 0 ? cdiv(M, E) : M;
  if (per <= 12) return 5;
  if (per <= 20) return 1;
  if (per <= 48) return 6;
  if (per <= 96) return kNumGroupedCfgs + 7;  // generic 128 x 256
  return kNumGroupedCfgs + 3;                 // generic 256 x 256
}

int64_t grouped_grid(int cfg, int64_t E, int64_t M, int64_t N) {
  if (cfg < kNumGroupedCfgs) return E * cdiv(N, skinny_tile_n(kGroupedCfgs[cfg]));
  const GenericCfg& g = kGenericCfgs[cfg - kNumGroupedCfgs];
  return (cdiv(M, g.bm) + E) * cdiv(N, g.bn);
}

}  // namespace fbg

extern "C" int fp8_block_gemm_plan(int64_t M, int64_t N, int64_t K, int out_dtype, int cu_count, int variant,
                                   int split_k, fbg_plan* out) {
  return fbg::make_plan(M, N, K, out_dtype, cu_count, variant, split_k, out, -1);
}

extern "C" int fp8_block_gemm_grouped_plan(int64_t E, int64_t M, int64_t N, int64_t K, fbg_plan* out) {
  if (!out || E < 0 || M < 0 || N < 0 || K < 0) return FBG_ERROR_INVALID_VALUE;
  if (K % 128 != 0) return FBG_ERROR_UNSUPPORTED;
  const int cfg = fbg::grouped_cfg_for(M, E, N, K, -1);
  memset(out, 0, sizeof(*out));
  out->variant = FBG_VARIANT_GROUPED;
  if (cfg < fbg::kNumGroupedCfgs) {
    const fbg::SkinnyCfg& k = fbg::kGroupedCfgs[cfg];
    out->tile_m = fbg::skinny_tile_m(k);
    out->tile_n = fbg::skinny_tile_n(k);
    out->waves = k.kw;
  } else {
    const fbg::GenericCfg& g = fbg::kGenericCfgs[cfg - fbg::kNumGroupedCfgs];
    out->tile_m = g.bm;
    out->tile_n = g.bn;
    out->waves = g.waves_m * g.waves_n;
  }
  out->split_k = 1;
  out->config = cfg;
  out->grid = fbg::grouped_grid(cfg, E, M, N);
  out->workspace_bytes = 0;
  return FBG_SUCCESS;
}

extern "C" const char* fp8_block_gemm_status_string(int status) {
  switch (status) {
    case FBG_SUCCESS: return "success";
    case FBG_ERROR_INVALID_VALUE: return "invalid value (null pointer, negative size, bad dtype or overlapping output)";
    case FBG_ERROR_UNSUPPORTED: return "unsupported (K % 128 != 0, misaligned pointer, or a forced variant's guard failed)";
    case FBG_ERROR_OUT_OF_MEMORY: return "out of memory (split-K workspace unavailable or too small)";
    case FBG_ERROR_HIP: return "HIP runtime error";
    case FBG_ERROR_SCRATCH_LIMIT:
      return "scratch limit (the split-K partials or tile count exceed fp8_block_gemm_noalloc's 4 MiB static scratch)";
    default: return "unknown status";
  }
}

extern "C" int fp8_block_gemm_version(void) { return 100; }
