// Kernel configurations of each variant.  One X-macro list per variant feeds
// both the host planner's table (which chooses a configuration) and the
// launchers' switch (which maps it to a template instance), so the two
// cannot disagree on a tile shape.  Plain host/device-neutral C++.
#pragma once

namespace fbg {

// Generic LDS-staged kernel: id, block tile BM x BN, waves WAVES_M x WAVES_N,
// LDS ring depth in groups, row-scale staging (1: chunks of several groups
// per row, loaded a few rows' runs per instruction; 0: one load per row and
// group, staged in the ring slot), mid-group refill (1: most of a group's
// refill goes out after a second barrier in the middle of the group, spread
// over several row blocks; the 256 x 256 tile).  Configuration 7 (128 x 256,
// 8 waves) serves the grouped GEMM (experts of ~50-100 rows) and the dense
// planner where it ties with 256 x 128.  Configuration 8 (configuration 3 with the mid-group refill:
// the dense planner takes it wherever it would take configuration 3) and 9
// (configuration 4's 64 x 64 tile with 2 x 2 waves of 32 x 32, so all four
// SIMDs run MFMAs; the dense planner takes it wherever it would take
// configuration 4), 10 (configuration 2's 64 x 128 tile with 2 x 2 waves)
// and 11 (configuration 0's 128 x 128 tile with 8 waves, taken for K of at
// most 1024) serve only the dense planner; the grouped GEMM offers 0-7
// (the mid-group refill measured slower there: the 4096-token MoE workload
// 259 -> 305 us).
#define FBG_GENERIC_CFGS(X)     \
  X(0, 128, 128, 2, 2, 4, 0, 0) \
  X(1, 256, 128, 2, 2, 3, 0, 0) \
  X(2, 64, 128, 1, 2, 4, 0, 0)  \
  X(3, 256, 256, 2, 4, 2, 1, 0) \
  X(4, 64, 64, 1, 2, 4, 0, 0)   \
  X(5, 128, 64, 2, 2, 3, 0, 0)  \
  X(6, 64, 32, 1, 2, 4, 0, 0)   \
  X(7, 128, 256, 2, 4, 3, 0, 0) \
  X(8, 256, 256, 2, 4, 2, 1, 1) \
  X(9, 64, 64, 2, 2, 4, 0, 0)   \
  X(10, 64, 128, 2, 2, 4, 0, 0) \
  X(11, 128, 128, 2, 4, 4, 0, 0)

// Skinny kernels (swap-AB and its split-K form): id, NB16 16-row blocks of
// weight rows (output columns n), MB16 16-column blocks of activation rows
// (output rows m), KW waves splitting the workgroup's K range, GPW groups
// per wave per chunk, ONE: 1 -- every wave stages its chunks through a single
// LDS area, the whole chunk's loads in flight at once (configurations whose
// KW * GPW groups cover a launch's K range, so a wave loads once, waits
// once); 2 -- the same with tiles of 8 activation rows (16 n x 8 m: the
// MFMA's activation rows 8-15 are computed but never stored), which such a
// tile never splits over K.
#define FBG_SWAP_CFGS(X) \
  X(0, 1, 4, 4, 1, 0)    \
  X(1, 1, 4, 1, 2, 0)    \
  X(2, 1, 1, 4, 1, 0)    \
  X(3, 1, 2, 4, 1, 0)    \
  X(4, 2, 4, 2, 1, 0)    \
  X(5, 1, 8, 4, 1, 0)    \
  X(6, 4, 1, 4, 1, 0)    \
  X(7, 2, 1, 4, 1, 0)    \
  X(8, 1, 4, 2, 2, 0)    \
  X(9, 2, 2, 4, 1, 0)    \
  X(10, 1, 1, 16, 2, 0)  \
  X(11, 1, 1, 8, 2, 0)   \
  X(12, 2, 8, 4, 1, 0)   \
  X(13, 1, 8, 8, 1, 0)   \
  X(14, 1, 4, 8, 1, 0)   \
  X(15, 1, 2, 8, 2, 0)   \
  X(16, 2, 1, 8, 1, 0)   \
  X(17, 4, 1, 8, 1, 0)   \
  X(18, 1, 4, 4, 2, 0)   \
  X(19, 2, 4, 4, 1, 0)   \
  X(20, 1, 1, 4, 4, 0)   \
  X(21, 2, 1, 4, 2, 0)   \
  X(22, 1, 1, 8, 4, 1)   \
  X(23, 1, 1, 8, 4, 2)

// Short-K (K == 256, two groups, fully unrolled): same fields, KW * GPW == 2.
#define FBG_SHORT_CFGS(X) \
  X(0, 1, 4, 1, 2)        \
  X(1, 2, 4, 1, 2)        \
  X(2, 1, 1, 1, 2)        \
  X(3, 1, 2, 1, 2)        \
  X(4, 4, 1, 1, 2)        \
  X(5, 1, 4, 2, 1)        \
  X(6, 2, 2, 1, 2)        \
  X(7, 1, 8, 2, 1)        \
  X(8, 2, 12, 2, 1)       \
  X(9, 1, 12, 2, 1)       \
  X(10, 2, 4, 2, 1)       \
  X(11, 4, 4, 2, 1)       \
  X(12, 1, 1, 2, 1)       \
  X(13, 2, 1, 2, 1)       \
  X(14, 1, 2, 2, 1)       \
  X(15, 2, 2, 2, 1)

// Grouped (mixture-of-experts) kernel: same fields as the skinny kernels.
#define FBG_GROUPED_CFGS(X) \
  X(0, 2, 1, 4, 1)          \
  X(1, 2, 2, 4, 1)          \
  X(2, 2, 4, 2, 1)          \
  X(3, 1, 1, 4, 1)          \
  X(4, 4, 1, 4, 1)          \
  X(5, 2, 1, 8, 1)          \
  X(6, 4, 4, 2, 1)          \
  X(7, 4, 2, 4, 1)          \
  X(8, 2, 4, 4, 1)          \
  X(9, 4, 4, 4, 1)          \
  X(10, 8, 2, 2, 1)

struct GenericCfg { int bm, bn, waves_m, waves_n, stages, scale_chunks, mid_refill; };
constexpr GenericCfg kGenericCfgs[] = {
#define X(id, bm, bn, wm, wn, st, sch, mid) {bm, bn, wm, wn, st, sch, mid},
    FBG_GENERIC_CFGS(X)
#undef X
};
constexpr int kNumGenericCfgs = sizeof(kGenericCfgs) / sizeof(kGenericCfgs[0]);
constexpr int kNumGroupedGenericCfgs = 8;  // generic configurations the grouped GEMM may run (0-7)

struct SkinnyCfg { int nb16, mb16, kw, gpw, one = 0; };
constexpr SkinnyCfg kSwapCfgs[] = {
#define X(id, nb, mb, kw, gpw, one) {nb, mb, kw, gpw, one},
    FBG_SWAP_CFGS(X)
#undef X
};
constexpr int kNumSwapCfgs = sizeof(kSwapCfgs) / sizeof(kSwapCfgs[0]);

constexpr SkinnyCfg kShortCfgs[] = {
#define X(id, nb, mb, kw, gpw) {nb, mb, kw, gpw},
    FBG_SHORT_CFGS(X)
#undef X
};
constexpr int kNumShortCfgs = sizeof(kShortCfgs) / sizeof(kShortCfgs[0]);

constexpr SkinnyCfg kGroupedCfgs[] = {
#define X(id, nb, mb, kw, gpw) {nb, mb, kw, gpw},
    FBG_GROUPED_CFGS(X)
#undef X
};
constexpr int kNumGroupedCfgs = sizeof(kGroupedCfgs) / sizeof(kGroupedCfgs[0]);

inline int skinny_tile_n(const SkinnyCfg& c) { return 16 * c.nb16; }
inline int skinny_tile_m(const SkinnyCfg& c) { return c.one == 2 ? 8 : 16 * c.mb16; }

}  // namespace fbg
