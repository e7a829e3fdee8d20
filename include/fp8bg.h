/*
 * fp8bg.h -- C ABI of the block-scaled FP8 GEMM library for AMD MI355X (gfx950).
 *
 * The operation (FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8 matmul
 * for Hopper", section "Description": FP8 E4M3 activations with per-token
 * 1x128 scales, FP8 E4M3 weights with [block_n, block_k] = [128, 128] scales;
 * section "Numerical safety": FP32 accumulation on every kernel path, then one
 * rounding to the bf16, fp16 or fp32 result):
 *
 *     C[m,n] = sum_g a_s[m,g] * b_s[n/128, g] * sum_{k = 128g}^{128g+127} A[m,k] * B[n,k]
 *
 * Layouts (all row-major, contiguous, no strides -- the same section's guard
 * requires contiguous strides and group_k == 128):
 *   A    [M, K]               OCP FP8 E4M3 bytes (torch.float8_e4m3fn)
 *   a_s  [M, K/128]           fp32, per-token, per 128-wide K group
 *   B    [N, K]               OCP FP8 E4M3 bytes (the weight W of y = x W^T)
 *   b_s  [ceil(N/128), K/128] fp32, per 128x128 weight block
 *   C    [M, N]               bf16 / fp16 / fp32 (out_dtype)
 *
 * Pointers are device pointers on the current HIP device unless a function
 * says otherwise.  The caller owns every buffer; the library reads A, a_s, B,
 * b_s, writes exactly C[0 .. M*N) and never reads C (no beta, no zero-fill
 * requirement).  All calls are asynchronous on `stream` (a hipStream_t passed
 * as void*, NULL = the null stream); device-side faults surface at the
 * caller's next synchronisation.  No function throws or aborts.
 *
 * Numerics: each kernel forms the fresh FP32 partial of one 128-wide group on
 * the MFMA units, then folds it as acc = fma(P, a_s*b_s, acc) in group order;
 * the cast to the output dtype is round-to-nearest-even.  Every call is
 * deterministic: the same inputs give the same bits on every run and stream.
 *
 * Environment variables (tuning and test hooks, read on every call; unset in
 * normal use): FBG_FORCE_CONFIG=<i> pins the tile configuration index of the
 * chosen variant (for fp8_block_gemm_grouped, the grouped configuration
 * index); an index that does not exist -> UNSUPPORTED.  FBG_RASTER_BAND=<rows>
 * sets the generic kernel's raster band height (default 8).  FBG_LOG=1
 * prints each call's plan to stderr.  FBG_TEST_FAIL_ALLOC=1 makes the
 * library-owned split-K workspace allocation fail (OUT_OF_MEMORY), for tests.
 */
#ifndef FP8BG_H
#define FP8BG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    FBG_SUCCESS = 0,
    FBG_ERROR_INVALID_VALUE = 1,  /* null pointer, negative size, bad dtype, C overlapping an input */
    FBG_ERROR_UNSUPPORTED = 2,    /* K % 128 != 0, misaligned pointer, a forced variant whose guard fails */
    FBG_ERROR_OUT_OF_MEMORY = 3,  /* split-K workspace could not be allocated / is too small */
    FBG_ERROR_HIP = 4,            /* a HIP runtime call or kernel launch failed */
    FBG_ERROR_SCRATCH_LIMIT = 5   /* fp8_block_gemm_noalloc: the split needs more than its static scratch */
};

/* Output dtypes. */
enum { FBG_OUT_BF16 = 0, FBG_OUT_FP16 = 1, FBG_OUT_FP32 = 2 };

/* Kernel variants (the four specialised paths of the section "Specialized
 * kernels and the optimization idea", re-designed for gfx950). */
enum {
    FBG_VARIANT_AUTO = 0,          /* the (M,N,K) dispatcher chooses */
    FBG_VARIANT_GENERIC = 1,       /* LDS-staged MFMA tiles, any shape */
    FBG_VARIANT_SHORT_K256 = 2,    /* K == 256: both groups unrolled, a_s*b_s pre-folded */
    FBG_VARIANT_SWAP_AB = 3,       /* C^T = B A^T: weight rows on the 16-row MFMA side, small M on the other */
    FBG_VARIANT_SWAP_AB_SPLITK = 4, /* swap-AB with K split over workgroups, fixed-order FP32 reduction */
    FBG_VARIANT_GROUPED = 5        /* reported by fp8_block_gemm_grouped_plan only; not a forcible variant */
};

/* One dispatcher decision (pure data, filled by fp8_block_gemm_plan). */
typedef struct fbg_plan {
    int32_t variant;      /* FBG_VARIANT_* actually used */
    int32_t tile_m;       /* output rows (M) per workgroup */
    int32_t tile_n;       /* output columns (N) per workgroup */
    int32_t split_k;      /* number of K splits (1 = none) */
    int32_t waves;        /* wavefronts (64 lanes) per workgroup */
    int32_t config;       /* kernel configuration index within the variant */
    int64_t grid;         /* workgroups launched */
    int64_t workspace_bytes; /* device workspace the call needs (0 if none) */
} fbg_plan;

/*
 * fp8_block_gemm -- C = block-scaled A * B^T, dispatcher-chosen kernel.
 *
 * M, N >= 0; K >= 0 with K % 128 == 0.  M == 0 or N == 0: success, nothing
 * launched.  K == 0: C is filled with zeros (the empty sum).  A and B must be
 * 16-byte aligned, a_s and b_s 4-byte aligned, C aligned to its element size.
 * A null pointer with a non-empty extent, a negative size, an unknown
 * out_dtype or a C range that overlaps an input range -> INVALID_VALUE;
 * K % 128 != 0, misalignment, M or N above INT32_MAX, K above 2^24 - 128
 * (the kernels' 32-bit offsets inside a tile's rows), or a scale array of 4 GiB
 * or more -> UNSUPPORTED.  The dispatcher's variant and tile are used
 * without a K split (the plan of fp8_block_gemm_plan with split_k = 1), so
 * the call needs no workspace and never allocates; it may be captured in a
 * HIP graph as it is.  Callers that want the split-K plan where the
 * dispatcher takes it pass a workspace to fp8_block_gemm_ex, or use
 * fp8_block_gemm_noalloc.
 */
int fp8_block_gemm(const void *A, const float *a_s, const void *B, const float *b_s,
                   void *C, int64_t M, int64_t N, int64_t K, int out_dtype, void *stream);

/*
 * fp8_block_gemm_ex -- the same operation with a forced variant and an
 * explicit workspace (for tests, benchmarks and stream capture).
 *
 * variant: FBG_VARIANT_* (AUTO = as fp8_block_gemm).  A forced variant whose
 * shape guard fails returns UNSUPPORTED; it never falls back silently.
 * split_k: 0 = the dispatcher's choice, else the number of K splits (only
 * SWAP_AB_SPLITK accepts > 1; it must not exceed K/128).
 * workspace / workspace_bytes: caller-owned device memory of at least
 * fp8_block_gemm_workspace_size(...) bytes, or NULL.  With NULL, AUTO and
 * split_k == 0 plan as fp8_block_gemm does (no K split, nothing allocated);
 * a split forced without a workspace takes it from a stream-ordered
 * allocation on `stream` (hipMallocAsync / hipFreeAsync, so concurrent calls
 * on different streams never share one; its counters zeroed by a small
 * kernel, no hipMemsetAsync; ~15-20 us per call, also as graph nodes under
 * capture; failure -> OUT_OF_MEMORY before anything is launched).  The
 * workspace holds FP32 partials and one
 * 32-bit arrival counter per output tile; the counters must be zero before
 * the first call that uses the buffer, and every completed call leaves them
 * zero again, so a buffer zeroed once can be reused by calls that are
 * ordered on one stream.  Calls that overlap in time must not share one.
 */
int fp8_block_gemm_ex(const void *A, const float *a_s, const void *B, const float *b_s,
                      void *C, int64_t M, int64_t N, int64_t K, int out_dtype, void *stream,
                      int variant, int split_k, void *workspace, size_t workspace_bytes);

/*
 * fp8_block_gemm_noalloc -- fp8_block_gemm_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same operation, arguments, variant and
 * split_k rules and statuses as fp8_block_gemm_ex, with the dispatcher's
 * split-K plan kept (as with a caller workspace); the split's FP32 partials
 * and arrival counters live in a static array of 4 MiB per GPU that the
 * library holds until the process ends (16 KiB of counters -- at most 4096
 * output tiles -- and the rest for partials; the automatic plans need at most
 * ~0.7 MB).  The call never calls hipMalloc, hipFree or any allocating
 * routine.  A split whose partials or tile count exceed the array ->
 * FBG_ERROR_SCRATCH_LIMIT, nothing launched.  The first call on a device
 * looks the array's address up and clears its counters with a kernel on
 * `stream`; every completed call leaves them zero.  All calls on one GPU
 * share its array: calls that overlap in time on one GPU (different streams,
 * or a graph replayed concurrently with another call) race and must not be
 * made; calls ordered on one stream are safe.
 */
int fp8_block_gemm_noalloc(const void *A, const float *a_s, const void *B, const float *b_s,
                           void *C, int64_t M, int64_t N, int64_t K, int out_dtype, void *stream,
                           int variant, int split_k);

/*
 * fp8_block_gemm_workspace_size -- bytes of workspace fp8_block_gemm_ex needs
 * for this shape, variant and split (0 when the chosen kernel needs none).
 * variant / split_k as in fp8_block_gemm_ex; when either is left to the
 * dispatcher the plan uses the current device's compute-unit count (one
 * cached HIP query).  Returns (size_t)-1 for an invalid request.
 */
size_t fp8_block_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int variant, int split_k);

/*
 * fp8_block_gemm_plan -- the dispatcher's decision for (M, N, K, out_dtype)
 * on a device with cu_count compute units (the pages' dispatch routes each
 * shape by (M, N, K) to the best-fit kernel, with the generic kernel as the
 * fallback: section "Description").  Pure host code: makes no HIP call, so
 * it can run without a GPU.  variant / split_k force a choice as in
 * fp8_block_gemm_ex; FBG_FORCE_CONFIG is not read here (the plan shows the
 * automatic tile configuration).  Returns SUCCESS and fills *out, or an
 * error status.
 */
int fp8_block_gemm_plan(int64_t M, int64_t N, int64_t K, int out_dtype, int cu_count,
                        int variant, int split_k, fbg_plan *out);

/*
 * fp8_block_gemm_grouped -- the grouped (mixture-of-experts) form: E experts
 * with their own weights, the tokens grouped by expert (the first page's
 * section "Description" names the MoE-style traffic these GEMMs serve; the
 * MoE kernel page, section "Summary", its per-expert token groups and decode
 * swap-AB path).  For every expert e and row m in [offsets[e], offsets[e+1]):
 *
 *     C[m,n] = sum_g a_s[m,g] * b_s[e, n/128, g] * sum_{k in group g} A[m,k] * B[e,n,k]
 *
 * A [M,K], a_s [M,K/128] and C [M,N] as for fp8_block_gemm; B [E,N,K] E4M3
 * (expert e's weight at B + e*N*K), b_s [E, ceil(N/128), K/128] fp32.
 * offsets: DEVICE pointer to E+1 int32, non-decreasing, offsets[0] = 0,
 * offsets[E] = M (typically written by the router on the GPU, so the call
 * never synchronises with the host).  The kernels clamp every offset into
 * [0, M]: malformed offsets can leave rows of C unwritten (or, for ranges
 * that overlap, written by more than one expert) but never make a kernel
 * read or write outside A, a_s, B, b_s or C.  Rows of C outside every
 * expert's range are not written.  Small experts run on skinny swap-AB
 * tiles (one workgroup per expert and column tile); prefill-sized experts
 * on the LDS-staged generic kernel, whose workgroups find their expert and
 * row tile with a scan of the offsets on the device.  M, N, K, E >= 0 with K % 128 == 0; M == 0 or
 * N == 0: nothing launched; K == 0 or E == 0: C is filled with zeros.
 * Alignment as for fp8_block_gemm, offsets 4-byte aligned; statuses as for
 * fp8_block_gemm (C overlapping any input -> INVALID_VALUE).  No workspace;
 * asynchronous on `stream`; deterministic.
 */
int fp8_block_gemm_grouped(const void *A, const float *a_s, const void *B, const float *b_s, void *C,
                           const int32_t *offsets, int64_t E, int64_t M, int64_t N, int64_t K,
                           int out_dtype, void *stream);

/*
 * fp8_block_gemm_grouped_plan -- the tile configuration fp8_block_gemm_grouped
 * uses for E experts holding M token rows in total (chosen by the mean rows
 * per expert), as a plan: variant FBG_VARIANT_GROUPED, tile_m = the most
 * token rows a tile holds (a tile computes only its 16-row blocks that hold
 * tokens), tile_n, waves, config, split_k 1, no workspace; grid = E *
 * ceil(N / tile_n) workgroups for the skinny tiles (those of empty experts
 * exit at once), (ceil(M / tile_m) + E) * ceil(N / tile_n) for the generic
 * kernel's tiles in grouped mode (the experts' row tiles fit in that bound;
 * surplus workgroups exit at once).  Pure host code.  Negative sizes ->
 * INVALID_VALUE; K % 128 != 0 -> UNSUPPORTED.
 */
int fp8_block_gemm_grouped_plan(int64_t E, int64_t M, int64_t N, int64_t K, fbg_plan *out);

/*
 * fp8_block_gemm_quantize_rows -- the producer of A and a_s: per-token 1x128
 * quantisation of bf16 activations to OCP E4M3 (the section "Description"
 * gives the GEMM per-token FP8 E4M3 activations with one de-quant scale per
 * 128-wide K group; the scale maps each group's largest magnitude onto
 * E4M3's largest finite value, 448).  For every row m and group g:
 *
 *     a_s[m,g] = max(max_{k in g} |x[m,k]|, 1e-12f) / 448        (fp32 division)
 *     A[m,k]   = E4M3 round-to-nearest-even of clamp(x[m,k] / a_s[m,g], -448, 448)
 *
 * with x[m,k] / a_s[m,g] an IEEE fp32 (correctly rounded) division.
 * x: [M,K] bf16, row-major, 16-byte aligned (read); A: [M,K] E4M3 bytes,
 * 8-byte aligned, and a_s: [M, K/128] fp32, 4-byte aligned (written in full).
 * The caller owns all three; outputs must not overlap x or each other.
 * M, K >= 0 with K % 128 == 0; M == 0 or K == 0: success, nothing launched.
 * A null pointer with a non-empty extent, a negative size or overlapping
 * buffers -> INVALID_VALUE; K % 128 != 0 or misalignment -> UNSUPPORTED.
 * NaN or infinite inputs are outside the contract.  Asynchronous on
 * `stream`; deterministic.
 */
int fp8_block_gemm_quantize_rows(const void *x, int64_t M, int64_t K, void *A, float *a_s, void *stream);

/*
 * fp8_block_gemm_quantize_blocks -- the producer of B and b_s: 128x128
 * block quantisation of bf16 weights to OCP E4M3 (the section "Description"
 * gives the GEMM FP8 E4M3 weights with [block_n, block_k] = [128, 128]
 * de-quant scales; the scale maps each block's largest magnitude onto 448).
 * For every block (nb, g) -- rows 128nb .. min(128nb+128, N), columns
 * 128g .. 128g+128:
 *
 *     b_s[nb,g] = max(max over the block of |w[n,k]|, 1e-12f) / 448     (fp32 division)
 *     B[n,k]    = E4M3 round-to-nearest-even of clamp(w[n,k] / b_s[nb,g], -448, 448)
 *
 * with w[n,k] / b_s an IEEE fp32 (correctly rounded) division.
 * w: [N,K] bf16, row-major, 16-byte aligned (read); B: [N,K] E4M3 bytes,
 * 8-byte aligned, and b_s: [ceil(N/128), K/128] fp32, 4-byte aligned
 * (written in full).  Ownership, statuses and asynchrony as for
 * fp8_block_gemm_quantize_rows; N may be any size >= 0.
 */
int fp8_block_gemm_quantize_blocks(const void *w, int64_t N, int64_t K, void *B, float *b_s, void *stream);

/* fp8_block_gemm_status_string -- static text for a status code. */
const char *fp8_block_gemm_status_string(int status);

/* fp8_block_gemm_version -- library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fp8_block_gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BG_H */
