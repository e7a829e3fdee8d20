/*
 * fp8bg_oracle.c -- plain CPU reference for the W8A8 block-scaled FP8 matmul.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only code that may load this library.
 * The GPU product path never links, loads or calls it, and this file shares
 * no code, header, table or constant with the HIP kernels.
 *
 * What it computes (FlagGems-vllm PR #693, "feat: optimize w8a8 block fp8
 * matmul for Hopper", section "Description": FP8 E4M3 inputs with per-token
 * activation scales and [block_n, block_k] weight de-quant scales; section
 * "Numerical safety": FP32 accumulation, then a cast to bf16 / fp16 / fp32):
 *
 *     C[m,n] = sum_g  a_s[m,g] * b_s[n/128, g] * sum_{k in group g} A[m,k]*B[n,k]
 *
 * with groups of 128 consecutive k.  A is [M,K] row-major, B is [N,K]
 * row-major (the weight of y = x W^T), a_s is [M, G] and b_s is
 * [ceil(N/128), G], G = ceil(K/128), all row-major fp32.
 *
 * Evaluation is the plain definition in fp64, written out loop by loop:
 *   - each E4M3 code is decoded exactly from its bit fields;
 *   - the 128-term group sum of products is exact in fp64 (a product of two
 *     E4M3 values has at most 8 significant bits and lies in [2^-18, 2^18),
 *     so 128 of them sum to a multiple of 2^-18 below 2^25: < 53 bits);
 *   - s = a_s * b_s is exact in fp64 (24 + 24 significant bits);
 *   - the only roundings are the G products p*s and G additions into acc.
 * The result is therefore the exact value up to a relative error of about
 * (2G+1) * 2^-53 of the sum of |terms|, far below any output-dtype ulp.
 *
 * The cast to the output dtype is one IEEE round-to-nearest-even step from
 * the fp64 value (the pages only say "casts"; RNE is the reading taken).
 *
 * It also computes the producers of the operands: the per-token 1 x 128
 * activation quantisation (fp8bg_oracle_quantize_rows) and the 128 x 128
 * weight-block quantisation (fp8bg_oracle_quantize_blocks), with the E4M3
 * encoder fp8bg_oracle_e4m3_encode written from the format definition.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <fenv.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 128

/* ------------------------------------------------------------------------ */
/* OCP FP8 E4M3 ("E4M3FN": no infinities, exponent bias 7, NaN only at       */
/* S.1111.111, largest finite value 448).                                    */
/* ------------------------------------------------------------------------ */
double fp8bg_oracle_e4m3_value(unsigned code)
{
    unsigned s = (code >> 7) & 1u;
    unsigned e = (code >> 3) & 15u;
    unsigned m = code & 7u;
    double mag;
    if (e == 15u && m == 7u)
        return NAN;
    if (e == 0u)
        mag = ldexp((double)m, -9);                 /* subnormal: m/8 * 2^(1-7) */
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* ------------------------------------------------------------------------ */
/* The block-scaled GEMM, fp64.                                              */
/* ------------------------------------------------------------------------ */
void fp8bg_oracle_gemm(const uint8_t *A, const float *a_s,
                       const uint8_t *B, const float *b_s,
                       int64_t M, int64_t N, int64_t K, double *C)
{
    double dec[256];
    for (unsigned c = 0; c < 256u; ++c)
        dec[c] = fp8bg_oracle_e4m3_value(c);

    const int64_t G = (K + ORACLE_GROUP - 1) / ORACLE_GROUP;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                const int64_t k0 = g * ORACLE_GROUP;
                const int64_t k1 = (k0 + ORACLE_GROUP < K) ? k0 + ORACLE_GROUP : K;
                double p = 0.0;                          /* exact group sum */
                for (int64_t k = k0; k < k1; ++k)
                    p += dec[A[m * K + k]] * dec[B[n * K + k]];
                double s = (double)a_s[m * G + g] * (double)b_s[(n / ORACLE_GROUP) * G + g];
                acc += p * s;
            }
            C[m * N + n] = acc;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* One-step fp64 -> {bf16, fp16, fp32} round-to-nearest-even.                */
/* ------------------------------------------------------------------------ */
enum { ORACLE_BF16 = 0, ORACLE_FP16 = 1, ORACLE_FP32 = 2 };

/* Round x to a binary format with p significand bits (hidden bit included)
 * and normal exponent range [emin, emax].  Returns the rounded value, or a
 * signed infinity when RNE overflows. */
static double round_to_format(double x, int p, int emin, int emax)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    int e;
    (void)frexp(fabs(x), &e);          /* |x| = f * 2^e, f in [0.5, 1) */
    int E = e - 1;                     /* floor(log2 |x|) */
    if (E < emin)
        E = emin;                      /* subnormal range: fixed quantum */
    double q = ldexp(1.0, E - p + 1);  /* spacing of the format at |x| */
    double r = nearbyint(x / q) * q;   /* x/q is exact; nearbyint ties to even */
    double maxv = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (fabs(r) > maxv)
        return copysign(INFINITY, x);
    return r;
}

static uint16_t encode_fp16(double r)
{
    uint16_t s = signbit(r) ? 0x8000u : 0u;
    double a = fabs(r);
    if (isnan(r))
        return 0x7E00u;
    if (isinf(a))
        return (uint16_t)(s | 0x7C00u);
    if (a == 0.0)
        return s;
    int e;
    (void)frexp(a, &e);
    int E = e - 1;
    if (E < -14)                                    /* subnormal: a = m * 2^-24 */
        return (uint16_t)(s | (uint16_t)(a / ldexp(1.0, -24)));
    unsigned mant = (unsigned)((a / ldexp(1.0, E) - 1.0) * 1024.0);
    return (uint16_t)(s | ((unsigned)(E + 15) << 10) | mant);
}

static uint32_t float_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* Rounds n fp64 values to out_dtype and writes their bit patterns to out
 * (uint16 for bf16 / fp16, uint32 for fp32).  Returns 0, or -1 for an
 * unknown dtype. */
int fp8bg_oracle_round(const double *x, int64_t n, int out_dtype, void *out)
{
    if (out_dtype != ORACLE_BF16 && out_dtype != ORACLE_FP16 && out_dtype != ORACLE_FP32)
        return -1;
    fesetround(FE_TONEAREST);
    for (int64_t i = 0; i < n; ++i) {
        double v = x[i];
        if (out_dtype == ORACLE_BF16) {
            uint16_t bits;
            if (isnan(v)) {
                bits = 0x7FC0u;
            } else {
                double r = round_to_format(v, 8, -126, 127);
                bits = (uint16_t)(float_bits((float)r) >> 16);   /* r is exact in fp32 */
            }
            ((uint16_t *)out)[i] = bits;
        } else if (out_dtype == ORACLE_FP16) {
            ((uint16_t *)out)[i] = encode_fp16(isnan(v) ? v : round_to_format(v, 11, -14, 15));
        } else {
            uint32_t bits = isnan(v) ? 0x7FC00000u
                                     : float_bits((float)round_to_format(v, 24, -126, 127));
            ((uint32_t *)out)[i] = bits;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token activation quantisation to E4M3 with one fp32 scale per row    */
/* and 128-wide group: the producer of A and a_s (the pages' per-token      */
/* 1 x 128 activation scales, FlagGems-vllm PR #693, section "Description").*/
/*                                                                          */
/*     amax   = max_{k in group} |x[m,k]|             (x: bf16 values)       */
/*     a_s    = max(amax, 1e-12f) / 448               (fp32 division, RNE)   */
/*     A[m,k] = E4M3_RNE(clamp(x[m,k] / a_s, -448, 448))   (fp32 division)  */
/*                                                                          */
/* 448 is E4M3's largest finite value, so the group's largest element maps  */
/* to (about) +-448; the 1e-12 floor keeps an all-zero group finite; the    */
/* clamp absorbs a quotient rounded just above 448.                         */
/* ------------------------------------------------------------------------ */

/* E4M3 code of a finite double with |x| <= 448, rounding to the nearest   */
/* representable value, ties to the even code.  Written from the format:   */
/* below 2^-6 the values are the multiples of 2^-9 (codes 0..8 carry on    */
/* into the first binade); in the binade [2^e, 2^(e+1)) they are the       */
/* multiples of 2^(e-3).                                                   */
unsigned fp8bg_oracle_e4m3_encode(double x)
{
    const unsigned sign = signbit(x) ? 0x80u : 0u;
    double a = fabs(x);
    unsigned code;
    if (a >= 448.0)
        return sign | 0x7Eu;
    if (a < ldexp(1.0, -6)) {
        const double q = nearbyint(ldexp(a, 9));        /* units of 2^-9, 0..8 */
        code = (unsigned)q;                              /* 8 is 2^-6 = e=1, m=0 */
    } else {
        int e2;
        frexp(a, &e2);                                   /* a in [2^(e2-1), 2^e2) */
        const int e = e2 - 1;                            /* unbiased exponent      */
        double q = nearbyint(ldexp(a, 3 - e));           /* units of 2^(e-3): 8..16 */
        int eb = e + 7;
        if (q >= 16.0) {                                 /* rounded up to 2^(e+1) */
            q = 8.0;
            eb += 1;
        }
        code = ((unsigned)eb << 3) | ((unsigned)q - 8u);
    }
    return sign | code;
}

static float bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* x: [M,K] bf16 bit patterns, row-major; q: [M,K] codes; a_s: [M, ceil(K/128)]. */
void fp8bg_oracle_quantize_rows(const uint16_t *x, int64_t M, int64_t K,
                                uint8_t *q, float *a_s)
{
    const int64_t G = (K + ORACLE_GROUP - 1) / ORACLE_GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t k0 = g * ORACLE_GROUP;
            const int64_t k1 = k0 + ORACLE_GROUP < K ? k0 + ORACLE_GROUP : K;
            float amax = 0.0f;
            for (int64_t i = k0; i < k1; ++i) {
                const float v = fabsf(bf16_value(x[m * K + i]));
                if (v > amax)
                    amax = v;
            }
            const float s = (amax > 1e-12f ? amax : 1e-12f) / 448.0f;
            a_s[m * G + g] = s;
            for (int64_t i = k0; i < k1; ++i) {
                float v = bf16_value(x[m * K + i]) / s;
                if (v > 448.0f) v = 448.0f;
                if (v < -448.0f) v = -448.0f;
                q[m * K + i] = (uint8_t)fp8bg_oracle_e4m3_encode((double)v);
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Weight quantisation to E4M3 with one fp32 scale per 128 x 128 block: the */
/* producer of B and b_s (the pages' [block_n, block_k] = [128, 128] weight */
/* de-quant scales, FlagGems-vllm PR #693, section "Description").          */
/*                                                                          */
/*     amax    = max over the block's rows n and columns k of |w[n,k]|      */
/*     b_s     = max(amax, 1e-12f) / 448                 (fp32 division)    */
/*     B[n,k]  = E4M3_RNE(clamp(w[n,k] / b_s, -448, 448))  (fp32 division)  */
/*                                                                          */
/* The last block row holds the N % 128 remaining rows when N is not a      */
/* multiple of 128 (b_s has ceil(N/128) rows).                               */
/* ------------------------------------------------------------------------ */

/* w: [N,K] bf16 bit patterns, row-major; q: [N,K] codes; b_s: [ceil(N/128), ceil(K/128)]. */
void fp8bg_oracle_quantize_blocks(const uint16_t *w, int64_t N, int64_t K,
                                  uint8_t *q, float *b_s)
{
    const int64_t NB = (N + ORACLE_GROUP - 1) / ORACLE_GROUP;
    const int64_t G = (K + ORACLE_GROUP - 1) / ORACLE_GROUP;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bn = 0; bn < NB; ++bn) {
        for (int64_t g = 0; g < G; ++g) {
            const int64_t n0 = bn * ORACLE_GROUP, n1 = n0 + ORACLE_GROUP < N ? n0 + ORACLE_GROUP : N;
            const int64_t c0 = g * ORACLE_GROUP, c1 = c0 + ORACLE_GROUP < K ? c0 + ORACLE_GROUP : K;
            float amax = 0.0f;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t c = c0; c < c1; ++c) {
                    const float v = fabsf(bf16_value(w[n * K + c]));
                    if (v > amax)
                        amax = v;
                }
            const float s = (amax > 1e-12f ? amax : 1e-12f) / 448.0f;
            b_s[bn * G + g] = s;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t c = c0; c < c1; ++c) {
                    float v = bf16_value(w[n * K + c]) / s;
                    if (v > 448.0f) v = 448.0f;
                    if (v < -448.0f) v = -448.0f;
                    q[n * K + c] = (uint8_t)fp8bg_oracle_e4m3_encode((double)v);
                }
        }
    }
}

/* Number of threads the oracle's OpenMP loops use. */
int fp8bg_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of the OpenMP loops (timing of the oracle on one
 * core and on all of them); no effect on any result. */
void fp8bg_oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
