/*
 * Exhaustive check behind the activation quantiser's division (CPU only).
 *
 * The GPU kernel forms x / a_s, a_s = max(amax, 1e-12f)/448, not with one
 * IEEE division per element but with y = 1/a_s (one correctly rounded
 * division per group) and one correction step (Markstein's):
 *     q = RN(x*y),  r = fma(-q, a_s, x),  q' = copysign(fma(r, y, q), x).
 * For every finite bf16 group maximum amax >= 0 and every bf16 x with
 * |x| <= amax (both signs) this program compares the E4M3 code of
 * clamp(q', +-448) with the code of clamp(RN(x / a_s), +-448) -- the oracle's
 * definition -- using the oracle's encoder.  Exit status 0 iff no code
 * differs.  IEEE fp32 arithmetic (x86-64 SSE, fmaf) stands in for the
 * GPU's v_mul_f32 / v_fma_f32, which are IEEE operations too.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

unsigned fp8bg_oracle_e4m3_encode(double x);   /* oracle/fp8bg_oracle.c */

static float bf16(uint32_t h) { uint32_t u = h << 16; float f; memcpy(&f, &u, 4); return f; }
static uint32_t fbits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

int main(void)
{
    long long pairs = 0, float_diff = 0, code_diff = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, float_diff, code_diff)
    for (int ab = 0; ab <= 0x7F7F; ++ab) {
        const float amax = bf16((uint32_t)ab);
        const float s = fmaxf(amax, 1e-12f) / 448.0f;
        const float y = 1.0f / s;
        for (uint32_t xb = 0; xb <= 0x7F7F; ++xb) {
            const float xa = bf16(xb);
            if (xa > amax)
                break;                      /* bf16 magnitudes grow with the bit pattern */
            for (int sg = 0; sg < 2; ++sg) {
                const float x = sg ? -xa : xa;
                const float d = x / s;
                const float q = x * y;
                const float r = fmaf(-q, s, x);
                const float q2 = copysignf(fmaf(r, y, q), x);
                ++pairs;
                if (fbits(d) != fbits(q2)) {
                    ++float_diff;
                    if (fp8bg_oracle_e4m3_encode(clamp448(d)) != fp8bg_oracle_e4m3_encode(clamp448(q2)))
                        ++code_diff;
                }
            }
        }
    }
    printf("pairs %lld quotient_bit_differences %lld code_differences %lld\n", pairs, float_diff, code_diff);
    return code_diff != 0;
}
