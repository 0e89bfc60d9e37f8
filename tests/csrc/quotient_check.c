/* CPU check of the division-free quotient the weight quantiser's fast path
 * uses: q0 = n * rb, r = fma(-b, q0, n), q = fma(r, rb, q0) with rb = fp32(1/b)
 * (Markstein's corrected quotient).  Every case compares q with the correctly
 * rounded n / b, bit for bit, where the code decision depends on it:
 *   six   n / 6 for every float n >= 2^-124 (stride S over the bit patterns)
 *   e4m3  t / g for t within 6 units in the last place of m * g, m every
 *         mantissa pattern of an E4M3 rounding midpoint, g every S-th 24-bit
 *         significand at the exponents given
 *   e2m1  |w| / d for |w| within 6 units of m * d, m every E2M1 midpoint
 * Build with -ffp-contract=off.  Usage: quotient_check STRIDE EXP...
 * Prints "bad <count> of <total>" per part; exit status 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float markstein(float n, float b, float rb)
{
    float q0 = n * rb;
    float r = fmaf(-b, q0, n);
    return fmaf(r, rb, q0);
}

static long near_mids(const float *mids, int nm, int bexp, uint32_t stride, long *total)
{
    long bad = 0;
    for (uint32_t mant = 0; mant < (1u << 23); mant += stride) {
        float b = fb(((uint32_t)(bexp + 127) << 23) | mant), rb = 1.0f / b;
        for (int k = 0; k < nm; ++k) {
            uint32_t c = bf(mids[k] * b);
            for (int o = -6; o <= 6; ++o) {
                float n = fb(c + (uint32_t)o);
                if (isinf(n) || isnan(n)) continue;
                ++*total;
                if (bf(markstein(n, b, rb)) != bf(n / b)) ++bad;
            }
        }
    }
    return bad;
}

int main(int argc, char **argv)
{
    uint32_t stride = argc > 1 ? (uint32_t)strtoul(argv[1], 0, 10) : 1;
    int fail = 0;
    long bad = 0, total = 0;
    const float rb6 = 1.0f / 6.0f;
    for (uint32_t u = 0x01800000u; u < 0x7F800000u; u += stride) {   /* n >= 2^-124 */
        float n = fb(u);
        ++total;
        if (bf(markstein(n, 6.0f, rb6)) != bf(n / 6.0f)) ++bad;
    }
    printf("six bad %ld of %ld\n", bad, total);
    fail |= bad != 0;

    float e4[48], e2[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    int ne4 = 0;
    for (int p = 0; p < 16; ++p)            /* midpoint significands: <= 4 fraction bits */
        for (int e = -10; e <= 8; e += 9) e4[ne4++] = ldexpf(1.0f + (float)p / 16.0f, e);
    for (int a = 2; a < argc; ++a) {
        int ex = atoi(argv[a]);
        bad = total = 0;
        bad = near_mids(e4, ne4, ex, stride, &total);
        printf("e4m3 exp %d bad %ld of %ld\n", ex, bad, total);
        fail |= bad != 0;
        bad = total = 0;
        bad = near_mids(e2, 7, ex, stride, &total);
        printf("e2m1 exp %d bad %ld of %ld\n", ex, bad, total);
        fail |= bad != 0;
    }
    return fail;
}
