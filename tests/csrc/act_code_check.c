/* CPU check of the division-free E2M1 code the vector product's in-launch
 * activation quantisation uses.  For a block scale s (an E4M3 value) and an
 * element a = |x| (a bf16 value):
 *   r = fp32(1 / s), q0 = a * r, e = fma(-q0, s, a), q = fma(e, r, q0)
 * (Markstein's corrected quotient), then the code is q rounded to the E2M1
 * grid {0, .5, 1, 1.5, 2, 3, 4, 6}, nearest, ties to the even code,
 * saturating at 6.  The reference is the code of the exact quotient a / s,
 * decided by exact comparisons of a with every midpoint times s (fp64, exact:
 * a has 8 significant bits, s 4, a midpoint 3).
 * Every positive bf16 a (subnormals included) is paired with every positive
 * E4M3 scale byte 0x01 .. 0x7E, for the pairs an activation block can hold
 * (a / s < 7: s = E4M3(amax / 6) >= amax / 6.5 and a <= amax), and beyond,
 * up to 2^16, for blocks whose scale saturates at 448.
 * Build with -ffp-contract=off.  Prints "bad <count> of <total>"; exit status
 * 1 on any mismatch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static double e4m3(unsigned b)
{
    unsigned e = (b >> 3) & 15, m = b & 7;
    return e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, (int)e - 7);
}

/* magnitude code of t on the E2M1 grid, nearest, ties to even, saturating:
 * the midpoints 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 between the codes; at a
 * tie the even code (0, 2, 4, 6 at 0.25, 1.25, 2.5, 5; codes 2, 4, 6 at 0.75,
 * 1.75, 3.5 from below) */
static unsigned code_of(double t)
{
    return (t > 0.25) + (t >= 0.75) + (t > 1.25) + (t >= 1.75) + (t > 2.5) + (t >= 3.5) + (t > 5.0);
}

int main(void)
{
    long bad = 0, total = 0;
    for (unsigned sb = 1; sb <= 0x7E; ++sb) {
        const float s = (float)e4m3(sb);
        const float r = 1.0f / s;
        for (uint32_t h = 1; h < 0x7F80; ++h) {           /* positive finite bf16 */
            const float a = fb(h << 16);
            if ((double)a >= 65536.0 * (double)s) continue;   /* saturated blocks too (scale clamped at 448) */
            ++total;
            /* exact: compare a with midpoint * s (both exact in fp64) */
            const double ad = a, sd = s;
            const unsigned ref = (ad > 0.25 * sd) + (ad >= 0.75 * sd) + (ad > 1.25 * sd) +
                                 (ad >= 1.75 * sd) + (ad > 2.5 * sd) + (ad >= 3.5 * sd) +
                                 (ad > 5.0 * sd);
            const float q0 = a * r;
            const float e = fmaf(-q0, s, a);
            const float q = fmaf(e, r, q0);
            if (code_of((double)q) != ref) {
                if (bad < 10)
                    printf("mismatch: a=%a s=%a q=%a code %u ref %u\n", a, s, q, code_of(q), ref);
                ++bad;
            }
        }
    }
    printf("bad %ld of %ld\n", bad, total);
    return bad ? 1 : 0;
}
