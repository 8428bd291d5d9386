/* The update kernel divides by the per-tensor bias corrections bc1 and bc2
 * (wave-uniform divisors b in [2^-60, 1]) without a full division per
 * element: with y = 1/b correctly rounded, q = RN(x*y), r = fma(-q, b, x)
 * (exact), the quotient is RN(q + r*y) = fma(r, y, q), taken when
 * 2^-100 <= |x| < 2^64; other x take the division.  The 8-bit block scales
 * amax/127 and amax/255 use the same form for amax in [2^-100, FLT_MAX].
 * This program checks the rule against IEEE division on the host (gcc, no
 * contraction, libm fmaf).
 *
 * Output, one line each:
 *   checked <n> mismatches <k>          (in-range x: must be 0)
 *   outside <n> differ <k>              (x outside the range: the short form
 *                                        is wrong for some, so the range test
 *                                        is needed)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u_of(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }

static float short_div(float x, float b, float y) {
    float q = x * y;
    float r = fmaf(-q, b, x);
    return fmaf(r, y, q);
}

/* xorshift64*: the sample generator (no arithmetic of the method) */
static uint64_t s_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd32(void) {
    s_state ^= s_state >> 12; s_state ^= s_state << 25; s_state ^= s_state >> 27;
    return (uint32_t)((s_state * 0x2545F4914F6CDD1Dull) >> 32);
}

int main(void) {
    float bs[64];
    int nb = 0;
    const double betas[] = {0.9, 0.999, 0.95, 0.99};
    const int ts[] = {1, 2, 3, 10, 100, 1000, 100000};
    for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 7; j += 2 - (i & 1))
            bs[nb++] = (float)(1.0 - pow(betas[i], ts[j]));
    bs[nb++] = 1.0f;
    bs[nb++] = 0x1p-60f;
    bs[nb++] = nextafterf(1.0f, 0.0f);
    while (nb < 24) {              /* random significands, exponents -60..-1 */
        float b = ldexpf(f_of(0x3f800000u | (rnd32() & 0x7fffffu)), -1 - (int)(rnd32() % 60));
        bs[nb++] = b;
    }
    long checked = 0, bad = 0;
    for (int ib = 0; ib < nb; ++ib) {
        const float b = bs[ib], y = 1.0f / b;
        /* every significand of x in [1, 2), both signs */
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            const float x = f_of(0x3f800000u | m);
            bad += u_of(short_div(x, b, y)) != u_of(x / b);
            bad += u_of(short_div(-x, b, y)) != u_of(-x / b);
            checked += 2;
        }
        /* random significands at the ends of the range and in between */
        const int exps[] = {-100, -99, -80, -40, -1, 20, 50, 63};
        for (int e = 0; e < 8; ++e)
            for (int k = 0; k < 4096; ++k) {
                const float x = ldexpf(f_of(0x3f800000u | (rnd32() & 0x7fffffu)), exps[e]);
                bad += u_of(short_div(x, b, y)) != u_of(x / b);
                ++checked;
            }
    }
    /* the 8-bit block scales amax/127 and amax/255: constant divisors, x in
     * [2^-100, FLT_MAX] (every significand at exponent 0, samples at all
     * exponents up to the largest) */
    const float cs[2] = {127.0f, 255.0f};
    for (int ic = 0; ic < 2; ++ic) {
        const float b = cs[ic], y = 1.0f / b;
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            const float x = f_of(0x3f800000u | m);
            bad += u_of(short_div(x, b, y)) != u_of(x / b);
            ++checked;
        }
        for (int e = -100; e <= 127; ++e)
            for (int k = 0; k < 2048; ++k) {
                const float x = ldexpf(f_of(0x3f800000u | (rnd32() & 0x7fffffu)), e);
                bad += u_of(short_div(x, b, y)) != u_of(x / b);
                ++checked;
            }
        const float top = 0x1.fffffep127f;
        bad += u_of(short_div(top, b, y)) != u_of(top / b);
        ++checked;
    }
    printf("checked %ld mismatches %ld\n", checked, bad);
    /* outside the range: zeros, subnormals and tiny values, inf, NaN, huge */
    long outside = 0, differ = 0;
    for (int ib = 0; ib < nb; ++ib) {
        const float b = bs[ib], y = 1.0f / b;
        const float specials[] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 0x1p-149f, 0x1p-130f,
                                  0x1p-110f, 0x1p64f, 0x1.fffffep127f};
        for (int k = 0; k < 10; ++k) {
            const float x = specials[k];
            const float want = x / b, got = short_div(x, b, y);
            differ += !(u_of(got) == u_of(want) || (isnan(got) && isnan(want)));
            ++outside;
        }
        for (int k = 0; k < 4096; ++k) {    /* subnormal x */
            const float x = f_of(1u + (rnd32() & 0x7fffffu));
            differ += u_of(short_div(x, b, y)) != u_of(x / b);
            ++outside;
        }
    }
    printf("outside %ld differ %ld\n", outside, differ);
    return 0;
}
