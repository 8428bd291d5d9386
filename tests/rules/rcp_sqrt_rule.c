/* Host models of the update kernel's square root and reciprocal (sqrt_rn and
 * rcp_rn in the kernel header).
 *
 * Square root: from
 * s = v_sqrt_f32(x) and t = v_rsq_f32(x), one correction
 * fma(fma(-s, s, x), t/2, s).  This host model (gcc, no contraction, libm
 * fmaf and sqrtf) runs the correction for every x of two binades ([1, 4):
 * both exponent parities, so every significand path of the square root)
 * with s and t taken as the correctly rounded sqrt(x) and 1/sqrt(x) or
 * either neighbour of each, and counts the results that differ from the
 * correctly rounded square root, per pair of offsets.
 *
 * Reciprocal: y + y*(1 - b*y) with both products in fmas, for every b in
 * [1, 2) (the rule scales exactly by powers of two in the normal range),
 * from y the correctly rounded 1/b or either neighbour.
 *
 * Output: one line per s offset (-1, 0, +1), three counts each (t offset
 * -1, 0, +1):  s<offset> <k> <k> <k>; then  rcp <k-1> <k0> <k+1>  (failures
 * per starting offset of y).
 * With correctly rounded inputs both rules are exact; from one-ulp inputs a
 * few x (b) are not, so the kernel's exactness is a property of the
 * hardware's own v_sqrt_f32, v_rsq_f32 and v_rcp_f32 outputs, which
 * tests/rules/rcp_sqrt_all.hip checks on the device for every input of the
 * ranges the kernel uses.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u_of(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }

int main(void) {
    long bad[3][3] = {{0}};
    for (uint32_t e = 127; e <= 128; ++e) {
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            const float x = f_of((e << 23) | m);
            const float want = sqrtf(x);                       /* correctly rounded */
            /* 1/sqrt(x) rounded once: the double quotient of a correctly
             * rounded double root is within 2^-52 relative, far below the
             * distance of 1/sqrt(x) from a float midpoint for these x */
            const float rs = (float)(1.0 / sqrt((double)x));
            for (int a = -1; a <= 1; ++a) {
                for (int b = -1; b <= 1; ++b) {
                    const float s = f_of(u_of(want) + (uint32_t)a);
                    const float t = f_of(u_of(rs) + (uint32_t)b);
                    const float got = fmaf(fmaf(-s, s, x), 0.5f * t, s);
                    bad[a + 1][b + 1] += u_of(got) != u_of(want);
                }
            }
        }
    }
    for (int a = 0; a < 3; ++a)
        printf("s%+d %ld %ld %ld\n", a - 1, bad[a][0], bad[a][1], bad[a][2]);
    long rbad[3] = {0, 0, 0};
    for (uint32_t m = 0; m < (1u << 23); ++m) {
        const float b = f_of(0x3f800000u | m);
        const float want = 1.0f / b;                         /* correctly rounded */
        for (int a = -1; a <= 1; ++a) {
            const float y = f_of(u_of(want) + (uint32_t)a);
            const float got = fmaf(fmaf(-b, y, 1.0f), y, y);
            rbad[a + 1] += u_of(got) != u_of(want);
        }
    }
    printf("rcp %ld %ld %ld\n", rbad[0], rbad[1], rbad[2]);
    return 0;
}
