/* Exhaustive host check of the short division the update kernel uses for the
 * per-tensor bias corrections and the 8-bit block scales: for a divisor b and
 * y = 1/b correctly rounded, q = RN(x*y), r = fma(-q, b, x) (exact), and the
 * quotient taken as fma(r, y, q) -- Markstein's correction step.
 *
 * Every pair of fp32 significands is tried: b = 1 + i*2^-23 for i in
 * [b_first, b_last), x = 1 + j*2^-23 for every j in [0, 2^23), and the result
 * is compared bit for bit with IEEE division x/b.  The quotient of two such
 * significands spans both of its possible binades, and scaling x and b by
 * powers of two scales every step exactly while nothing leaves the normal
 * range (the kernel takes the short form only for 2^-100 <= |x| < 2^64 and
 * b in [2^-60, 1]), and negation is exact, so a clean run over all 2^23
 * divisors covers every operand the kernel hands to it.
 *
 * Build: gcc -O3 -march=native -ffp-contract=off -fopenmp (every operation
 * separately rounded; the two fmaf calls are the only fused ones).
 * Usage:  div_exhaustive [b_first [b_last]]   (default: all 2^23 divisors)
 * Output: divisors <n> pairs <n> mismatches <k>
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define SIG (1u << 23)

static inline float f_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static inline uint32_t u_of(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }

int main(int argc, char **argv) {
    const long first = argc > 1 ? atol(argv[1]) : 0;
    const long last = argc > 2 ? atol(argv[2]) : (long)SIG;
    if (first < 0 || last > (long)SIG || first > last) {
        fprintf(stderr, "divisor range must lie in [0, %u]\n", SIG);
        return 2;
    }
    long bad = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad)
    for (long i = first; i < last; ++i) {
        const float b = f_of(0x3f800000u | (uint32_t)i);
        const float y = 1.0f / b;
        long local = 0;
        for (uint32_t j = 0; j < SIG; ++j) {
            const float x = f_of(0x3f800000u | j);
            const float q = x * y;
            const float r = fmaf(-q, b, x);
            const float s = fmaf(r, y, q);
            local += u_of(s) != u_of(x / b);
        }
        bad += local;
    }
    printf("divisors %ld pairs %ld mismatches %ld\n", last - first,
           (last - first) * (long)SIG, bad);
    return bad != 0;
}
