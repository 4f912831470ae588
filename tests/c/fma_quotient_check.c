/*
 * Exhaustive check of the division-free code rounding of the fused decode
 * kernel, for every fp16 value x and every per-token scale s = fl32(a / 127)
 * of a positive finite fp16 a >= |x|, with r = fl32(1 / s):
 *  1. the fast code t = fma(x, r, 128) rounds to rint(fl32(x / s)) + 128
 *     unless |t - rint(t)| > 0.5 - 2^-16 (the kernel's near-tie test);
 *  2. q0 = fl32(x r), e = fma(-q0, s, x), q = fma(e, r, q0) equals the
 *     correctly rounded quotient fl32(x / s) (Markstein's correction step),
 *     which the kernel uses for the chunks the test flags.
 * Prints the number of pairs, fast-path misses the test would not flag, and
 * quotient mismatches; exits 1 if either count is not zero.
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math [-fopenmp] -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

static float fp16_value(uint16_t h)
{
    int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    double v = e == 0 ? ldexp((double)m, -24) : ldexp((double)(m | 1024), e - 25);
    return (float)(sign ? -v : v);
}

int main(void)
{
    long long pairs = 0, bad = 0, unflagged = 0, flagged = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad, unflagged, flagged)
    for (int ah = 1; ah < 0x7c00; ++ah) {
        const float a = fp16_value((uint16_t)ah);
        const float s = a / 127.0f;
        const float r = 1.0f / s;
        for (int xh = 0; xh <= ah; ++xh) {
            for (int sg = 0; sg < 2; ++sg) {
                const float x = fp16_value((uint16_t)(xh | (sg << 15)));
                const float q0 = x * r;
                const float e = fmaf(-q0, s, x);
                const float q = fmaf(e, r, q0);
                const float exact = x / s;
                ++pairs;
                if (q != exact)
                    ++bad;
                const float t = fmaf(x, r, 128.0f);
                const float n = rintf(t);
                const int flag = fabsf(t - n) > 0.5f - 0x1p-16f;
                flagged += flag;
                if (!flag && n != rintf(exact) + 128.0f)
                    ++unflagged;
            }
        }
    }
    printf("pairs %lld flagged %lld unflagged-misses %lld mismatches %lld\n", pairs, flagged, unflagged, bad);
    return bad != 0 || unflagged != 0;
}
