/* Checks the reciprocal-based quotient of the FP8 quantizer kernels against
 * the correctly rounded fp32 division, over bf16 inputs:
 *   s = amax / 448 (amax a positive finite bf16 value, s in [2^-64, 2^64]),
 *   y = 1 / s, q0 = x * y, r = fma(q0, s, -x), q = fma(-r, y, q0)
 * for every bf16 x with |x| <= amax.  A pair passes if q equals x / s bit for
 * bit, or if both are below 2^-10 in magnitude with the sign of x (then both
 * encode to the same signed e4m3 zero).  The residual is formed as q0 s - x
 * and subtracted (r' = -r exactly, rounding being symmetric), so that a
 * zero x keeps its sign through both fmas (-0 * y + -0 = -0) and no
 * copysign is needed; the program also checks that q equals the
 * copysign(fma(fma(-q0, s, x), y, q0), x) form bit for bit.
 * usage: quot_check <amax stride> ; prints "pairs <n> exact <e> bad <b>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bf16(uint32_t h)
{
    uint32_t u = h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

int main(int argc, char** argv)
{
    const int stride = argc > 1 ? atoi(argv[1]) : 1;
    long pairs = 0, exact = 0, bad = 0;
    for (uint32_t ha = 1; ha < 0x7F80; ha += (uint32_t)stride) {
        const float amax = bf16(ha);
        volatile float s = amax / 448.0f;
        if (!(s >= 0x1p-64f && s <= 0x1p64f))
            continue;
        volatile float y = 1.0f / s;
        for (uint32_t hx = 0; hx <= ha; ++hx)
            for (int neg = 0; neg < 2; ++neg) {
                const float x = bf16(hx | (neg ? 0x8000u : 0u));
                const float want = x / s;
                const float q0 = x * y;
                const float r = fmaf(q0, s, -x);
                const float got = fmaf(-r, y, q0);
                const float old = copysignf(fmaf(fmaf(-q0, s, x), y, q0), x);
                ++pairs;
                if (bits(got) != bits(old)) {
                    if (++bad <= 5)
                        printf("forms differ amax=%a x=%a %a %a\n", amax, x, got, old);
                    continue;
                }
                if (bits(got) == bits(want)) {
                    ++exact;
                    continue;
                }
                if (fabsf(want) < 0x1p-10f && fabsf(got) < 0x1p-10f &&
                    signbit(want) == signbit(got))
                    continue;
                if (++bad <= 5)
                    printf("mismatch amax=%a x=%a want=%a got=%a\n", amax, x, want, got);
            }
    }
    printf("pairs %ld exact %ld bad %ld\n", pairs, exact, bad);
    return bad != 0;
}
