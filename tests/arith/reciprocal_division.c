/*
 * The NVFP4 encoder's division: E2M1 code of fl32(x / e) (IEEE division)
 * against the code of copysign(fl32(q0 + r y), x) with y = fl32(1 / e),
 * q0 = fl32(x y), r = fma(-q0, e, x) (Markstein's correction of a division by
 * a correctly rounded reciprocal), for every finite bf16 x (zeros and
 * subnormals included) and divisors e = fl32(dec(b) t) in [2^-100, 2^100]
 * over all E4M3 codes b and `nt` pseudo-random tensor scales t, wherever the
 * quotient stays below 2^100 in magnitude.  Prints the number of cases and
 * of differing codes; exit status 1 on any difference.
 *
 * usage: reciprocal_division <nt> <seed>
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E4M3FN code -> value (exact) */
static float dec_e4m3(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    return e ? u2f(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
}

/* binary32 -> E2M1 code: nearest even, saturate at +-6, sign kept (the
 * values 0, .5, 1, 1.5, 2, 3, 4, 6 in codes 0..7, bit 3 the sign) */
static uint32_t enc_e2m1(float v)
{
    static const float val[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    const uint32_t sign = (f2u(v) >> 28) & 8u;
    const float a = fabsf(v);
    uint32_t best = 0;
    for (uint32_t c = 1; c < 8; ++c) {
        const float mid = 0.5f * (val[c - 1] + val[c]);   /* exact */
        if (a > mid || (a == mid && (c & 1u) == 0)) best = c;
    }
    return sign | best;
}

int main(int argc, char **argv)
{
    const int nt = argc > 1 ? atoi(argv[1]) : 8;
    srand(argc > 2 ? (unsigned)atoi(argv[2]) : 1u);
    long checked = 0, bad = 0;
    for (int ti = 0; ti < nt; ++ti) {
        /* half the scales with random bits over the whole exponent range, half near 1 */
        float t;
        if (ti % 2 == 0) {
            const uint32_t u = (((uint32_t)rand() << 8) ^ (uint32_t)rand()) & 0x007FFFFFu;
            t = u2f(u | ((uint32_t)(1 + rand() % 253) << 23));
        } else {
            t = ldexpf(1.0f + (float)(rand() % 1000) / 1000.0f, rand() % 200 - 100);
        }
        for (uint32_t b = 1; b < 127; ++b) {
            volatile float e = dec_e4m3(b) * t;
            if (!(e >= 0x1p-100f && e <= 0x1p100f)) continue;
            volatile float y = 1.0f / e;
            for (uint32_t h = 0; h < 65536; ++h) {
                const float x = u2f(h << 16);
                if (!isfinite(x)) continue;
                volatile float q = x / e;
                if (!(fabsf(q) <= 0x1p100f)) continue;
                volatile float q0 = x * y;
                const float r = fmaf(-q0, e, x);
                const float q1 = copysignf(fmaf(r, y, q0), x);
                ++checked;
                if (enc_e2m1(q) != enc_e2m1(q1)) {
                    if (bad < 10) printf("x=%a e=%a q=%a q1=%a\n", x, e, q, q1);
                    ++bad;
                }
            }
        }
    }
    printf("checked %ld differing %ld\n", checked, bad);
    return bad != 0;
}
