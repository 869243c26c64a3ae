/*
 * Checks an identity the per-row quantizer kernel relies on (not part of the oracle):
 * with s a positive binary32 scale, y = RN(1/s) and, for every x,
 *     q0 = RN(x * y),  r = fma(-q0, s, x) (exact),  q1 = RN(r * y + q0),
 * q1 equals the correctly rounded quotient RN(x / s) (Markstein's theorem on
 * division by a correctly rounded reciprocal and an exact remainder), up to the sign
 * of a zero quotient. The kernel computes one IEEE division per row and three
 * operations per element instead of one division per element, so its codes
 * rint(x / s) equal the definition's.
 *
 * Domain checked: every finite binary16 x with |x| <= absmax, and random binary32
 * x with |x| <= absmax, for absmax log-uniform in [1e-10, 65504] (s = absmax / 127).
 * A second domain covers the re-quantization epilogue, whose scales come from the caller:
 * s any binary32 with exponent in [-100, 100] (random significands, plus all-ones and
 * one-ulp-above-a-power significands), x = s * u with |u| <= 128, and x next to each
 * tie (k + 1/2) s.
 * A third domain covers the block-asymmetric weight producer: a block's min and max drawn
 * with a log-uniform spread in [1e-9, 1e3] around a centre log-uniform in [1e-6, 1e3] of
 * either sign (so blocks of one sign, with quotients up to ~1e6, are included),
 * s = max((max - min) / 255, 1e-8), and x uniform in [min, max] plus min and max themselves.
 * Usage: quotient_identity <trials>. Exit status 0 iff no mismatch.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_f16(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    float v;
    if (e == 0)
        v = ldexpf((float)m, -24);
    else if (e == 31)
        return NAN;
    else
        v = ldexpf((float)(m | 1024), e - 25);
    return sign ? -v : v;
}

static uint64_t state = 88172645463325252ull;
static uint32_t next(void) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (uint32_t)state;
}

static int same(float a, float b) { return a == b; }   /* +0 == -0 */

int main(int argc, char** argv) {
    const int trials = argc > 1 ? atoi(argv[1]) : 200;
    long checked = 0, bad = 0;
    for (int t = 0; t < trials; ++t) {
        const double la = log(1e-10) + (log(65504.0) - log(1e-10)) * (next() / 4294967296.0);
        const float amax = (float)exp(la);
        volatile float s = fmaxf(amax, 1e-10f) / 127.0f;
        volatile float y = 1.0f / s;
        for (uint32_t h = 0; h < 65536 + 4096; ++h) {
            float x;
            if (h < 65536) {
                x = from_f16((uint16_t)h);
                if (isnan(x) || fabsf(x) > amax)
                    continue;
            } else {
                x = amax * ((float)(next() >> 8) / 16777216.0f) * ((next() & 1) ? 1.0f : -1.0f);
            }
            volatile float q = x / s;
            volatile float q0 = x * y;
            const float r = fmaf(-q0, s, x);
            const float q1 = fmaf(r, y, q0);
            ++checked;
            if (!same(q, q1)) {
                if (bad < 5)
                    printf("mismatch: absmax %a x %a x/s %a identity %a\n", amax, x, (float)q, q1);
                ++bad;
            }
        }
    }
    for (int t = 0; t < trials * 20; ++t) {
        uint32_t mant = next() & 0x7FFFFFu;
        if (t % 5 == 0)
            mant = 0x7FFFFFu;                 /* significand 1.111...1 */
        else if (t % 5 == 1)
            mant = 1;                         /* one ulp above a power of two */
        const int ex = (int)(next() % 201) - 100;
        uint32_t bits = ((uint32_t)(ex + 127) << 23) | mant;
        float sf;
        memcpy(&sf, &bits, 4);
        volatile float s = sf;
        volatile float y = 1.0f / s;
        for (int i = 0; i < 4096 + 256 * 3; ++i) {
            float x;
            if (i < 4096) {
                x = s * (128.0f * ((float)(next() >> 8) / 16777216.0f)) * ((next() & 1) ? 1.0f : -1.0f);
            } else {
                const int k = (i - 4096) / 3 - 128;
                const float tie = ((float)k + 0.5f) * s;
                const int d = (i - 4096) % 3;
                x = d == 0 ? tie : (d == 1 ? nextafterf(tie, INFINITY) : nextafterf(tie, -INFINITY));
            }
            volatile float q = x / s;
            volatile float q0 = x * y;
            const float r = fmaf(-q0, s, x);
            const float q1 = fmaf(r, y, q0);
            ++checked;
            if (!same(q, q1)) {
                if (bad < 5)
                    printf("mismatch: s %a x %a x/s %a identity %a\n", (float)s, x, (float)q, q1);
                ++bad;
            }
        }
    }
    for (int t = 0; t < trials * 20; ++t) {
        const double lc = log(1e-6) + (log(1e3) - log(1e-6)) * (next() / 4294967296.0);
        const double lw = log(1e-9) + (log(1e3) - log(1e-9)) * (next() / 4294967296.0);
        const float c = (float)exp(lc) * ((next() & 1) ? 1.0f : -1.0f);
        const float half = (float)exp(lw) * 0.5f;
        const float mn = c - half, mx = c + half;
        if (!(mx > mn))
            continue;
        volatile float s = fmaxf((mx - mn) / 255.0f, 1e-8f);
        volatile float y = 1.0f / s;
        for (int i = 0; i < 2048 + 2; ++i) {
            const float x = i == 2048 ? mn : i == 2049 ? mx
                                       : mn + (mx - mn) * ((float)(next() >> 8) / 16777216.0f);
            volatile float q = x / s;
            volatile float q0 = x * y;
            const float r = fmaf(-q0, s, x);
            const float q1 = fmaf(r, y, q0);
            ++checked;
            if (!same(q, q1)) {
                if (bad < 5)
                    printf("mismatch: block [%a, %a] s %a x %a x/s %a identity %a\n", mn, mx, (float)s, x, (float)q, q1);
                ++bad;
            }
        }
    }
    printf("checked %ld quotients, %ld mismatches\n", checked, bad);
    return bad != 0;
}
