/* CPU check of the quotient scheme the INT4 and INT8 quantizers use instead
 * of an IEEE fp32 divide per element: y = RN(1/s), q0 = x*y, then two FMA
 * residual steps q' = q + (x - q*s)*y (Markstein's theorem: once q is
 * faithful and y is within half an ulp of 1/s, the step returns RN(x/s)).
 * The codes from the scheme are compared with those from x/s:
 *   INT4: every positive finite fp16 scale, quotients within six ulps of each
 *         half-integer 0.5 .. 15.5, plus random diffs; code = clamp(rint, 0, 15).
 *   INT8: random 16-bit block maxima, s = max/127, quotients within three ulps
 *         of each half-integer -126.5 .. 126.5; scales outside [2^-100, 2^100)
 *         divide; code = clamp(rint, -127, 127).
 * Prints the number of mismatching codes per part; exit status 1 if any. */
#include <math.h>
#include <stdlib.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint64_t rs = 88172645463325252ull;
static uint64_t rnd(void) { rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17; return rs; }
static float from_f16(uint16_t h) { _Float16 v; memcpy(&v, &h, 2); return (float)v; }
static float from_bf16(uint16_t b) { uint32_t u = (uint32_t)b << 16; float f; memcpy(&f, &u, 4); return f; }
static float scheme(float x, float s, float y) {
    const float q0 = x * y;
    const float q1 = fmaf(fmaf(-q0, s, x), y, q0);
    return fmaf(fmaf(-q1, s, x), y, q1);
}
static float step(float v, int n) {
    for (int j = 0; j < (n < 0 ? -n : n); ++j) v = nextafterf(v, n > 0 ? INFINITY : -INFINITY);
    return v;
}
static unsigned int4_ref(float d, float s) { return s > 0.f ? (unsigned)fminf(fmaxf(rintf(d / s), 0.f), 15.f) : 0u; }
static unsigned int4_new(float d, float s) {
    const float y = 1.0f / s, q0 = d * y;
    const float q = isfinite(q0) ? scheme(d, s, y) : q0;
    return s > 0.f ? (unsigned)fminf(fmaxf(rintf(q), 0.f), 15.f) : 0u;
}
static float int8_ref(float x, float s) { return s > 0.f ? fminf(fmaxf(rintf(x / s), -127.f), 127.f) : 0.f; }
static float int8_new(float x, float s) {
    const float q = (s >= 0x1p-100f && s < 0x1p100f) ? scheme(x, s, 1.0f / s) : x / s;
    return s > 0.f ? fminf(fmaxf(rintf(q), -127.f), 127.f) : 0.f;
}
int main(int argc, char** argv) {
    long maxima = argc > 1 ? atol(argv[1]) : 200000;
    long n4 = 0, bad4 = 0, n8 = 0, bad8 = 0;
    for (uint32_t hs = 1; hs < 0x7C00; ++hs) {
        const float s = from_f16((uint16_t)hs);
        for (int k = 0; k < 16; ++k)
            for (int d = -6; d <= 6; ++d) {
                const float x = step((k + 0.5f) * s, d);
                ++n4; bad4 += int4_ref(x, s) != int4_new(x, s);
            }
        for (int r = 0; r < 16; ++r) {
            const float x = (float)((double)(rnd() % 2000000) / 100000.0 - 2.0) * s;
            ++n4; bad4 += int4_ref(x, s) != int4_new(x, s);
        }
    }
    const float specials[] = {0.f, -0.f, INFINITY, -INFINITY, NAN, 1e30f, -1e30f, 65504.f, 1e-30f, -1e-40f};
    const float sspec[] = {0.f, INFINITY, NAN, from_f16(1), from_f16(0x3C00), from_f16(0x7BFF)};
    for (int i = 0; i < 10; ++i)
        for (int j = 0; j < 6; ++j) { ++n4; bad4 += int4_ref(specials[i], sspec[j]) != int4_new(specials[i], sspec[j]); }
    for (long it = 0; it < maxima; ++it) {
        float amax;
        if (it & 1) { do amax = from_f16((uint16_t)(rnd() % 0x7C00) + 1); while (!(amax > 0.f)); }
        else { do amax = from_bf16((uint16_t)(rnd() & 0x7FFF)); while (!isfinite(amax) || amax == 0.f); }
        if (it % 1000 == 0) amax = INFINITY;
        const float s = amax / 127.0f;
        for (int k = -127; k <= 127; k += (int)(it % 7) + 1)
            for (int d = -3; d <= 3; ++d) {
                const float x = step((k + 0.5f) * s, d);
                if (!(fabsf(x) <= amax)) continue;
                ++n8; bad8 += int8_ref(x, s) != int8_new(x, s);
            }
    }
    printf("int4: %ld codes, %ld mismatches\nint8: %ld codes, %ld mismatches\n", n4, bad4, n8, bad8);
    return (bad4 || bad8) ? 1 : 0;
}
