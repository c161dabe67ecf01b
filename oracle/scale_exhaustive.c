/* Exhaustive check of the INT4 scale definition (test infrastructure only).
 *
 * The INT4 scale is defined in two rounding steps, s = fp16_rne(fp32_rne(d/15)),
 * because that is what a GPU computes with a correctly rounded fp32 divide
 * followed by an fp16 convert. This program proves, for every positive finite
 * fp32 range d, that the two-step value equals the single correctly rounded
 * fp16 value of the exact rational d/15, computed here with integer
 * arithmetic only (no floating-point division involved in the reference).
 *
 * Modes:
 *   scale_exhaustive all            -> prints "checked N mismatches M"
 *   scale_exhaustive exact < hexlist -> for each fp32 bit pattern (hex) on stdin,
 *                                       prints the exact fp16_rne(d/15) bits (hex)
 * Build: gcc -O2 -fopenmp scale_exhaustive.c -o scale_exhaustive
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

/* fp32 bits -> fp16 bits, round to nearest, ties to even (integer only). */
static uint16_t f32_to_f16_rne(uint32_t x) {
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ex = (x >> 23) & 0xFFu, man = x & 0x7FFFFFu;
    if (ex == 0xFFu) return (uint16_t)(sign | 0x7C00u | (man ? 0x200u : 0u));
    int e = (int)ex - 127;
    uint32_t m = ex ? (man | 0x800000u) : man;
    if (!ex) e = -126;
    if (e > 15) return (uint16_t)(sign | 0x7C00u);
    if (e >= -14) {
        uint32_t f = m >> 13, rem = m & 0x1FFFu;
        if (rem > 0x1000u || (rem == 0x1000u && (f & 1u))) f++;
        return (uint16_t)(sign | ((((uint32_t)(e + 15)) << 10) + (f - 1024u)));
    }
    int shift = -(e + 1);                 /* value / 2^-24 = m * 2^(e+1) */
    if (shift > 25) return (uint16_t)sign;
    uint32_t f = m >> shift, rem = m & ((1u << shift) - 1u), half = 1u << (shift - 1);
    if (rem > half || (rem == half && (f & 1u))) f++;
    return (uint16_t)(sign | f);
}

static int bitlen(uint64_t v) { int n = 0; while (v) { n++; v >>= 1; } return n; }

/* fp16_rne of the exact rational M * 2^E / 15 (M > 0). Integer arithmetic only. */
static uint16_t exact_div15_to_f16(uint32_t M, int E) {
    int bl = bitlen(M);
    /* X = M 2^E / 15 lies in [2^(bl-1+E-4), 2^(bl+E-4+1)); pick floor(log2 X). */
    int e = bl - 1 + E - 4;
    if (bl >= 4) {
        if ((uint64_t)M >= ((uint64_t)15u << (bl - 4))) e += 1;
    } else {
        if (((uint64_t)M << (4 - bl)) >= 15u) e += 1;
    }
    /* overflow: X >= 65520 rounds to infinity */
    if (e >= 16) return 0x7C00u;
    if (e < -14) e = -14;
    int sh = E - e + 10;                  /* f = X / 2^(e-10) = M 2^sh / 15 */
    uint64_t f;
    if (sh >= 0) {
        unsigned __int128 num = (unsigned __int128)M << sh;
        f = (uint64_t)(num / 15u);
        unsigned rem = (unsigned)(num % 15u);
        if (2u * rem > 15u) f++;          /* 15 is odd: no exact ties */
    } else {
        if (-sh > 100) return 0;          /* far below half a quantum */
        unsigned __int128 den = (unsigned __int128)15u << (-sh);
        f = (uint64_t)(M / den);
        unsigned __int128 rem = M % den;
        unsigned __int128 twice = rem * 2u;
        if (twice > den || (twice == den && (f & 1u))) f++;
    }
    if (e == -14 && f < 1024u) return (uint16_t)f;               /* subnormal (or min normal by carry) */
    uint64_t bits = (((uint64_t)(e + 15)) << 10) + (f - 1024u);  /* carry into exponent is fine */
    if (bits >= 0x7C00u) return 0x7C00u;
    return (uint16_t)bits;
}

static uint16_t exact_for_bits(uint32_t d) {
    uint32_t ex = (d >> 23) & 0xFFu, man = d & 0x7FFFFFu;
    if (ex == 0 && man == 0) return 0;
    uint32_t M = ex ? (man | 0x800000u) : man;
    int E = ex ? (int)ex - 150 : -149;
    return exact_div15_to_f16(M, E);
}

static uint16_t twostep_for_bits(uint32_t d) {
    float f;
    memcpy(&f, &d, 4);
    volatile float q = f / 15.0f;        /* correctly rounded IEEE fp32 division */
    float qq = q;
    uint32_t qb;
    memcpy(&qb, &qq, 4);
    return f32_to_f16_rne(qb);
}

int main(int argc, char** argv) {
    if (argc > 1 && strcmp(argv[1], "exact") == 0) {
        unsigned v;
        while (scanf("%x", &v) == 1) printf("%04x\n", exact_for_bits(v));
        return 0;
    }
    if (argc > 1 && strcmp(argv[1], "twostep") == 0) {
        unsigned v;
        while (scanf("%x", &v) == 1) printf("%04x\n", twostep_for_bits(v));
        return 0;
    }
    long long mismatches = 0, checked = 0;
#pragma omp parallel for reduction(+ : mismatches, checked) schedule(static)
    for (long long i = 1; i < 0x7F800000LL; i++) {
        uint32_t d = (uint32_t)i;
        if (exact_for_bits(d) != twostep_for_bits(d)) mismatches++;
        checked++;
    }
    printf("checked %lld mismatches %lld\n", checked, mismatches);
    return mismatches != 0;
}
