// Asymmetric INT4 quantization of one 32-channel group (device code).
//
// Format (HyQuant pages: "How HyQuant uses hybrid-precision attention to cut
// decode compute", "What the authors tested": non-retained K and V are held
// as Key-4bit / Value-4bit; the group size, scale and zero types and the
// rounding are this library's reading):
//   mn, mx over the group; d = mx - mn (exact in fp32 for 16-bit inputs);
//   s = fp16_rne(fp32 d / 15)   (IEEE correctly rounded fp32 divide);
//   z = fp16_rne(mn);
//   code = clamp(rint_even(fp32(x - z) / s), 0, 15), or 0 when s == 0
//   (the quotient correctly rounded, as an IEEE fp32 divide gives it).
// Packed canonically: byte i = code[2i] | code[2i+1] << 4.
#pragma once

#include "hq_internal.h"

namespace hq {

#pragma clang fp contract(off)

// x: the 32 input values as fp32 (exact copies of 16-bit data).
// packed[w] holds channels 8w..8w+7 (nibble n = channel 8w+n).
__device__ inline void int4_quant_group(const float (&x)[kGroup], uint32_t (&packed)[4],
                                        uint32_t& s_bits, uint32_t& z_bits) {
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int i = 1; i < kGroup; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
    }
    const float d = mx - mn;
    const float sq = d / 15.0f;
    const _Float16 s16 = (_Float16)sq;
    const _Float16 z16 = (_Float16)mn;
    const float s = (float)s16;
    const float z = (float)z16;
    s_bits = (uint32_t)__builtin_bit_cast(uint16_t, s16);
    z_bits = (uint32_t)__builtin_bit_cast(uint16_t, z16);
    // diff / s, correctly rounded, without a full divide per element: y is
    // the correctly rounded reciprocal (one IEEE divide per group), q0 = diff * y
    // is within a few ulps, one FMA residual step makes it faithful, and by
    // Markstein's theorem (faithful quotient, reciprocal within half an ulp,
    // exact FMA residual) a second step gives the correctly rounded quotient.
    // An infinite diff (z rounded to -inf in fp16) keeps diff * y, whose sign
    // and infinity are those of the quotient; s = 0, inf or NaN end as code 0
    // on both forms.
    const float y = 1.0f / s;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const float diff = x[8 * w + n] - z;
            const float q0 = diff * y;
            const float q1 = fmaf(fmaf(-q0, s, diff), y, q0);
            const float q2 = fmaf(fmaf(-q1, s, diff), y, q1);
            const float qv = __builtin_isfinite(q0) ? q2 : q0;
            float c = rintf(qv);
            c = fminf(fmaxf(c, 0.0f), 15.0f);
            const uint32_t code = (s > 0.0f) ? (uint32_t)c : 0u;
            word |= code << (4 * n);
        }
        packed[w] = word;
    }
}

// Unpack 8 bf16/fp16 values of a 16-byte chunk into fp32.
template <bool F16>
__device__ inline void unpack8(const uint4& u, float* out) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = h16_to_f32<F16>(w[i] & 0xFFFFu);
        out[2 * i + 1] = h16_to_f32<F16>(w[i] >> 16);
    }
}

#pragma clang fp contract(on)

}  // namespace hq
