// hq_decode_attn: split-K decode attention over the hybrid KV cache (gfx950).
//
// HyQuant pages: "HyQuant: Hybrid-Precision Quantization for LLM
// Attention", TL;DR and "Key results" (KV dequantization fused into the
// decode attention so dequantized values never round-trip through memory);
// "How HyQuant uses hybrid-precision attention to cut decode compute", "What
// hybrid-precision attention changes" (no full-precision copy of the cache is
// expanded first). The low-bit and 16-bit paths share one online-softmax
// state ("HyQuant: ...", "How this relates to prior wiki pages").
//
// Design (MI355X, wave64, HBM-bound, VALU-heavy):
//  * One workgroup = 4 waves = one (b, g) and a contiguous span of 64-token
//    tiles (a split); every wave takes every 4th tile of the span. All G query
//    heads of the KV head are processed together, so each cache byte is read
//    once per step.
//  * Token phase, lane = token: the lane loads its token's 64 B of K codes
//    (4 x 128-bit, contiguous across the wave) and its K and V scales/zeros.
//    Codes become bf16 (or fp16) "128 + 8c" magic values with one shift + one
//    and-or per pair and meet the query in v_dot2 (exact products, fp32
//    accumulation); the group's scale and zero are applied afterwards:
//    q.k~ = s * (q/8 . (128 + 8c)) + (z - 16 s) * sum(q). Query pairs are
//    uniform and live in scalar registers.
//  * Online softmax per tile in log2 units (v_exp_f32) with a lazy rescale
//    (only when the running max grows by more than 2^8); wave maxima use DPP
//    and v_permlane16/32_swap, no LDS.
//  * PV on INT4 tiles: the V codes are stored pre-paired, slot t with slot
//    t + 32, so the weights w = p * s * 2^-E of the two tokens form one fp16
//    pair (one v_permlane32_swap); the channel-phase lane (8 channels x 16
//    tokens) turns each code pair into fp16 "1024 + c" / "64 + c" magic
//    values with one v_bfi_b32 and accumulates with v_dot2_f32_f16 in fp32. E is a running power-of-two
//    scale (exact rescale when it grows) keeping every w below 2^15, so the
//    fp16 weights stay finite and normal down to p*s ~ 2^-29 of the bound.
//    The magic bias is removed exactly with the sum of the same fp16 weights;
//    sum(p*z) accumulates in fp32 in the token phase.
//  * 16-bit tiles (kept columns, window ring) use fp32 FMAs on the 16-bit
//    rows.
//  * Each workgroup writes one partial (m, l, o[128]) per head; a second
//    kernel merges the splits of each (b, g) (split weights staged in LDS,
//    coalesced partial reads).
#include "hq_internal.h"

namespace hq {
namespace {

constexpr int kWaves = 4;
constexpr float kLazy = 8.0f;  // log2-domain growth that triggers a rescale

struct DecodeParams {
    hq_cache c;
    const uint32_t* qp;    // [B][Hkv][4][G][16]  pairs for the INT4 path (prescaled)
    const uint32_t* qn;    // [B][Hkv][G][64]     natural pairs for the 16-bit path
    const float* qsum;     // [B][Hkv][G][4]      per-group sum of q
    float* part_m;         // [B][Hkv][nsplit][G]
    float* part_l;         // [B][Hkv][nsplit][G]
    float* part_o;         // [B][Hkv][nsplit][G][128]
    int32_t nsplit, tps, G;
    float scale2;          // sm_scale * log2(e)
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <bool F16>
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c,
                                      false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ inline float dot2h(uint32_t a, uint32_t b, float c) { return dot2<true>(a, b, c); }

// (a & mask) | c for c & mask == 0, in one v_bfi_b32 with register constants
// (a VOP3 op cannot take two literals, so the compiler would otherwise emit and + or).
__device__ inline uint32_t bfi(uint32_t mask, uint32_t a, uint32_t c) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(mask), "v"(a), "v"(c));
    return r;
}

// Four magic-biased code pairs from one dword of 8 nibbles (channels 8i+n) for
// the QK dot products. Pair n holds channels (n, n+4). bf16: value 128 + 8c
// (code in bits 3..6); fp16: value 1024 + 16c (code in bits 4..7).
template <bool F16>
__device__ inline void extract_pairs(uint32_t w, uint32_t* pr, uint32_t M, uint32_t C) {
    if constexpr (F16) {
        pr[0] = bfi(M, w << 4, C);
        pr[1] = bfi(M, w, C);
        pr[2] = bfi(M, w >> 4, C);
        pr[3] = bfi(M, w >> 8, C);
    } else {
        pr[0] = bfi(M, w << 3, C);
        pr[1] = bfi(M, w >> 1, C);
        pr[2] = bfi(M, w >> 5, C);
        pr[3] = bfi(M, w >> 9, C);
    }
}
// The V-code word of slots (P, P+32), channels 4Q+n: fp16 magic pairs with
// one bfi each (and one shift for n >= 2). Even channels (code in bits 0..3)
// read 1024 + c with magic 0x6400, odd channels (bits 4..7) read 64 + c with
// magic 0x5400: every channel carries the code with factor 1.
__device__ inline void extract_vpairs(uint32_t d, uint32_t* cp, uint32_t M_lo, uint32_t M_hi, uint32_t C_lo,
                                      uint32_t C_hi) {
    const uint32_t d8 = d >> 8;
    cp[0] = bfi(M_lo, d, C_lo);
    cp[1] = bfi(M_hi, d, C_hi);
    cp[2] = bfi(M_lo, d8, C_lo);
    cp[3] = bfi(M_hi, d8, C_hi);
}
template <bool F16>
constexpr float kBias = F16 ? 64.0f : 16.0f;

__device__ inline uint32_t u4w(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int CTRL>
__device__ inline float dppmov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Maximum over the 64 lanes, every lane gets it (no LDS traffic).
__device__ inline float wave_max_fast(float v) {
    v = fmaxf(v, dppmov<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dppmov<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dppmov<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dppmov<0x140>(v));  // row_mirror
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}
// Lanes 0..31 receive the value of lane l + 32 (lanes 32..63 get junk).
__device__ inline float upper_half(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[1]);
}
template <int CTRL>
__device__ inline float dpp_add(float v) { return v + dppmov<CTRL>(v); }
// Sum over the 64 lanes, every lane gets it (no LDS traffic).
__device__ inline float wave_sum_fast(float v) {
    v = dpp_add<0xB1>(v);
    v = dpp_add<0x4E>(v);
    v = dpp_add<0x141>(v);
    v = dpp_add<0x140>(v);
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

__device__ inline void lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ inline void store_out(void* out, int dt, size_t i, float r) {
    if (dt == HQ_F32)
        static_cast<float*>(out)[i] = r;
    else if (dt == HQ_F16)
        static_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_f16_bits(r);
    else {
        uint32_t x = __float_as_uint(r);
        x += 0x7FFFu + ((x >> 16) & 1u);
        static_cast<uint16_t*>(out)[i] = (uint16_t)(x >> 16);
    }
}

template <int G, bool F16>
__global__ __launch_bounds__(256) void k_decode_split(DecodeParams p) {
    // fp16 weight pairs of the INT4 tile: word (pair P, group g, head h) at
    // P*4G + ((g ^ (P/8 % 4)) * G) + h
    __shared__ uint32_t lds_pw[kWaves][32 * 4 * G];
    __shared__ float lds_p[kWaves][kTile * G];          // 16-bit tiles: p per token
    __shared__ float lds_m[kWaves][G], lds_l[kWaves][G];
    __shared__ float lds_o[kWaves][G][kD];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int Hkv = p.c.Hkv, W = p.c.window;
    const int bg = b * Hkv + g;
    const int4 cnt = *reinterpret_cast<const int4*>(p.c.counts + 4 * bg);
    const int T = cnt.x, n_q = cnt.y, n_keep = cnt.z;
    const int nring = T < W ? T : W;
    const int nqt = (n_q + kTile - 1) / kTile, nkt = (n_keep + kTile - 1) / kTile;
    const int nwt = (nring + kTile - 1) / kTile;
    const int total = nqt + nkt + nwt;
    const int v0 = s * p.tps;
    if (v0 >= total) return;
    const int v1 = min(v0 + p.tps, total);

    const int qt_cap = p.c.cap_q / kTile, kt_cap = p.c.cap_keep / kTile, wt_cap = W / kTile;
    const uint32_t* qp = p.qp + (size_t)bg * 4 * G * 16;
    const uint32_t* qn = p.qn + (size_t)bg * G * 64;
    const float* qs = p.qsum + (size_t)bg * G * 4;

    // token-phase state
    float m[G], l[G], zacc[G][4], wsum[G][4];
    // channel-phase state, in units of 2^E / 16: INT4 tiles add magic-biased
    // sums (bias removed at the end with wsum), 16-bit tiles add p*v*16*2^-E
    float acc[G][8];
    int E = -1000;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) zacc[h][i] = wsum[h][i] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }
    const int u = lane >> 4, c8 = lane & 15, gk = c8 >> 2;
    uint32_t* pw_w = lds_pw[wave];
    float* p_w = lds_p[wave];
    const uint32_t ONES = 0x3C003C00u;  // fp16 (1, 1)
    // extraction constants kept in VGPRs (opaque to constant folding)
    uint32_t kM = F16 ? 0x00F000F0u : 0x00780078u, kC = F16 ? 0x64006400u : 0x43004300u;
    uint32_t vMlo = 0x000F000Fu, vMhi = 0x00F000F0u, vClo = 0x64006400u, vChi = 0x54005400u;
    asm("" : "+v"(kM), "+v"(kC), "+v"(vMlo), "+v"(vMhi), "+v"(vClo), "+v"(vChi));
    float s_thr = 0.f;  // 2^(E+7): a V scale at or above it needs a larger E

    for (int v = v0 + wave; v < v1; v += kWaves) {
        float lg[G];
        const bool int4_tile = v < nqt;
        int count, tile;
        float vs[4], vz[4];
        uint4 vw[4];
        if (int4_tile) {
            // ----------------------------- token phase, INT4 tile
            tile = v;
            count = n_q;
            const bool valid = tile * kTile + lane < n_q;
            const uint8_t* kc = reinterpret_cast<const uint8_t*>(p.c.k_codes) +
                                ((size_t)bg * qt_cap + tile) * kTileBytesQ;
            const size_t slot_g = (size_t)bg * p.c.cap_q + tile * kTile + lane;
            uint4 kw[4];
#pragma unroll
            for (int grp = 0; grp < 4; ++grp)
                kw[grp] = *reinterpret_cast<const uint4*>(kc + kcode_off(lane, grp));
            uint4 km = reinterpret_cast<const uint4*>(p.c.k_meta)[slot_g];
            uint4 vm = reinterpret_cast<const uint4*>(p.c.v_meta)[slot_g];
            {   // V codes requested before QK so their latency overlaps the QK work
                const uint8_t* vc = reinterpret_cast<const uint8_t*>(p.c.v_codes) +
                                    ((size_t)bg * qt_cap + tile) * kTileBytesQ;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) vw[kk] = *reinterpret_cast<const uint4*>(vc + kk * 1024 + lane * 16);
            }
            if (!valid) {
                km = make_uint4(0, 0, 0, 0);
                vm = km;
            }
#pragma unroll
            for (int h = 0; h < G; ++h) lg[h] = 0.f;
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const uint32_t mk = u4w(km, grp), mv = u4w(vm, grp);
                const float sk = f16_to_f32(mk & 0xFFFFu), zk = f16_to_f32(mk >> 16);
                vs[grp] = f16_to_f32(mv & 0xFFFFu);
                vz[grp] = f16_to_f32(mv >> 16);
                const float zz = zk - kBias<F16> * sk;
                uint32_t pr[16];
#pragma unroll
                for (int i = 0; i < 4; ++i) extract_pairs<F16>(u4w(kw[grp], i), pr + 4 * i, kM, kC);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint32_t* qh = qp + (grp * G + h) * 16;
                    float a = 0.f;
#pragma unroll
                    for (int e = 0; e < 16; ++e) a = dot2<F16>(pr[e], qh[e], a);
                    lg[h] = fmaf(sk, a, fmaf(zz, qs[h * 4 + grp], lg[h]));
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) lg[h] = valid ? lg[h] * p.scale2 : -INFINITY;
        } else {
            // ----------------------------- token phase, 16-bit tile
            const bool keep = v < nqt + nkt;
            tile = keep ? v - nqt : v - nqt - nkt;
            count = keep ? n_keep : nring;
            const bool valid = tile * kTile + lane < count;
            const uint8_t* kt = keep ? reinterpret_cast<const uint8_t*>(p.c.k_keep) +
                                           ((size_t)bg * kt_cap + tile) * kTileBytes16
                                     : reinterpret_cast<const uint8_t*>(p.c.k_win) +
                                           ((size_t)bg * wt_cap + tile) * kTileBytes16;
#pragma unroll
            for (int h = 0; h < G; ++h) lg[h] = 0.f;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const uint4 kk = *reinterpret_cast<const uint4*>(kt + k16_off(lane, c));
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const uint32_t* qh = qn + h * 64 + 4 * c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) lg[h] = dot2<F16>(u4w(kk, i), qh[i], lg[h]);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) lg[h] = valid ? lg[h] * p.scale2 : -INFINITY;
        }

        // ----------------------------- online softmax (wave-uniform update)
        float pr_h[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            // lazy max: the full reduction only runs when some logit exceeds m + 2^8
            if (__any(lg[h] > m[h] + kLazy)) {
                const float tmax = wave_max_fast(lg[h]);
                const float alpha = __builtin_amdgcn_exp2f(m[h] - tmax);
                m[h] = tmax;
                l[h] *= alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    zacc[h][i] *= alpha;
                    wsum[h][i] *= alpha;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] *= alpha;
            }
            pr_h[h] = __builtin_amdgcn_exp2f(lg[h] - m[h]);
            l[h] += pr_h[h];
        }

        if (int4_tile) {
            // running power-of-two scale 2^E with p*s*2^-E < 2^15 (p <= 2^8 by the lazy
            // rescale, s < 2^(e_s+1)): fp16 weights stay finite and mostly normal
            const float s4 = fmaxf(fmaxf(vs[0], vs[1]), fmaxf(vs[2], vs[3]));
            if (__any(s4 >= s_thr && s4 > 0.f)) {
                const float smax = wave_max_fast(s4);
                const int e_need = (int)((__float_as_uint(smax) >> 23) & 0xFF) - 127 - 6;
                const float r = E <= -1000 ? 0.f : (e_need > E ? __builtin_ldexpf(1.0f, E - e_need) : 1.0f);
#pragma unroll
                for (int h = 0; h < G; ++h) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[h][i] *= r;
#pragma unroll
                    for (int i = 0; i < 4; ++i) wsum[h][i] *= r;
                }
                E = e_need > E ? e_need : E;
                s_thr = __builtin_ldexpf(1.0f, E + 7);
            }
            const float f = E <= -1000 ? 1.0f : __builtin_ldexpf(1.0f, -E);
            // fp16 weight pairs (slot lane, slot lane + 32), built by lanes 0..31
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const float sf = vs[grp] * f;
                uint32_t words[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    zacc[h][grp] = fmaf(pr_h[h], vz[grp], zacc[h][grp]);
                    const float w = pr_h[h] * sf;
                    const float w2 = upper_half(w);
                    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
                    h2_t pk = {(_Float16)w, (_Float16)w2};
                    words[h] = __builtin_bit_cast(uint32_t, pk);
                    wsum[h][grp] = dot2h(words[h], ONES, wsum[h][grp]);
                }
                if (lane < 32) {
                    const int P = lane;
                    uint32_t* dst = pw_w + P * 4 * G + ((grp ^ ((P >> 3) & 3)) * G);
#pragma unroll
                    for (int h = 0; h < G; ++h) dst[h] = words[h];
                }
            }
            lds_fence();
            // ----------------------------- channel phase, INT4 V
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int P = 8 * u + j;
                uint32_t pw[G];
                const uint32_t* src = pw_w + P * 4 * G + ((gk ^ u) * G);
#pragma unroll
                for (int h = 0; h < G; ++h) pw[h] = src[h];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t d = u4w(vw[j >> 1], (j & 1) * 2 + e);
                    uint32_t cp[4];
                    extract_vpairs(d, cp, vMlo, vMhi, vClo, vChi);
#pragma unroll
                    for (int n = 0; n < 4; ++n)
#pragma unroll
                        for (int h = 0; h < G; ++h) acc[h][4 * e + n] = dot2h(cp[n], pw[h], acc[h][4 * e + n]);
                }
            }
            lds_fence();
        } else {
            if (E <= -1000) E = 0;  // no INT4 tile yet: fix the accumulator unit
            const float k16 = __builtin_ldexpf(1.0f, -E);
#pragma unroll
            for (int h = 0; h < G; ++h) p_w[lane * G + h] = pr_h[h] * k16;
            lds_fence();
            // ----------------------------- channel phase, 16-bit V
            const bool keep = v < nqt + nkt;
            const uint8_t* vt = keep ? reinterpret_cast<const uint8_t*>(p.c.v_keep) +
                                           ((size_t)bg * kt_cap + tile) * kTileBytes16
                                     : reinterpret_cast<const uint8_t*>(p.c.v_win) +
                                           ((size_t)bg * wt_cap + tile) * kTileBytes16;
#pragma unroll 4
            for (int i = 0; i < 16; ++i) {
                const int slot = 16 * u + i;
                const uint4 vv = *reinterpret_cast<const uint4*>(vt + i * 1024 + lane * 16);
                if (tile * kTile + slot < count) {
                    float x[8];
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        x[2 * w] = h16_to_f32<F16>(u4w(vv, w) & 0xFFFFu);
                        x[2 * w + 1] = h16_to_f32<F16>(u4w(vv, w) >> 16);
                    }
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        const float pw = p_w[slot * G + h];
#pragma unroll
                        for (int ch = 0; ch < 8; ++ch) acc[h][ch] = fmaf(pw, x[ch], acc[h][ch]);
                    }
                }
            }
            lds_fence();
        }
    }

    // ----------------------------- wave epilogue
    // acc units: o = 2^E * (acc - bias * wsum) + sum(p z), bias 1024 on even
    // and 64 on odd channels (the fp16 magic values); 16-bit tiles added
    // p*v*2^-E directly.
    const float unit = E <= -1000 ? 0.f : __builtin_ldexpf(1.0f, E);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        l[h] = wave_sum_fast(l[h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            zacc[h][i] = wave_sum_fast(zacc[h][i]);
            wsum[h][i] = unit * wave_sum_fast(lane < 32 ? wsum[h][i] : 0.f);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            acc[h][i] += __shfl_xor(acc[h][i], 16);
            acc[h][i] += __shfl_xor(acc[h][i], 32);
        }
    }
    if (lane < 16) {
        const int gq = lane >> 2;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float z_even = fmaf(-1024.0f, wsum[h][gq], zacc[h][gq]);
            const float z_odd = fmaf(-64.0f, wsum[h][gq], zacc[h][gq]);
#pragma unroll
            for (int i = 0; i < 8; ++i) lds_o[wave][h][8 * lane + i] = fmaf(unit, acc[h][i], (i & 1) ? z_odd : z_even);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            lds_m[wave][h] = m[h];
            lds_l[wave][h] = l[h];
        }
    }
    __syncthreads();
    // ----------------------------- merge the waves, write the split partial
    const size_t pbase = ((size_t)bg * p.nsplit + s) * G;
    for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
        const int h = idx / kD, d = idx % kD;
        float M = lds_m[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, lds_m[w][h]);
        float o = 0.f, L = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = lds_m[w][h];
            const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            o = fmaf(f, lds_o[w][h][d], o);
            L = fmaf(f, lds_l[w][h], L);
        }
        p.part_o[(pbase + h) * kD + d] = o;
        if (d == 0) {
            p.part_m[pbase + h] = M;
            p.part_l[pbase + h] = L;
        }
    }
}

// Rearranges the query for the split kernel: INT4-path pairs (prescaled by
// 1/8 for bf16, 1/16 for fp16, exact), natural pairs and group sums.
template <bool F16>
__global__ __launch_bounds__(1024) void k_decode_prep(const uint16_t* q, int Hq, int G, uint32_t* qp,
                                                      uint32_t* qn, float* qsum) {
    const int g = blockIdx.x, b = blockIdx.y, Hkv = gridDim.x;
    const int bg = b * Hkv + g;
    const int h = threadIdx.x >> 7, t = threadIdx.x & 127;   // one thread per (head, channel)
    const float sc = F16 ? 0.0625f : 0.125f;
    const uint16_t* qh = q + ((size_t)b * Hq + g * G + h) * kD;
    if (t < 64) {
        qn[((size_t)bg * G + h) * 64 + t] = (uint32_t)qh[2 * t] | ((uint32_t)qh[2 * t + 1] << 16);
        // INT4 arrangement: entry (grp, 4i + n) = (q[32grp+8i+n], q[32grp+8i+n+4]) * 2^-3 / 2^-4
        const int grp = t >> 4, e = t & 15, i = e >> 2, n = e & 3;
        const int d0 = 32 * grp + 8 * i + n;
        const float a = h16_to_f32<F16>(qh[d0]) * sc, c = h16_to_f32<F16>(qh[d0 + 4]) * sc;
        uint32_t wa, wc;
        if constexpr (F16) {
            wa = f32_to_f16_bits(a);
            wc = f32_to_f16_bits(c);
        } else {
            wa = __float_as_uint(a) >> 16;  // exact: power-of-two scaling of a bf16 value
            wc = __float_as_uint(c) >> 16;
        }
        qp[(((size_t)bg * 4 + grp) * G + h) * 16 + e] = wa | (wc << 16);
    }
    // group sums of exactly the values the pairs carry (rescaled), in double
    float a = h16_to_f32<F16>(qh[t]) * sc;
    if constexpr (F16) a = f16_to_f32(f32_to_f16_bits(a));
    double acc = (double)a;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) acc += __shfl_xor(acc, o);
    if ((t & 31) == 0) qsum[((size_t)bg * G + h) * 4 + (t >> 5)] = (float)(acc / sc);
}

__global__ __launch_bounds__(128) void k_decode_reduce(const hq_cache c, const float* part_m, const float* part_l,
                                                       const float* part_o, int nsplit, int tps, int G, int Hq,
                                                       void* out, int out_dt) {
    extern __shared__ float sh[];  // [nsplit] weights, then 1/L
    const int gh = blockIdx.x, b = blockIdx.y;
    const int g = gh / G, h = gh % G, d = threadIdx.x;
    const int bg = b * c.Hkv + g;
    const int4 cnt = *reinterpret_cast<const int4*>(c.counts + 4 * bg);
    const int T = cnt.x, n_q = cnt.y, n_keep = cnt.z;
    const int nring = T < c.window ? T : c.window;
    const int total = (n_q + kTile - 1) / kTile + (n_keep + kTile - 1) / kTile + (nring + kTile - 1) / kTile;
    const int active = min((total + tps - 1) / tps, nsplit);
    const size_t base = (size_t)bg * nsplit * G + h;
    float* wsp = sh;
    __shared__ float red[2];
    // split weights 2^(m_s - M) and 1/L, one split per thread
    float ms = -INFINITY, ls = 0.f;
    if (d < active) {
        ms = part_m[base + (size_t)d * G];
        ls = part_l[base + (size_t)d * G];
    }
    for (int i = d + 128; i < active; i += 128) {  // more than 128 splits: fold
        const float m2 = part_m[base + (size_t)i * G];
        if (m2 > ms) ms = m2;
    }
    float M = wave_max(ms);
    if ((d & 63) == 0) red[d >> 6] = M;
    __syncthreads();
    M = fmaxf(red[0], red[1]);
    __syncthreads();
    float L = 0.f;
    for (int i = d; i < active; i += 128) {
        const float mi = part_m[base + (size_t)i * G];
        const float f = mi == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mi - M);
        wsp[i] = f;
        L = fmaf(f, part_l[base + (size_t)i * G], L);
    }
    (void)ls;
    L = wave_sum(L);
    if ((d & 63) == 0) red[d >> 6] = L;
    __syncthreads();
    const float invL = 1.0f / (red[0] + red[1]);
    const float* po = part_o + base * kD + d;
    float O[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int sp = 0;
    for (; sp + 8 <= active; sp += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) O[j] = fmaf(wsp[sp + j], po[(size_t)(sp + j) * G * kD], O[j]);
    }
    for (; sp < active; ++sp) O[0] = fmaf(wsp[sp], po[(size_t)sp * G * kD], O[0]);
    const float r = (((O[0] + O[1]) + (O[2] + O[3])) + ((O[4] + O[5]) + (O[6] + O[7]))) * invL;
    store_out(out, out_dt, ((size_t)b * Hq + g * G + h) * kD + d, r);
}

struct WsLayout {
    size_t qp, qn, qsum, pm, pl, po, total;
};
inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
WsLayout ws_layout(const hq_cache& c, int32_t Hq, int32_t nsplit) {
    const size_t BG = (size_t)c.B * c.Hkv;
    const int G = Hq / c.Hkv;
    WsLayout w;
    w.qp = 0;
    w.qn = w.qp + al(BG * 4 * G * 16 * 4);
    w.qsum = w.qn + al(BG * G * 64 * 4);
    w.pm = w.qsum + al(BG * G * 4 * 4);
    w.pl = w.pm + al(BG * nsplit * G * 4);
    w.po = w.pl + al(BG * nsplit * G * 4);
    w.total = w.po + al(BG * nsplit * G * kD * 4);
    return w;
}

template <int G, bool F16>
void launch_split(const DecodeParams& p, dim3 grid, hipStream_t s) {
    k_decode_split<G, F16><<<grid, 256, 0, s>>>(p);
}

}  // namespace

int32_t decode_max_tiles(const hq_cache& c) {
    return c.cap_q / kTile + c.cap_keep / kTile + c.window / kTile;
}

size_t decode_ws_bytes(const hq_cache& c, int32_t Hq, int32_t nsplit) {
    return ws_layout(c, Hq, nsplit).total;
}

hipError_t launch_decode(const hq_cache& c, const void* q, void* out, hq_dtype out_dt,
                         const DecodeLaunch& d, hipStream_t s) {
    const WsLayout w = ws_layout(c, d.Hq, d.nsplit);
    char* ws = static_cast<char*>(d.ws);
    DecodeParams p;
    p.c = c;
    p.qp = reinterpret_cast<uint32_t*>(ws + w.qp);
    p.qn = reinterpret_cast<uint32_t*>(ws + w.qn);
    p.qsum = reinterpret_cast<float*>(ws + w.qsum);
    p.part_m = reinterpret_cast<float*>(ws + w.pm);
    p.part_l = reinterpret_cast<float*>(ws + w.pl);
    p.part_o = reinterpret_cast<float*>(ws + w.po);
    p.nsplit = d.nsplit;
    p.tps = d.tiles_per_split;
    p.G = d.G;
    p.scale2 = d.sm_scale_log2;
    const bool f16 = c.dt == HQ_F16;
    dim3 pg(c.Hkv, c.B);
    if (f16)
        k_decode_prep<true><<<pg, 128 * d.G, 0, s>>>(static_cast<const uint16_t*>(q), d.Hq, d.G,
                                               const_cast<uint32_t*>(p.qp), const_cast<uint32_t*>(p.qn),
                                               const_cast<float*>(p.qsum));
    else
        k_decode_prep<false><<<pg, 128 * d.G, 0, s>>>(static_cast<const uint16_t*>(q), d.Hq, d.G,
                                                const_cast<uint32_t*>(p.qp), const_cast<uint32_t*>(p.qn),
                                                const_cast<float*>(p.qsum));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid(d.nsplit, c.Hkv, c.B);
    switch (d.G * 2 + (f16 ? 1 : 0)) {
        case 2: launch_split<1, false>(p, grid, s); break;
        case 3: launch_split<1, true>(p, grid, s); break;
        case 4: launch_split<2, false>(p, grid, s); break;
        case 5: launch_split<2, true>(p, grid, s); break;
        case 8: launch_split<4, false>(p, grid, s); break;
        case 9: launch_split<4, true>(p, grid, s); break;
        case 16: launch_split<8, false>(p, grid, s); break;
        case 17: launch_split<8, true>(p, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t shb = (size_t)d.nsplit * sizeof(float);
    k_decode_reduce<<<dim3(c.Hkv * d.G, c.B), 128, shb, s>>>(c, p.part_m, p.part_l, p.part_o, d.nsplit,
                                                              d.tiles_per_split, d.G, d.Hq, out, (int)out_dt);
    return hipGetLastError();
}

}  // namespace hq
