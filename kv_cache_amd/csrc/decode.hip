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
// Design (MI355X, wave64). One workgroup = 4 waves = one (b, g) and a
// contiguous span of 64-token tiles (a split); every wave takes every 4th
// tile of the span. All G query heads of the KV head are processed together,
// so each cache byte is read once per step.
//
// INT4 tiles run on the matrix cores: with G query heads per KV head, QK and
// PV of a tile are small dense products, and on gfx950 a 16x16x32 fp16 MFMA
// does the work of ~64 VALU dot2 instructions in a sixteenth of their issue
// time even with 12 of its 16 columns idle. The codes are dequantized in
// registers, never written back:
//  * QK: D[4j+h][t] = sum over group j of q'_h[c] * (bias_c + code[t][c]),
//    with A = the query (row 4j+h is head h restricted to group j, so the 16
//    rows cover 4 groups x 4 heads and one accumulator holds the per-group
//    partial dots) and B = the K codes turned into fp16 "1024 + c" / "64 + c"
//    values by one and-or per register (plus one shift per word). The
//    accumulator starts at -sum(q' * bias); the group's scale and zero are
//    applied per (token, group) lane, the four groups are summed through an
//    LDS transpose that lands one token per lane for the softmax. q' is the
//    query scaled per head by a power of two into fp16 range (exact).
//  * Online softmax per tile in log2 units with a lazy rescale (only when
//    the running max grows by more than 2^8).
//  * PV: D[c][h] += sum_t (bias_t + code[t][c]) * w[t][h] with A = the V
//    codes (same extraction) and B = fp16 weights w = p * s_v * 2^-E staged
//    through LDS. E is a running power of two keeping every w below 2^15;
//    the bias is removed exactly with the sum of the same fp16 weights and
//    sum(p * z_v) is accumulated in fp32 per token.
//  * The query operands (q', the per-group sums, the per-head scale) are
//    built in LDS by each INT4 workgroup while its first two tiles are in
//    flight; a separate launch for them costs more than the work itself.
//  * 16-bit tiles (kept columns, window ring) use v_dot2 / fp32 FMAs on the
//    16-bit rows (they are a few percent of the tiles), with every K and V
//    load of a tile issued before its first use.
//  * Each workgroup writes one partial (m, l, o[128]) per head; a second
//    kernel merges the splits of each (b, g).
#include <atomic>

#include "hq_internal.h"

namespace hq {
namespace {

constexpr int kWaves = 4;
constexpr float kLazy = 8.0f;  // log2-domain growth that triggers a rescale

typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));

constexpr int kTps16 = 16;  // 16-bit tiles per split

struct DecodeParams {
    hq_cache c;
    const uint32_t* qw;    // [B][Hq][64] query words (channels 2c, 2c + 1 of word c); 16-byte aligned
    int32_t Hq;
    float* part_m;         // [B][Hkv][nsplit][G]
    float* part_l;         // [B][Hkv][nsplit][G]
    float* part_o;         // [B][Hkv][nsplit][G][128]
    int32_t nsplit, G;     // G: query heads per KV head (the partials' and the query's head count)
    int32_t nsq;           // INT4 splits (the first nsq partials of a (b, g))
    int32_t halves;        // 2: the kernel's heads are half of G, the two halves run as separate workgroups
    float scale2;          // sm_scale * log2(e)
};

template <bool F16>
__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (F16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                               false);
}

__device__ inline uint32_t u4w(const uint4& v, int i) { return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w; }

// The 8 codes of one operand word -> fp16 operand registers (elements 2k, 2k+1
// in register k): nibbles at bits 0..3 of a half read 1024 + c (magic 0x6400),
// at bits 4..7 read 64 + c (magic 0x5400). The masks and magics are passed in
// VGPRs so that each register is one v_and_or_b32 (a VOP3 instruction can
// read only one literal constant).
struct CodeConsts {
    uint32_t m_lo, m_hi, c_lo, c_hi;
};
__device__ inline CodeConsts code_consts() {
    CodeConsts k{0x000F000Fu, 0x00F000F0u, 0x64006400u, 0x54005400u};
    asm("" : "+v"(k.m_lo), "+v"(k.m_hi), "+v"(k.c_lo), "+v"(k.c_hi));
    return k;
}
__device__ inline halfx8 codes_to_f16(uint32_t d, const CodeConsts& k) {
    const uint32_t d8 = d >> 8;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {(d & k.m_lo) | k.c_lo, (d & k.m_hi) | k.c_hi, (d8 & k.m_lo) | k.c_lo, (d8 & k.m_hi) | k.c_hi};
    return __builtin_bit_cast(halfx8, v);
}
// Magic bias of operand element e (= slot or channel index mod 8).
__device__ inline float elem_bias(int e) { return (e & 2) ? 64.0f : 1024.0f; }

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

// fp64 sum over each 16-lane row, every lane gets its row's sum: DPP moves
// on both words of the double (quad swaps, then the half-row and row
// mirrors), no LDS round trips.
template <int CTRL>
__device__ inline double dpp_d(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)u, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(u >> 32), (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ inline double row16_sum_d(double v) {
    v += dpp_d<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_d<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_d<0x141>(v);  // row_half_mirror
    v += dpp_d<0x140>(v);  // row_mirror
    return v;
}

// Sum over the four 16-lane rows: lane l gets v(l) + v(l^32) + v(l^16) +
// v(l^48) (two swaps between halves / rows, no LDS traffic).
__device__ inline float rows_sum4(float v) {
    auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
    auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
}

// Orders this wave's LDS writes before its later LDS reads (other lanes'
// data). LDS operations of one wave execute in order, so this only has to
// stop the compiler from reordering; it must not wait for global loads.
__device__ inline void lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
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


// MODE 0: the n INT4 tiles of a (b, g); split s = blockIdx.x < nsq covers
// tiles [s*n/nsq, (s+1)*n/nsq). MODE 1: its 16-bit tiles (kept, then ring),
// divided the same way over the remaining splits; split s writes partial
// nsq + s. Every workgroup writes its partial (empty ones carry m = -inf).
template <int G>
struct SplitSmem {
    static constexpr int NHB = (G + 3) / 4;
    float4 y[kWaves][4 * NHB * 64];
    __align__(16) uint16_t w[kWaves][4 * 2 * 4 * G * 8];
    float p[kWaves][kTile * G];
    float m[kWaves][G], l[kWaves][G];
    float o[kWaves][G][kD];
    uint4 qa[NHB * 4 * 64];
    float qc[NHB * 4 * 8];  // [hb][group j][head r][sum q' * bias, sum q']
    float qsc[8];           // per head 2^-k
};

template <int G, bool F16, int MODE, bool NT = true>
__device__ __attribute__((always_inline)) inline void split_body(const DecodeParams& p, SplitSmem<G>& sm, int s,
                                                                 int half) {
    constexpr int NHB = (G + 3) / 4;  // 4-head blocks of the QK product
    // per wave: QK partials y[block nb][head block][lane] (float4), the PV
    // weights w[group][token half][token octet][head][8 slots] (fp16), the
    // 16-bit tiles' p per token
    auto& lds_y = sm.y;
    auto& lds_w = sm.w;
    auto& lds_p = sm.p;
    auto& lds_m = sm.m;
    auto& lds_l = sm.l;
    auto& lds_o = sm.o;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (scalar)
    const int g = blockIdx.y, b = blockIdx.z;
    const int Hkv = p.c.Hkv, W = p.c.window;
    const int bg = b * Hkv + g;
    const int4 cnt = *reinterpret_cast<const int4*>(p.c.counts + 4 * bg);
    const int T = cnt.x, n_q = cnt.y, n_keep = cnt.z;
    const int nring = T < W ? T : W;
    const int nqt = (n_q + kTile - 1) / kTile, nkt = (n_keep + kTile - 1) / kTile;
    const int nwt = (nring + kTile - 1) / kTile;
    const int total = nqt + nkt + nwt;
    // the splits of each kind divide that kind's tiles evenly (the launch
    // sizes the split counts for the capacity, the counts give the tiles)
    const int n16s = p.nsplit - p.nsq, n16t = total - nqt;
    const int v0 = MODE == 0 ? s * nqt / p.nsq : nqt + s * n16t / n16s;
    const int v1 = MODE == 0 ? (s + 1) * nqt / p.nsq : nqt + (s + 1) * n16t / n16s;
    const int split_out = MODE == 0 ? s : p.nsq + s;
    if (v0 >= v1) {  // nothing here: an empty partial
        const size_t pb = ((size_t)bg * p.nsplit + split_out) * p.G + half * G;
        for (int idx = threadIdx.x; idx < G * kD; idx += 256) {
            p.part_o[pb * kD + idx] = 0.f;
            if (idx < G) {
                p.part_m[pb + idx] = -INFINITY;
                p.part_l[pb + idx] = 0.f;
            }
        }
        return;
    }

    const int kt_cap = p.c.cap_keep / kTile, wt_cap = W / kTile;
    // the 16-bit tiles take the query's own words: word h*64 + c holds channels 2c, 2c + 1 of head h
    const uint32_t* qn = p.qw + ((size_t)bg * p.G + half * G) * (kD / 2);  // Hq = Hkv * p.G

    // softmax state (lane = token), channel accumulators
    float m[G], l[G], zacc[G][4], wsb[G][4];
    floatx4 dpv[8];                  // INT4 PV: D[16mb + 4(lane/16) + r][head lane%16]
    float acc[G][8];                 // 16-bit PV: channel-phase layout
    int E = -1000;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) zacc[h][i] = wsb[h][i] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) dpv[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int u = lane >> 4;
    float* p_w = lds_p[wave];
    float4* y_w = lds_y[wave];
    uint16_t* w_w = lds_w[wave];
    float s_thr = 0.f;  // 2^(E+7): a V scale at or above it needs a larger E
    const float ebias = elem_bias(lane & 7);  // magic bias of this lane's slot in the PV operand
    const CodeConsts cc = code_consts();

    if constexpr (MODE == 0) {
        struct TileRegs {
            uint4 kd[4], kmv, vmv, vd[4];
        };
        // one (b, g)'s INT4 codes / metadata: its span of the pools, as buffer
        // resources whose range check keeps every load inside the span
        const QSpan qs = q_span(p.c, bg);
        const int wq = qs.tiles * kTileBytesQ;
        const __amdgpu_buffer_rsrc_t rkc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const uint8_t*>(p.c.k_codes) + (size_t)qs.tile0 * kTileBytesQ), (short)0, wq,
            0x00020000);
        const __amdgpu_buffer_rsrc_t rvc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const uint8_t*>(p.c.v_codes) + (size_t)qs.tile0 * kTileBytesQ), (short)0, wq,
            0x00020000);
        const __amdgpu_buffer_rsrc_t rkm = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const uint8_t*>(p.c.k_meta) + (size_t)qs.tile0 * 1024), (short)0, qs.tiles * 1024,
            0x00020000);
        const __amdgpu_buffer_rsrc_t rvm = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(reinterpret_cast<const uint8_t*>(p.c.v_meta) + (size_t)qs.tile0 * 1024), (short)0, qs.tiles * 1024,
            0x00020000);
        const int voff = lane * 16;
        auto ld = [&](const __amdgpu_buffer_rsrc_t& r, int soff) {
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, NT ? kLoadNT : 0));
        };
        auto load_tile = [&](int v, TileRegs& r) {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) r.kd[nb] = ld(rkc, v * kTileBytesQ + nb * 1024);
            r.kmv = ld(rkm, v * 1024);
            r.vmv = ld(rvm, v * 1024);
#pragma unroll
            for (int i = 0; i < 4; ++i) r.vd[i] = ld(rvc, v * kTileBytesQ + i * 1024);
        };
        // The query is loaded first, then the first two tiles, so the query's
        // operands are built while the tiles are in flight (waiting for the
        // query leaves the 20 tile loads outstanding).
        uint32_t qword[(G + kWaves - 1) / kWaves];
#pragma unroll
        for (int i = 0; i * kWaves < G; ++i) {
            const int h = wave + i * kWaves;
            qword[i] = h < G ? qn[h * 64 + lane] : 0u;
        }
        const int t0 = v0 + wave < v1 ? v0 + wave : v0;
        TileRegs ta, tb;
        __builtin_amdgcn_sched_barrier(0);
        load_tile(t0, ta);
        __builtin_amdgcn_sched_barrier(0);  // keep tile t0's loads ahead of tile t0 + 4's
        load_tile(t0 + kWaves < v1 ? t0 + kWaves : t0, tb);
        __builtin_amdgcn_sched_barrier(0);

        // ---- query operands in LDS. Per head a power-of-two scale 2^k into
        // fp16 range (q' = q 2^k, exact for every value above 2^-24 of the
        // head's maximum). Lane l of the wave of head h holds channels 2l,
        // 2l + 1: one word of the QK A operand (K-step ks = l/16 = channel
        // group j, lane 4ks + h%4 + 16((l%16)/4), register l%4); the words of
        // rows that hold another group's head, or no head, are zero. Per group
        // the sums of q' and of q' * bias (exact in fp64, rounded once).
        auto& lds_qa = sm.qa;
        uint32_t* qa32 = reinterpret_cast<uint32_t*>(lds_qa);
        for (int w = threadIdx.x; w < NHB * 1024; w += 256) {
            const int hb = w >> 10, ks = (w >> 8) & 3, mrow = (w >> 2) & 15;
            if ((mrow >> 2) != ks || 4 * hb + (mrow & 3) >= G) qa32[w] = 0u;
        }
        if (threadIdx.x < NHB * 16 && 4 * (threadIdx.x >> 4) + (threadIdx.x & 3) >= G) {
            sm.qc[(threadIdx.x >> 2) * 8 + 2 * (threadIdx.x & 3)] = 0.f;
            sm.qc[(threadIdx.x >> 2) * 8 + 2 * (threadIdx.x & 3) + 1] = 0.f;
        }
#pragma unroll
        for (int i = 0; i * kWaves < G; ++i) {
            const int h = wave + i * kWaves;
            if (h < G) {
                const uint32_t word = qword[i];
                const float x0 = h16_to_f32<F16>(word & 0xFFFFu), x1 = h16_to_f32<F16>(word >> 16);
                const float mx = wave_max_fast(fmaxf(fabsf(x0), fabsf(x1)));
                const int e = mx > 0.f ? (int)((__float_as_uint(mx) >> 23) & 0xFF) - 127 : 0;
                const int k = mx > 0.f ? min(max(14 - e, -100), 100) : 0;
                if (lane == 0) sm.qsc[h] = __builtin_ldexpf(1.0f, -k);
                const uint32_t h0 = f32_to_f16_bits(__builtin_ldexpf(x0, k));
                const uint32_t h1 = f32_to_f16_bits(__builtin_ldexpf(x1, k));
                const int hb = h >> 2, ks = lane >> 4;
                qa32[hb * 1024 + ks * 256 + (4 * ks + (h & 3) + 16 * ((lane & 15) >> 2)) * 4 + (lane & 3)] =
                    h0 | (h1 << 16);
                const double y0 = (double)f16_to_f32(h0), y1 = (double)f16_to_f32(h1);
                const double sq = row16_sum_d(y0 + y1);
                const double sb = row16_sum_d(y0 * (double)elem_bias((2 * lane) & 7) +
                                              y1 * (double)elem_bias((2 * lane + 1) & 7));
                if ((lane & 15) == 0) {
                    sm.qc[(hb * 4 + ks) * 8 + 2 * (h & 3)] = (float)sb;
                    sm.qc[(hb * 4 + ks) * 8 + 2 * (h & 3) + 1] = (float)sq;
                }
            }
        }
        __syncthreads();
        // per-head logit scale 2^-k * sm_scale * log2(e); the QK A operands and
        // the per-group constants of this lane's group j = lane/16
        float qscale[G];
#pragma unroll
        for (int h = 0; h < G; ++h) qscale[h] = sm.qsc[h] * p.scale2;
        floatx4 qb0[NHB];
        float qsj[NHB][4];
        halfx8 qreg[NHB][4];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) qreg[hb][ks] = __builtin_bit_cast(halfx8, lds_qa[(hb * 4 + ks) * 64 + lane]);
            const float* qcj = sm.qc + (hb * 4 + (lane >> 4)) * 8;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                qb0[hb][r] = -qcj[2 * r];
                qsj[hb][r] = qcj[2 * r + 1];
            }
        }

        auto step = [&](int v, const TileRegs& tr) {
            float lg[G];
            float vs[4], vz[4];
            // ----------------------------- QK on the matrix cores, INT4 tile
            const bool valid = v * kTile + lane < n_q;
            const uint4* kd = tr.kd;
            const uint4 kmv = tr.kmv;
            uint4 vmv = tr.vmv;
            const uint4* vd = tr.vd;
            if (!valid) vmv = make_uint4(0, 0, 0, 0);
            // four independent accumulators (one per 16-token block), K-step
            // outer, so consecutive MFMAs do not wait on each other
            floatx4 dq[4][NHB];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int hb = 0; hb < NHB; ++hb) dq[nb][hb] = qb0[hb];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                halfx8 qk[NHB];
#pragma unroll
                for (int hb = 0; hb < NHB; ++hb) qk[hb] = qreg[hb][ks];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const halfx8 kb = codes_to_f16(u4w(kd[nb], ks), cc);
#pragma unroll
                    for (int hb = 0; hb < NHB; ++hb)
                        dq[nb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qk[hb], kb, dq[nb][hb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const uint32_t md = u4w(kmv, nb);
                const float sk = f16_to_f32(md & 0xFFFFu), zk = f16_to_f32(md >> 16);
#pragma unroll
                for (int hb = 0; hb < NHB; ++hb) {
                    float4 y;
                    y.x = fmaf(sk, dq[nb][hb][0], zk * qsj[hb][0]);
                    y.y = fmaf(sk, dq[nb][hb][1], zk * qsj[hb][1]);
                    y.z = fmaf(sk, dq[nb][hb][2], zk * qsj[hb][2]);
                    y.w = fmaf(sk, dq[nb][hb][3], zk * qsj[hb][3]);
                    y_w[(nb * NHB + hb) * 64 + lane] = y;
                }
            }
            lds_fence();
            // lane = token: sum the four group partials
            {
                const int nb = lane >> 4, tl = lane & 15;
#pragma unroll
                for (int hb = 0; hb < NHB; ++hb) {
                    float4 a = y_w[(nb * NHB + hb) * 64 + tl];
#pragma unroll
                    for (int j = 1; j < 4; ++j) {
                        const float4 bq = y_w[(nb * NHB + hb) * 64 + tl + 16 * j];
                        a.x += bq.x;
                        a.y += bq.y;
                        a.z += bq.z;
                        a.w += bq.w;
                    }
                    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * hb + r < G) lg[4 * hb + r] = valid ? av[r] * qscale[4 * hb + r] : -INFINITY;
                }
            }
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const uint32_t mv = u4w(vmv, grp);
                vs[grp] = f16_to_f32(mv & 0xFFFFu);
                vz[grp] = f16_to_f32(mv >> 16);
            }
            // ----------------------------- online softmax (wave-uniform update)
            float pr_h[G];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (__any(lg[h] > m[h] + kLazy)) {
                    const float tmax = wave_max_fast(lg[h]);
                    const float alpha = __builtin_amdgcn_exp2f(m[h] - tmax);
                    m[h] = tmax;
                    l[h] *= alpha;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        zacc[h][i] *= alpha;
                        wsb[h][i] *= alpha;
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[h][i] *= alpha;
#pragma unroll
                    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) dpv[mb][r] = (lane & 15) == h ? dpv[mb][r] * alpha : dpv[mb][r];
                }
                pr_h[h] = __builtin_amdgcn_exp2f(lg[h] - m[h]);
                l[h] += pr_h[h];
            }

            {
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
                        for (int i = 0; i < 4; ++i) wsb[h][i] *= r;
                    }
#pragma unroll
                    for (int mb = 0; mb < 8; ++mb) dpv[mb] *= r;
                    E = e_need > E ? e_need : E;
                    s_thr = __builtin_ldexpf(1.0f, E + 7);
                }
                const float f = E <= -1000 ? 1.0f : __builtin_ldexpf(1.0f, -E);
                // fp16 weights of this token into the B-operand layout
                // w[grp][t/32][(t%32)/8][h][t%8]
                const int wbase = ((lane >> 5) * 4 + ((lane >> 3) & 3)) * G * 8 + (lane & 7);
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    const float sf = vs[grp] * f;
#pragma unroll
                    for (int h = 0; h < G; ++h) {
                        zacc[h][grp] = fmaf(pr_h[h], vz[grp], zacc[h][grp]);
                        const _Float16 w16 = (_Float16)(pr_h[h] * sf);
                        wsb[h][grp] = fmaf(ebias, (float)w16, wsb[h][grp]);
                        w_w[grp * 2 * 4 * G * 8 + wbase + h * 8] = __builtin_bit_cast(uint16_t, w16);
                    }
                }
                lds_fence();
                // ----------------------------- PV on the matrix cores
                const int hs = (lane & 15) < G ? (lane & 15) : 0;
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        const halfx8 wb = __builtin_bit_cast(
                            halfx8, *reinterpret_cast<const uint4*>(w_w + ((grp * 2 + ks) * 4 + (lane >> 4)) * G * 8 + hs * 8));
#pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int mb = 2 * grp + half;
                            const halfx8 va = codes_to_f16(u4w(vd[grp], half * 2 + ks), cc);
                            dpv[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, wb, dpv[mb], 0, 0, 0);
                        }
                    }
                }
                lds_fence();
            }
        };
        // Two tiles per wave per iteration: both tiles' loads are issued
        // before either is used. The next pair's loads are issued once both
        // steps are done (unconditionally within the pair, so that the waits
        // for tile v never cover tile v + 4's loads).
        for (int v = v0 + wave; v < v1; v += 2 * kWaves) {
            step(v, ta);
            if (v + kWaves < v1) step(v + kWaves, tb);
            if (v + 2 * kWaves < v1) {
                __builtin_amdgcn_sched_barrier(0);
                load_tile(v + 2 * kWaves, ta);
                __builtin_amdgcn_sched_barrier(0);
                load_tile(v + 3 * kWaves < v1 ? v + 3 * kWaves : v + 2 * kWaves, tb);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
    // QK of a 16-bit tile on the matrix cores: D[h][t] = sum_c q_h[c] k_t[c]
    // with v_mfma_f32_16x16x32 on the 16-bit inputs (exact products, fp32
    // accumulation): A = the query, lane l holding head l % 16 (zero rows for
    // heads >= G) and channels 32 ks + 8 (l / 16) .. + 7 of K-step ks, loaded
    // once; B = the tile's K rows, lane l holding those channels of token
    // 16 nb + l % 16 (one 16-byte load each). D of token block nb: lane l
    // (l < 16) holds heads 0..3 of token 16 nb + l; three lane swaps per head
    // gather the four blocks into the lane = token layout of the softmax.
    intx4 qa16[4];
    {
        const int hrow = lane & 15;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            qa16[ks] = hrow < G ? *reinterpret_cast<const intx4*>(qn + hrow * 64 + 16 * ks + 4 * (lane >> 4))
                                : intx4{0, 0, 0, 0};
    }
    uint4 kk16[16], vv16[16];
    for (int v = v0 + wave; v < v1; v += kWaves) {
        float lg[G];
        int count, tile;
        {
            // ----------------------------- token phase, 16-bit tile
            const bool keep = v < nqt + nkt;
            tile = keep ? v - nqt : v - nqt - nkt;
            count = keep ? n_keep : nring;
            const bool valid = tile * kTile + lane < count;
            const uint8_t* kt = keep ? reinterpret_cast<const uint8_t*>(p.c.k_keep) + ((size_t)bg * kt_cap + tile) * kTileBytes16
                                     : reinterpret_cast<const uint8_t*>(p.c.k_win) + ((size_t)bg * wt_cap + tile) * kTileBytes16;
            const uint8_t* vt = keep ? reinterpret_cast<const uint8_t*>(p.c.v_keep) + ((size_t)bg * kt_cap + tile) * kTileBytes16
                                     : reinterpret_cast<const uint8_t*>(p.c.v_win) + ((size_t)bg * wt_cap + tile) * kTileBytes16;
            // every K and V load of the tile is issued up front: one memory
            // latency per tile (V does not depend on the scores)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    kk16[4 * nb + ks] =
                        *reinterpret_cast<const uint4*>(kt + k16_off(16 * nb + (lane & 15), 4 * ks + (lane >> 4)));
#pragma unroll
            for (int i = 0; i < 16; ++i) vv16[i] = *reinterpret_cast<const uint4*>(vt + i * 1024 + lane * 16);
            floatx4 d[4];
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                d[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if constexpr (F16)
                        d[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(halfx8, qa16[ks]),
                                                                      __builtin_bit_cast(halfx8, kk16[4 * nb + ks]),
                                                                      d[nb], 0, 0, 0);
                    else
                        d[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa16[ks]),
                                                                       __builtin_bit_cast(bf16x8, kk16[4 * nb + ks]),
                                                                       d[nb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                // rows 1 of blocks 0 / 2 <- rows 0 of blocks 1 / 3, then the
                // upper half of the first <- the lower half of the second
                const auto s01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(d[0][h]), __float_as_uint(d[1][h]), false, false);
                const auto s23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(d[2][h]), __float_as_uint(d[3][h]), false, false);
                const auto s = __builtin_amdgcn_permlane32_swap(s01[0], s23[0], false, false);
                lg[h] = valid ? __uint_as_float(s[0]) * p.scale2 : -INFINITY;
            }
        }

        // ----------------------------- online softmax (wave-uniform update)
        float pr_h[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (__any(lg[h] > m[h] + kLazy)) {
                const float tmax = wave_max_fast(lg[h]);
                const float alpha = __builtin_amdgcn_exp2f(m[h] - tmax);
                m[h] = tmax;
                l[h] *= alpha;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    zacc[h][i] *= alpha;
                    wsb[h][i] *= alpha;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[h][i] *= alpha;
#pragma unroll
                for (int mb = 0; mb < 8; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dpv[mb][r] = (lane & 15) == h ? dpv[mb][r] * alpha : dpv[mb][r];
            }
            pr_h[h] = __builtin_amdgcn_exp2f(lg[h] - m[h]);
            l[h] += pr_h[h];
        }

        {
            if (E <= -1000) E = 0;  // no INT4 tile yet: fix the accumulator unit
            const float k16 = __builtin_ldexpf(1.0f, -E);
#pragma unroll
            for (int h = 0; h < G; ++h) p_w[lane * G + h] = pr_h[h] * k16;
            lds_fence();
            // ----------------------------- channel phase, 16-bit V
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int slot = 16 * u + i;
                const uint4 vv = vv16[i];
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

    }
    // ----------------------------- wave epilogue
    // o = 2^E * (D - sum(bias * w)) + sum(p z) on INT4 tiles, 2^E * acc on
    // 16-bit tiles.
    const float unit = E <= -1000 ? 0.f : __builtin_ldexpf(1.0f, E);
    if constexpr (MODE == 0) {
        // The 9G per-lane sums (l[h], zacc[h][grp], wsb[h][grp]) over the
        // wave: two swaps leave 16 partials of each in lanes 0..15, which go
        // through this wave's QK transpose area (free after the last tile);
        // lane k < 9G then adds the 16 partials of sum k (fewer cross-lane
        // steps than a 64-lane reduction per sum).
        constexpr int NV = 9 * G, RS = 17;
        static_assert(NV * RS + NV <= 4 * NHB * 64 * 4, "reduction area exceeds the wave's QK transpose area");
        float* red = reinterpret_cast<float*>(y_w);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float vl = rows_sum4(l[h]);
            if (lane < 16) red[h * RS + lane] = vl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float vz = rows_sum4(zacc[h][i]), vw = rows_sum4(wsb[h][i]);
                if (lane < 16) {
                    red[(G + 4 * h + i) * RS + lane] = vz;
                    red[(5 * G + 4 * h + i) * RS + lane] = vw;
                }
            }
        }
        lds_fence();
        if (lane < NV) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) s += red[lane * RS + j];
            red[NV * RS + lane] = s;
        }
        lds_fence();
        const float* sums = red + NV * RS;
#pragma unroll
        for (int h = 0; h < G; ++h) l[h] = sums[h];
        // the lane's head hl reads its group sums straight from LDS (a
        // lane-indexed pick from registers is promoted to a per-thread LDS
        // array, whose address needs the workgroup size from the dispatch
        // packet: a long scalar-load stall per wave)
        const int hl = lane & 15;
        if (hl < G) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const float z = sums[G + 4 * hl + grp], wb = sums[5 * G + 4 * hl + grp];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int mb = 2 * grp + half;
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        lds_o[wave][hl][16 * mb + 4 * (lane >> 4) + r] = fmaf(unit, dpv[mb][r] - wb, z);
                }
            }
        }
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) l[h] = wave_sum_fast(l[h]);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[h][i] = rows_sum4(acc[h][i]);
        if (lane < 16) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int i = 0; i < 8; ++i) lds_o[wave][h][8 * lane + i] = unit * acc[h][i];
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
    const size_t pbase = ((size_t)bg * p.nsplit + split_out) * p.G + half * G;
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

// One launch covers both kinds of split: workgroups x < nsq take INT4 tiles,
// the rest take 16-bit tiles, so the two kinds run side by side.
template <int G, bool F16, bool NT = true>
__global__ __launch_bounds__(256, G <= 4 ? 2 : 1) void k_decode_split(DecodeParams p) {
    __shared__ SplitSmem<G> sm;
    int x = blockIdx.x, half = 0;
    if (p.halves == 2) {
        // the two head halves of split x are 8 workgroups apart in dispatch
        // order, so they land on the same XCD and share its L2
        half = (x >> 3) & 1;
        x = (x >> 4) * 8 + (x & 7);
        if (x >= p.nsplit) return;
    }
    if (x < p.nsq)
        split_body<G, F16, 0, NT>(p, sm, x, half);
    else
        split_body<G, F16, 1, NT>(p, sm, x - p.nsq, half);
}

// Cross-split merge: out[b][h] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s, over the partials of every split of the (b, g).
__global__ __launch_bounds__(128) void k_decode_reduce(const hq_cache c, const float* __restrict__ part_m,
                                                       const float* __restrict__ part_l,
                                                       const float* __restrict__ part_o, int nsplit, int G, int Hq,
                                                       void* out, int out_dt) {
    // One thread per output channel. The partials are merged in chunks of R
    // splits whose loads are all issued before any of them is used; a chunk
    // whose maximum exceeds the running one rescales the running sums (every
    // split writes a partial; empty ones have m = -inf and are skipped).
    constexpr int R = 16;
    const int gh = blockIdx.x, b = blockIdx.y;
    const int g = gh / G, h = gh % G, d = threadIdx.x;
    const int bg = b * c.Hkv + g;
    const size_t base = (size_t)bg * nsplit * G + h;
    const float* po = part_o + base * kD + d;
    float run_m = -INFINITY, L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += R) {
        float mv[R], lv[R], ov[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int i = min(s0 + j, nsplit - 1);
            mv[j] = part_m[base + (size_t)i * G];
            lv[j] = part_l[base + (size_t)i * G];
            ov[j] = po[(size_t)i * G * kD];
        }
        float mc = -INFINITY;
#pragma unroll
        for (int j = 0; j < R; ++j)
            if (s0 + j < nsplit) mc = fmaxf(mc, mv[j]);
        const float nm = fmaxf(run_m, mc);
        if (nm == -INFINITY) continue;
        const float sc = run_m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(run_m - nm);
        L *= sc;
        O *= sc;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (s0 + j < nsplit && mv[j] != -INFINITY) {
                const float f = __builtin_amdgcn_exp2f(mv[j] - nm);
                L = fmaf(f, lv[j], L);
                O = fmaf(f, ov[j], O);
            }
        }
        run_m = nm;
    }
    store_out(out, out_dt, ((size_t)b * Hq + g * G + h) * kD + d, O / L);
}

struct WsLayout {
    size_t pm, pl, po, total;
};
inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
WsLayout ws_layout(const hq_cache& c, int32_t Hq, int32_t nsplit) {
    const size_t BG = (size_t)c.B * c.Hkv;
    const int G = Hq / c.Hkv;
    WsLayout w;
    w.pm = 0;
    w.pl = w.pm + al(BG * nsplit * G * 4);
    w.po = w.pl + al(BG * nsplit * G * 4);
    w.total = w.po + al(BG * nsplit * G * kD * 4);
    return w;
}

template <int G, bool F16>
void launch_split(const DecodeParams& p, int Hkv, int B, hipStream_t s) {
    // INT4 splits (x < nsq) come first in dispatch order; the 16-bit ones
    // fill in as slots free up.
    // the query goes in as a separate read-only, non-aliased argument so that
    // its wave-uniform reads become scalar loads
    const int gx = p.halves == 2 ? (p.nsplit + 7) / 8 * 16 : p.nsplit;
    // the two-halves launch reads with the default cache policy: the L2 then
    // keeps the lines for the sibling workgroup (measured faster than the
    // non-temporal hint there)
    if (p.halves == 2)
        k_decode_split<G, F16, false><<<dim3(gx, Hkv, B), 256, 0, s>>>(p);
    else
        k_decode_split<G, F16><<<dim3(gx, Hkv, B), 256, 0, s>>>(p);
}


}  // namespace

int32_t decode_nsq(const hq_cache& c, int32_t tps) { return (c.cap_q / kTile + tps - 1) / tps; }
int32_t decode_nsplit(const hq_cache& c, int32_t tps) {
    return decode_nsq(c, tps) + (c.cap_keep / kTile + c.window / kTile + kTps16 - 1) / kTps16;
}

// The fixed scratch of hq_decode_attn_noalloc (the split partials), one copy
// per device for the life of the process. Host code never uses this name as
// an address: each device's copy is looked up once with hipGetSymbolAddress
// and that pointer is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** out) {
    static std::atomic<void*> cached[64];  // per device, zero-initialised
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = cached[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        cached[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return hipSuccess;
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
    p.qw = static_cast<const uint32_t*>(q);
    p.Hq = d.Hq;
    p.part_m = reinterpret_cast<float*>(ws + w.pm);
    p.part_l = reinterpret_cast<float*>(ws + w.pl);
    p.part_o = reinterpret_cast<float*>(ws + w.po);
    p.nsplit = d.nsplit;
    p.nsq = decode_nsq(c, d.tiles_per_split);
    p.G = d.G;
    p.halves = d.G == 8 ? 2 : 1;  // eight heads run as two workgroups of four
    p.scale2 = d.sm_scale_log2;
    const bool f16 = c.dt == HQ_F16;
    switch (d.G * 2 + (f16 ? 1 : 0)) {
        case 2: launch_split<1, false>(p, c.Hkv, c.B, s); break;
        case 3: launch_split<1, true>(p, c.Hkv, c.B, s); break;
        case 4: launch_split<2, false>(p, c.Hkv, c.B, s); break;
        case 5: launch_split<2, true>(p, c.Hkv, c.B, s); break;
        case 8: launch_split<4, false>(p, c.Hkv, c.B, s); break;
        case 9: launch_split<4, true>(p, c.Hkv, c.B, s); break;
        case 16: launch_split<4, false>(p, c.Hkv, c.B, s); break;
        case 17: launch_split<4, true>(p, c.Hkv, c.B, s); break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_decode_reduce<<<dim3(c.Hkv * d.G, c.B), 128, 0, s>>>(c, p.part_m, p.part_l, p.part_o, d.nsplit, d.G, d.Hq,
                                                          out, (int)out_dt);
    return hipGetLastError();
}

}  // namespace hq
