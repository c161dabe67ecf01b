// hq_probe_select: vertical-line probe and top-k column selection (gfx950).
//
// HyQuant pages: "HyQuant: Hybrid-Precision Quantization for LLM
// Attention", TL;DR and "What problem it solves" (a small number of key
// columns are attended to by almost every query row; a lightweight pattern
// signal finds them without calibration), "Gaps" (the probe works on the
// attention map, the tensor the method otherwise avoids forming); "How HyQuant
// uses hybrid-precision attention to cut decode compute", "Why preserve
// selected positions?" (keep the top 5% high-score positions) and "Memory and
// runtime costs" (finding the columns costs a few percent of the runtime).
//
// Column score c[j] = sum over the G query heads and the last R probe rows of
// the row-normalised causal softmax. Only the probe rows' slice of the map
// (G R rows x T keys per (b, g); at 32K and G R = 256, 0.8% of the T x T map)
// is ever formed, and each of its logits is computed once: pass 1 computes
// the logits, each term 2^(z - m) against an integer reference m per (row,
// key chunk), the rows' normalisers per chunk, and stores the terms (fp32)
// in the workspace; a combine kernel merges the chunks into (M, 1/L) per
// row; pass 2 streams the stored terms and adds them per column with the
// weights 2^(m - M) / L in fp64.
//
// Logits, exactly, on the int8 matrix cores. Every 16-bit value x of a set
// (a 32-row tile of probe queries, or one key) becomes the integer
// X = rint(x * 2^sh), |X| <= 2^30, with one power-of-two shift sh per set,
// and X is split into four signed base-256 digits X = sum_a d_a 256^(3 - a)
// (d_0 in [-65, 65], the others in [-128, 127]). A dot product of a query
// row and a key is then 2^(48 - shq - shk) * sum_d 256^-d A_d with
// A_d = sum_{a + b = d} sum_c dq_a[c] dk_b[c], every A_d an exact int32 sum
// from v_mfma_i32_32x32x32_i8. The 13 digit pairs with a + b <= 4 are
// computed; the rest of the product is bounded, not dropped silently: per
// (query tile, key) the kernel evaluates, from the digits and the rounding
// residuals x - X 2^-sh themselves, a bound on the logit error (rounding
// residuals times the other operand's magnitude, plus the three omitted
// pairs bounded through the query digit planes' l1 norms and the key's
// shift). On the workloads this bound is ~1e-8 in log2 units; a 32-key tile
// where any key's bound exceeds kLogitBudget has its logits recomputed from
// the 16-bit inputs in fp64 (exact products, fp64 sums), so every logit
// carries at most the budget's error. Each term 2^(z - m) is split exactly in fp64 into 2^n 2^f
// (n = rint(z - m), |f| <= 1/2); f is rounded to fp32 (error <= 2^-26) and
// 2^f taken by the hardware base-2 exponential (v_exp_f32, relative error at
// most 1.5 2^-24 on [-1/2, 1/2]: checked over every fp32 input there with
// hq_diag_exp2_error, which finds 1.395 2^-24), then scaled by 2^n exactly; that fp32 value is
// both the stored term and what the row's normaliser adds, in fp64. Every
// normaliser and column sum accumulates in fp64 relative to integer
// references, so rescaling by a power of two is exact. Scores are rounded
// once to fp32. Resulting bound on each returned score, for the softmax with
// the fp32 scale the caller passes: a term is off by at most
// d = ln2 (kLogitBudget + 2^-26) + 1.5 2^-24 relative, a row's normaliser by at
// most d too (a sum of such terms), so a score (a sum of term / normaliser)
// by at most 2 d + 2^-24 < 3.3e-7, and two columns can change order only
// where their exact scores differ by less than 6.6e-7 relative. (The fp64
// roundings of the logit, of z - m and of the split, each below 2^-33 in log2
// units for logits below 2^19 in magnitude, are far below these terms.)
//
// Top-k: one workgroup per (b, g); 4-pass 8-bit radix select on the fp32 bit
// patterns (scores are >= 0, so bit order = value order) with LDS histograms
// and a wave-parallel scan over the bins, then an index-ordered compaction
// (each thread a contiguous run of candidates, two block scans) that takes
// all scores above the threshold and the lowest-index ties.
#include "hq_internal.h"

namespace hq {
namespace {

typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kRT = 32;            // probe rows per row tile (one wave)
constexpr int kKT = 32;            // keys per key tile
constexpr int kTilesPerWg = 8;     // row tiles (waves) per workgroup at most
constexpr int kPlanes = 4;         // base-256 digits per value
constexpr int kDS = kD + 16;       // LDS bytes per key in a digit plane (pad: no bank conflicts)
constexpr int kColCols = 1024;     // columns per pass-2 workgroup (256 threads x 4)
constexpr int kTopkLds = 34816;    // candidates the top-k stages in LDS (136 KiB + padding)
constexpr int kHistCopies = 8;     // copies of the top-k's radix histogram (8 KiB of LDS)
constexpr int kUnset = -(1 << 20);  // placeholder reference of a row with no valid logit yet in the chunk:
                                     // y = z + 2^20 keeps z to 2^-33 until the row's first valid logit moves it
constexpr int kMoveGap = 100;      // a row's reference moves when a logit exceeds it by more than this (log2
                                   // units), so every stored term 2^(z - ref) is at most 2^100 (fp32 range)
constexpr double kLogitBudget = 0.5e-7;  // largest logit error accepted from the digit path (log2 units)

struct ProbeParams {
    const uint16_t* q;     // [B][Hq][R][D]
    const uint16_t* k;     // [B][Hkv][Tmax][D]
    const int32_t* seq_lens;
    double2* part;         // [B][Hkv][nchunk][NRp] (m, l) per key chunk: l = sum 2^(z - m), m an integer
    double2* rownorm;      // [B][Hkv][NRp] (M, 1/L) per row: p = 2^(z - M) / L
    float* emap;           // [B][Hkv][NRp][Tp] the probe rows' terms 2^(z - m) of pass 1, m the row's
                           // reference in the key's chunk (0 outside the causal map)
    float* col_scores;     // [B][Hkv][Tmax]
    int32_t B, Hq, Hkv, Tmax, Tp, R, G, NR, NRp, ngroups, nchunk, chunk;
    double sc2;            // sm_scale * log2(e)
};

// Row `row` of the (b, g) probe rows: head g*G + row / R, probe row row % R,
// at position T - R + row % R (negative positions are not rows of the map).
__device__ inline const uint16_t* qrow(const ProbeParams& p, int b, int g, int row) {
    const int h = row / p.R, r = row % p.R;
    return p.q + (((size_t)b * p.Hq + g * p.G + h) * p.R + r) * kD;
}

template <bool F16>
__device__ inline void unpack8(const uint4& u, float* x) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = h16_to_f32<F16>(w[j] & 0xFFFFu);
        x[2 * j + 1] = h16_to_f32<F16>(w[j] >> 16);
    }
}

// Shift of a set whose largest magnitude is mx: |x| * 2^sh < 2^30.
__device__ inline int set_shift(float mx) { return mx > 0.f ? 30 - __builtin_amdgcn_frexp_expf(mx) : 0; }

// x -> X = rint(x 2^sh) (exact int32) and the residual |x 2^sh - X| (<= 1/2).
__device__ inline int to_fixed(float x, int sh, float& res) {
    const float t = __builtin_ldexpf(x, sh);  // exact: a power-of-two scaling
    const float tr = __builtin_rintf(t);
    res = fabsf(t - tr);                       // exact
    return (int)tr;
}
// The four balanced base-256 digits of X (|X| <= 2^30) are the bytes of
// (X + 0x808080) ^ 0x808080: byte 3 = d_0 (top), byte 0 = d_3.
__device__ inline uint32_t digit_bytes(int X) { return (uint32_t)(X + 0x808080) ^ 0x808080u; }
// Byte `by` of four words, packed into one word (element order z0..z3).
__device__ inline uint32_t gather_byte(uint32_t z0, uint32_t z1, uint32_t z2, uint32_t z3, int by) {
    const uint32_t sel = (uint32_t)by | ((uint32_t)(by + 4) << 8) | 0x0C0C0000u;
    const uint32_t lo = __builtin_amdgcn_perm(z1, z0, sel);  // z0[by], z1[by], 0, 0
    const uint32_t hi = __builtin_amdgcn_perm(z3, z2, sel);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}
__device__ inline int sbyte(uint32_t w, int i) { return (int)(int8_t)(w >> (8 * i)); }

// Reductions over 16-lane groups (one key's threads) without LDS traffic:
// DPP moves within rows of 16 lanes.
template <int CTRL>
__device__ inline uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) { return __uint_as_float(dpp_u<CTRL>(__float_as_uint(v))); }
__device__ inline float max16(float v) {
    v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
    return fmaxf(v, dpp_f<0x140>(v));  // row_mirror
}
__device__ inline float sum16(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    return v + dpp_f<0x140>(v);
}
// One term 2^y (fp32): y = n + f split exactly in fp64 (n = rint(y),
// |f| <= 1/2), f rounded to fp32, 2^f by the hardware exponential, then the
// exact power-of-two scaling (0 below the fp32 range, inf above; such terms
// occur only for elements outside the map, whose term is dropped).
__device__ inline float exp2_term(double y) {
    const double n = __builtin_rint(y);
    return __builtin_ldexpf(__builtin_amdgcn_exp2f((float)(y - n)), (int)n);
}

// Per-key data of the key tile in LDS.
struct KeyTile {
    int8_t d[kPlanes][kKT][kDS];  // digit planes, key-major, the MFMA B operand
    int sh[kKT];                   // shift of the key
    float rho[kKT];                // sum over channels of |residual| * 2^-sh (an upper bound, real units)
    float kmax[kKT];               // max |k|
};

// Digit planes 2 and 3 of one wave's query tile (row-major like the key
// planes; the MFMA A operand of the pairs (2, b) and (3, b)).
struct QPlanes {
    int8_t d[2][kRT][kDS];
};

struct __align__(16) ProbeSmem {  // 16-byte rows: the MFMA operands are read as 128-bit LDS loads
    KeyTile kt[2];
    QPlanes q23[kTilesPerWg];
};

// Key tile [key0, key0 + 32) of one (b, g): thread t (of the workgroup's
// 512) moves channels 8 (t % 16) .. + 7 of key key0 + t / 16. The load is
// issued a tile ahead; the conversion to digit planes and statistics writes
// the LDS tile (keys >= key_end are zero).
__device__ inline uint4 load_keys(const uint16_t* kbase, int key0, int key_end) {
    const int t = threadIdx.x, key = key0 + (t >> 4), c0 = (t & 15) * 8;
    return key < key_end ? *reinterpret_cast<const uint4*>(kbase + (size_t)key * kD + c0) : make_uint4(0, 0, 0, 0);
}
template <bool F16>
__device__ inline void store_keys(const uint4& u, KeyTile& kt) {
    const int t = threadIdx.x, kk = t >> 4, c0 = (t & 15) * 8;
    float x[8];
    unpack8<F16>(u, x);
    float mx = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(x[j]));
    mx = max16(mx);  // the 16 threads of a key are one 16-lane row of a wave
    const int sh = set_shift(mx);
    uint32_t z[8];
    float rsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float r;
        z[j] = digit_bytes(to_fixed(x[j], sh, r));
        rsum += r;
    }
#pragma unroll
    for (int a = 0; a < kPlanes; ++a) {
        const int by = 3 - a;
        uint2 w;
        w.x = gather_byte(z[0], z[1], z[2], z[3], by);
        w.y = gather_byte(z[4], z[5], z[6], z[7], by);
        *reinterpret_cast<uint2*>(&kt.d[a][kk][c0]) = w;
    }
    rsum = sum16(rsum);
    if ((t & 15) == 0) {
        kt.sh[kk] = sh;
        kt.rho[kk] = __builtin_ldexpf(rsum * (1.0f + 0x1p-16f), -sh);
        kt.kmax[kk] = mx;
    }
}

// One wave's probe rows (a 32-row tile): digit planes as MFMA A operands
// (lane l holds row l % 32, channels 32 ks + 16 (l / 32) .. + 15 of K-step
// ks), and the tile's statistics.
struct QTile {
    intx4 d[2][4];     // planes 0 and 1 (planes 2 and 3 are in LDS)
    int sh;
    float qmax, rho;   // max |q|; max over rows of sum |residual| (real units)
    int n2, n3;        // max over rows of sum |d_2|, sum |d_3|
};
template <bool F16>
__device__ inline QTile convert_queries(const ProbeParams& p, int b, int g, int T, int rt, QPlanes& q23) {
    const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
    const int row = rt * kRT + m;
    const bool ok = row < p.NR && T - p.R + row % p.R >= 0;
    const uint16_t* src = ok ? qrow(p, b, g, row) : nullptr;
    float x[4][16];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const uint4 u0 = ok ? *reinterpret_cast<const uint4*>(src + 32 * ks + 16 * hf) : make_uint4(0, 0, 0, 0);
        const uint4 u1 = ok ? *reinterpret_cast<const uint4*>(src + 32 * ks + 16 * hf + 8) : make_uint4(0, 0, 0, 0);
        unpack8<F16>(u0, x[ks]);
        unpack8<F16>(u1, x[ks] + 8);
    }
    float mx = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(x[ks][j]));
    mx = wave_max(mx);
    QTile t;
    t.sh = set_shift(mx);
    t.qmax = mx;
    float rsum = 0.f;
    int n2 = 0, n3 = 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        uint32_t z[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            float r;
            z[j] = digit_bytes(to_fixed(x[ks][j], t.sh, r));
            rsum += r;
            n2 += abs(sbyte(z[j], 1));
            n3 += abs(sbyte(z[j], 0));
        }
#pragma unroll
        for (int a = 0; a < kPlanes; ++a) {
            const int by = 3 - a;
            const intx4 w{(int)gather_byte(z[0], z[1], z[2], z[3], by), (int)gather_byte(z[4], z[5], z[6], z[7], by),
                          (int)gather_byte(z[8], z[9], z[10], z[11], by), (int)gather_byte(z[12], z[13], z[14], z[15], by)};
            if (a < 2) t.d[a][ks] = w;
            else *reinterpret_cast<intx4*>(&q23.d[a - 2][lane & 31][32 * ks + 16 * (lane >> 5)]) = w;
        }
    }
    // per row: both halves of the row (lanes l, l ^ 32); then the tile maximum
    rsum += __shfl_xor(rsum, 32);
    n2 += __shfl_xor(n2, 32);
    n3 += __shfl_xor(n3, 32);
    t.rho = __builtin_ldexpf(wave_max(rsum * (1.0f + 0x1p-16f)), -t.sh);
    t.n2 = (int)wave_max((float)n2);
    t.n3 = (int)wave_max((float)n3);
    return t;
}

// Exact digit sums of a 32-row x 32-key tile: D[row][key] with lane l holding
// key l % 32 and rows 8 (i / 4) + 4 (l / 32) + i % 4 in element i. hi =
// 256 A_0 + A_1, mid = 256 A_2 + A_3, lo = A_4 (all within int32).
struct DigitSums {
    intx16 hi, mid, lo;
};
__device__ inline DigitSums tile_digit_sums(const QTile& q, const QPlanes& q23, const KeyTile& kt) {
    const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
    DigitSums s;
    // A_0 first, then hi = 256 A_0 accumulates A_1 (one accumulator fewer
    // live during the main loop; key plane 0 is read twice)
    intx16 hi = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        hi = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[0][ks], *reinterpret_cast<const intx4*>(&kt.d[0][n][32 * ks + 16 * hf]),
                                                  hi, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) hi[i] <<= 8;
    intx16 a2 = {}, a3 = {}, a4 = {};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        intx4 kb[kPlanes];
#pragma unroll
        for (int a = 0; a < kPlanes; ++a) kb[a] = *reinterpret_cast<const intx4*>(&kt.d[a][n][32 * ks + 16 * hf]);
        const intx4 q2 = *reinterpret_cast<const intx4*>(&q23.d[0][n][32 * ks + 16 * hf]);
        hi = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[0][ks], kb[1], hi, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[0][ks], kb[2], a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[0][ks], kb[3], a3, 0, 0, 0);
        hi = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[1][ks], kb[0], hi, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[1][ks], kb[1], a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[1][ks], kb[2], a3, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q.d[1][ks], kb[3], a4, 0, 0, 0);
        a2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q2, kb[0], a2, 0, 0, 0);
        a3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q2, kb[1], a3, 0, 0, 0);
        a4 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q2, kb[2], a4, 0, 0, 0);
    }
    // the pairs (3, 0) and (3, 1) only where the tile's query digit plane 3 is
    // not all zero (a wave-uniform test; a zero plane contributes exactly 0,
    // and the int32 sums are exact in any order). Plane 3 holds the bits of
    // values below 2^-22 of the tile's largest magnitude, so most query
    // tiles skip these 8 MFMAs.
    if (__builtin_amdgcn_readfirstlane(q.n3) != 0) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const intx4 q3 = *reinterpret_cast<const intx4*>(&q23.d[1][n][32 * ks + 16 * hf]);
            a3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q3, *reinterpret_cast<const intx4*>(&kt.d[0][n][32 * ks + 16 * hf]),
                                                      a3, 0, 0, 0);
            a4 = __builtin_amdgcn_mfma_i32_32x32x32_i8(q3, *reinterpret_cast<const intx4*>(&kt.d[1][n][32 * ks + 16 * hf]),
                                                      a4, 0, 0, 0);
        }
    }
    s.hi = hi;
#pragma unroll
    for (int i = 0; i < 16; ++i) s.mid[i] = (a2[i] << 8) + a3[i];
    s.lo = a4;
    return s;
}

// Bound (log2 units) on the error of the digit path's logits of this lane's
// key (lane % 32) against every row of the tile: rounding residuals times the
// other operand, and the omitted pairs (2,3), (3,2), (3,3) through the query
// digit planes' l1 norms, weighted by the key's own shift.
__device__ inline double key_error_bound(const QTile& q, const KeyTile& kt, double asc2) {
    const int n = threadIdx.x & 31;
    const float kmax = kt.kmax[n], krho = kt.rho[n];
    const double res = (double)q.rho * kmax + ((double)q.qmax + q.rho) * krho;
    // |D_23| <= n2 * 128, |D_32| <= n3 * 128, |D_33| <= n3 * 128 (|d| <= 128),
    // weights 2^(8 - sh), 2^(8 - sh), 2^(-sh)
    const double om = __builtin_ldexp(128.0 * ((double)q.n2 + (double)q.n3 * (1.0 + 0x1p-8)), 8 - q.sh - kt.sh[n]);
    return (res + om) * asc2 * (1.0 + 0x1p-20);
}

// One logit from the 16-bit inputs: exact products, fp64 sum (the fallback;
// rare, so a few registers and no unrolling keep the common path's occupancy).
template <bool F16>
__device__ inline double exact_logit(const ProbeParams& p, int b, int g, const uint16_t* kbase, int key, int row) {
    double acc = 0.0;
    const uint32_t* qr = reinterpret_cast<const uint32_t*>(qrow(p, b, g, row));
    const uint32_t* kr = reinterpret_cast<const uint32_t*>(kbase + (size_t)key * kD);
#pragma unroll 1
    for (int c = 0; c < kD / 2; ++c) {
        const uint32_t wq = qr[c], wk = kr[c];
        acc = __builtin_fma((double)h16_to_f32<F16>(wq & 0xFFFFu), (double)h16_to_f32<F16>(wk & 0xFFFFu), acc);
        acc = __builtin_fma((double)h16_to_f32<F16>(wq >> 16), (double)h16_to_f32<F16>(wk >> 16), acc);
    }
    return acc * p.sc2;
}

// The probe row held in element i of this lane (MFMA D layout).
__device__ inline int elem_row(int rt, int i) { return rt * kRT + 8 * (i >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (i & 3); }

// The tile's logits in log2 units (z = q . k * sm_scale * log2 e) less a
// per-element integer offset (the row's reference), for the 16 elements of
// this lane: from the digit sums (the offset enters the inner fma, two
// roundings in all), or, when the tile's error bound
// exceeds the budget (a wave-uniform decision, so the common path is one
// straight run over the 16 independent elements), recomputed in fp64 from
// the 16-bit inputs (exact products, fp64 sums). Elements outside the map
// (key >= key_end, row >= NR) get 0.
template <bool F16>
__device__ inline void tile_logits(const ProbeParams& p, const QTile& q, const QPlanes& q23, const KeyTile& kt,
                                   int b, int g, const uint16_t* kbase, int key, int key_end, int rt,
                                   const int (&off)[16], double (&z)[16]) {
    const DigitSums s = tile_digit_sums(q, q23, kt);
    // the whole tile takes the fallback when any of its keys' bounds exceeds
    // the budget (wave-uniform)
    const bool fallback = __builtin_amdgcn_ballot_w64(!(key_error_bound(q, kt, fabs(p.sc2)) <= kLogitBudget)) != 0;
    if (!fallback) {
        // z - off = F (65536 hi + mid) 256 + (F lo - off), F = 2^(16 - shq - shk) sm_scale log2 e
        const double F = __builtin_ldexp(p.sc2, 16 - q.sh - kt.sh[threadIdx.x & 31]);
        const double F256 = 256.0 * F;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const double u = __builtin_fma((double)s.hi[i], 65536.0, (double)s.mid[i]);  // exact
            z[i] = __builtin_fma(u, F256, __builtin_fma((double)s.lo[i], F, -(double)off[i]));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = elem_row(rt, i);
            z[i] = (key < key_end && row < p.NR) ? exact_logit<F16>(p, b, g, kbase, key, row) - (double)off[i] : 0.0;
        }
    }
}

// Whether element i's probe row is a row of the map (row < NR, position
// >= 0) and the key (< key_end) is at or before its position. Rows' positions
// are T - R + row % R, so keys below T - R pass for every real row.
__device__ inline bool elem_valid(const ProbeParams& p, int T, int row, int key, int key_end) {
    if (key >= key_end || row >= p.NR) return false;
    return key <= T - p.R + row % p.R;
}
// Bit i: element i's row is a row of the map (row < NR, position >= 0).
__device__ inline uint32_t row_mask(const ProbeParams& p, int T, int rt) {
    uint32_t mk = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = elem_row(rt, i);
        mk |= (row < p.NR && T - p.R + row % p.R >= 0) ? 1u << i : 0u;
    }
    return mk;
}
// Mask of the elements of a key tile [key0, key0 + 32): keys below T - R are
// before every row's position, so only the last tiles need the causal test.
__device__ inline uint32_t tile_mask(const ProbeParams& p, int T, int rt, uint32_t rowmk, int key0, int key_end) {
    const int key = key0 + (threadIdx.x & 31);
    if (key >= key_end) return 0u;
    if (key0 + kKT - 1 <= T - p.R) return rowmk;
    uint32_t mk = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) mk |= elem_valid(p, T, elem_row(rt, i), key, key_end) ? 1u << i : 0u;
    return mk;
}

// Whether every element of the wave's tile is in the map (wave-uniform): then
// the element loops need no mask.
__device__ inline bool tile_full(uint32_t mk) { return __builtin_amdgcn_ballot_w64(mk != 0xFFFFu) == 0; }

// One stored term of pass 1, streamed past the caches.
__device__ inline void store_term(const __amdgpu_buffer_rsrc_t& r, int voff, int soff, float e) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(e), r, voff, soff, kLoadNT);
}

// Pass 1: per (key chunk, row group, g, b): for every probe row of the group,
// (m, l) over the chunk's keys with m an integer reference and
// l = sum 2^(z - m), and every term 2^(z - m) stored (fp32) for pass 2. One
// wave per 32-row tile; the key tiles are converted to digits once per
// workgroup into LDS (double-buffered) and read by every wave. A row's
// reference is the same in the 32 lanes of a half-wave (the lanes are the
// tile's keys): it is set from the first tile with a valid logit of the row
// and moves up only when a logit exceeds it by more than kMoveGap; a move
// rescales the lane's sum and the terms the lane already stored for the row
// by the same power of two, exactly (down to fp32 underflow).
template <bool F16>
__global__ __launch_bounds__(512) void k_probe_rowstats(ProbeParams p) {
    __shared__ ProbeSmem sm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int chunk = blockIdx.x, grp = blockIdx.y % p.ngroups, g = blockIdx.y / p.ngroups, b = blockIdx.z;
    const int T = p.seq_lens[b];
    const int bg = b * p.Hkv + g;
    const int rt = grp * kTilesPerWg + wave;
    const int key_lo = chunk * p.chunk;
    double2* part = p.part + ((size_t)bg * p.nchunk + chunk) * p.NRp;
    const bool active = rt * kRT < p.NRp;  // wave-uniform: the last group may have fewer tiles
    if (key_lo >= T) {  // no key of this chunk exists: empty statistics
        if (lane < 32 && active) part[rt * kRT + lane] = make_double2(-INFINITY, 0.0);
        return;
    }
    const int key_hi = min(key_lo + p.chunk, T);
    const int ntile = (key_hi - key_lo + kKT - 1) / kKT;
    const uint16_t* kbase = p.k + (size_t)bg * p.Tmax * kD;
    const QTile q = convert_queries<F16>(p, b, g, T, rt, sm.q23[wave]);
    const uint32_t rowmk = row_mask(p, T, rt);
    // this lane's stored terms: element i is row rt*32 + 8(i/4) + 4(lane/32) + i%4,
    // key key0 + lane % 32; a buffer resource over the tile's rows from key_lo
    // (32-bit offsets: at most 32 rows x Tp keys)
    const int hoff = 4 * (lane >> 5);
    const __amdgpu_buffer_rsrc_t emr = __builtin_amdgcn_make_buffer_rsrc(
        p.emap + ((size_t)bg * p.NRp + rt * kRT) * p.Tp + key_lo, (short)0, kRT * p.Tp * 4 - key_lo * 4, 0x00020000);
    const int evoff = ((lane & 31) + hoff * p.Tp) * 4;
    int m[16];  // integer references, uniform over the half-wave (kUnset: none yet)
    uint32_t unset = 0xFFFFu;  // bit i: element i's row has no reference yet (uniform over the half-wave)
    double l[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m[i] = kUnset;
        l[i] = 0.0;
    }

    store_keys<F16>(load_keys(kbase, key_lo, key_hi), sm.kt[0]);
    __syncthreads();
    for (int t = 0; t < ntile; ++t) {
        const int cur = t & 1;
        const int key0 = key_lo + kKT * t;
        const uint4 nxt = load_keys(kbase, key0 + kKT, t + 1 < ntile ? key_hi : 0);  // next tile, in flight
        if (active) {
            const int key = key0 + (lane & 31);
            double z[16];
            // z: y = z - m, the exponent of the term against the row's reference
            // (m = kUnset for a row without one yet: y = z + 2^20)
            tile_logits<F16>(p, q, sm.q23[wave], sm.kt[cur], b, g, kbase, key, key_hi, rt, m, z);
            const uint32_t mk = tile_mask(p, T, rt, rowmk, key0, key_hi);
            const bool full = tile_full(mk);
            // a row without a reference moves at its first valid logit
            bool move = (mk & unset) != 0u;
            if (full) {  // wave-uniform: every element is in the map
#pragma unroll
                for (int i = 0; i < 16; ++i) move |= z[i] > (double)kMoveGap;
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) move |= ((mk >> i) & 1u) && z[i] > (double)kMoveGap;
            }
            if (__builtin_amdgcn_ballot_w64(move) != 0) {
                // rare (once per row and chunk, at its first valid logits):
                // the half-wave's largest valid y of each element's row
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    double v = ((mk >> i) & 1u) ? z[i] : -INFINITY;
#pragma unroll
                    for (int o = 1; o < 32; o <<= 1) v = fmax(v, __shfl_xor(v, o));
                    // the same decision in all 32 lanes of the half (same rows, same unset bits)
                    if (v > (double)kMoveGap || (((unset >> i) & 1u) && v != -INFINITY)) {
                        const int mn = (int)__builtin_ceil(fmax(fmin(v + (double)m[i], 2.0e9), -2.0e9));
                        const int sh = m[i] - mn;
                        if (l[i] != 0.0) {  // this lane has stored nonzero terms of the row: rescale them
                            l[i] = __builtin_ldexp(l[i], sh);
                            const int so = (8 * (i >> 2) + (i & 3)) * p.Tp * 4;
                            for (int u = 0; u < t; ++u) {
                                const float x = __uint_as_float(
                                    __builtin_amdgcn_raw_buffer_load_b32(emr, evoff, so + kKT * u * 4, 0));
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(__builtin_ldexpf(x, sh)), emr,
                                                                      evoff, so + kKT * u * 4, 0);
                            }
                        }
                        z[i] += (double)sh;  // exact: an integer shift of a value below 2^21
                        m[i] = mn;
                        unset &= ~(1u << i);
                    }
                }
            }
            // straight-line code over the 16 independent elements in both
            // forms (a masked element's exponential is computed, then dropped)
            if (full) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = exp2_term(z[i]);
                    l[i] += (double)e;
                    store_term(emr, evoff, ((8 * (i >> 2) + (i & 3)) * p.Tp + key0 - key_lo) * 4, e);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = exp2_term(z[i]);
                    const float ev = ((mk >> i) & 1u) ? e : 0.f;
                    l[i] += (double)ev;
                    store_term(emr, evoff, ((8 * (i >> 2) + (i & 3)) * p.Tp + key0 - key_lo) * 4, ev);
                }
            }
        }
        if (t + 1 < ntile) store_keys<F16>(nxt, sm.kt[cur ^ 1]);
        __syncthreads();
    }
    if (!active) return;
    // the 32 lanes of each half hold the same rows (different keys) with the
    // same references: their sums add
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) l[i] += __shfl_xor(l[i], o);
    }
    if ((lane & 31) == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            part[elem_row(rt, i)] = make_double2(l[i] > 0.0 ? (double)m[i] : -INFINITY, l[i]);
    }
}

// Merge the chunk statistics of every probe row: M = the largest chunk
// reference, L = sum l 2^(m - M); stores (M, 1/L). One pass over the chunks
// in order with a running maximum: every rescale is by a power of two, so L
// is the same exact-rescale sum in any order of maxima; the loads of 8
// chunks are issued before they are used.
__global__ __launch_bounds__(256) void k_probe_rowfinal(ProbeParams p) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int bg = b * p.Hkv + g;
    const int T = p.seq_lens[b];
    const int nch = (T + p.chunk - 1) / p.chunk;
    for (int row = threadIdx.x; row < p.NRp; row += 256) {
        const double2* pc = p.part + (size_t)bg * p.nchunk * p.NRp + row;
        double M = -INFINITY, L = 0.0;
        for (int c0 = 0; c0 < nch; c0 += 8) {
            double2 v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = c0 + j < nch ? pc[(size_t)(c0 + j) * p.NRp] : make_double2(-INFINITY, 0.0);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (v[j].x == -INFINITY) continue;
                if (v[j].x > M) {
                    L = M == -INFINITY ? 0.0 : __builtin_ldexp(L, (int)fmax(M - v[j].x, -2000.0));
                    M = v[j].x;
                }
                L += __builtin_ldexp(v[j].y, (int)fmax(v[j].x - M, -2000.0));
            }
        }
        p.rownorm[(size_t)bg * p.NRp + row] = L > 0.0 ? make_double2(M, 1.0 / L) : make_double2(-INFINITY, 0.0);
    }
}

// Pass 2: per (1,024-column block, g, b): c[j] = sum over the probe rows r of
// E[r][j] * w[r][chunk(j)], E the terms pass 1 stored and
// w = 2^(m_chunk - M) / L the row's weight for that chunk (fp64). Thread t
// takes columns j0 + 4t .. + 3 and adds the rows in order, in fp64.
__global__ __launch_bounds__(256) void k_probe_colsum(ProbeParams p) {
    __shared__ double wt[kColCols / 256][2 * kTilesPerWg * kRT];  // [chunk in the block][row], NR <= 512
    const int g = blockIdx.y, b = blockIdx.z;
    const int bg = b * p.Hkv + g;
    const int T = p.seq_lens[b];
    const int j0 = blockIdx.x * kColCols;
    const int c0 = j0 / p.chunk;  // chunks are 256 .. 4,096 keys: a block spans 1, 2 or 4 of them, or lies in one
    const int ncb = min(max(kColCols / p.chunk, 1), p.nchunk - c0);
    for (int idx = threadIdx.x; idx < ncb * p.NR; idx += 256) {
        const int cc = idx / p.NR, row = idx - cc * p.NR;
        const double2 pr = p.part[((size_t)bg * p.nchunk + c0 + cc) * p.NRp + row];
        const double2 rn = p.rownorm[(size_t)bg * p.NRp + row];
        wt[cc][row] = (pr.x == -INFINITY || rn.y == 0.0)
                          ? 0.0
                          : __builtin_ldexp(rn.y, (int)fmax(pr.x - rn.x, -2000.0));  // pr.x <= rn.x
    }
    __syncthreads();
    const int j = j0 + 4 * (int)threadIdx.x;
    if (j >= p.Tmax) return;
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    if (j < T) {
        const double* w = wt[j / p.chunk - c0];
        const float* e = p.emap + (size_t)bg * p.NRp * p.Tp + j;
#pragma unroll 8
        for (int r = 0; r < p.NR; ++r) {
            const floatx4 v = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(e + (size_t)r * p.Tp));
            const double wr = w[r];
            a0 = __builtin_fma(wr, (double)v[0], a0);
            a1 = __builtin_fma(wr, (double)v[1], a1);
            a2 = __builtin_fma(wr, (double)v[2], a2);
            a3 = __builtin_fma(wr, (double)v[3], a3);
        }
    }
    float* out = p.col_scores + (size_t)bg * p.Tmax;
    const double a[4] = {a0, a1, a2, a3};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (j + i < p.Tmax) out[j + i] = j + i < T ? (float)a[i] : 0.0f;
}

// ---------------------------------------------------------------- top-k

// Exclusive prefix sum of v over the 1024 threads of the block (16 waves);
// total = the sum over all threads.
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
        const uint32_t c = wsum[w];
        before += w < wave ? c : 0;
        tot += c;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

__global__ __launch_bounds__(1024) void k_topk_select(const float* col_scores, const int32_t* seq_lens, int Hkv,
                                                     int Tmax, hq_policy pol, int stride, int32_t* sel_idx,
                                                     int32_t* sel_count, hq_thresh* thresh) {
    // the candidates' score bits, staged once when they fit (one padding
    // word per 32, so the compaction's per-thread runs fall in different
    // banks); longer contexts read them from global memory in every pass
    __shared__ uint32_t sx[kTopkLds + kTopkLds / 32];
    // kHistCopies copies of the 256-bin histogram, lane l adding to copy
    // l % kHistCopies: the scores of a pass crowd into a few bins, and lanes
    // of one wave adding to one LDS word are serialised
    __shared__ uint32_t hist[kHistCopies * 256];
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t sh_prefix, sh_mask, sh_remaining;
    __shared__ int sh_jk;
    const int g = blockIdx.x, b = blockIdx.y;
    const int bg = b * Hkv + g;
    const int tid = threadIdx.x, lane = tid & 63;
    const int T = seq_lens[b];
    const int ncand = T > pol.window ? T - pol.window : 0;
    const int k = keep_count(T, pol);
    const uint32_t* xs = reinterpret_cast<const uint32_t*>(col_scores + (size_t)bg * Tmax);
    int32_t* sel = sel_idx + (size_t)bg * stride;
    for (int i = k + tid; i < stride; i += 1024) sel[i] = -1;
    if (k == 0) {
        if (tid == 0) {
            sel_count[bg] = 0;
            thresh[bg] = hq_thresh{INFINITY, -1};
        }
        return;
    }
    const bool staged = ncand <= kTopkLds;  // uniform
    if (staged)
        for (int j = tid; j < ncand; j += 1024) sx[j + (j >> 5)] = xs[j];
    auto rd = [&](int j) { return staged ? sx[j + (j >> 5)] : xs[j]; };
    if (tid == 0) {
        sh_prefix = 0;
        sh_mask = 0;
        sh_remaining = (uint32_t)k;
        sh_jk = -1;
    }
    // Radix select, 8 bits per pass from the top: the threshold's bits are
    // fixed one byte at a time; sh_remaining counts the candidates still to
    // take among those matching the fixed bits.
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < kHistCopies * 256; i += 1024) hist[i] = 0;
        __syncthreads();
        const uint32_t prefix = sh_prefix, mask = sh_mask;
        for (int base = 0; base < ncand; base += 1024) {
            const int j = base + tid;
            const uint32_t x = j < ncand ? rd(j) : 0u;
            // (a wave-level add of the lanes sharing a bin, against the
            // contention of the top byte's few bins, measured slower)
            if (j < ncand && (x & mask) == prefix)
                atomicAdd(&hist[(lane & (kHistCopies - 1)) * 256 + ((x >> shift) & 255u)], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // the highest bin at which the count from the top reaches the
            // remaining number: lane l holds bins 255 - 4l .. 252 - 4l
            const uint32_t rem = sh_remaining;
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = 0;
#pragma unroll
                for (int c = 0; c < kHistCopies; ++c) h[i] += hist[c * 256 + 255 - 4 * lane - i];
            }
            const uint32_t s4 = h[0] + h[1] + h[2] + h[3];
            uint32_t incl = s4;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t t = __shfl_up(incl, off);
                if (lane >= off) incl += t;
            }
            const uint32_t excl = incl - s4;
            if (excl < rem && rem <= incl) {  // exactly one lane
                uint32_t cum = excl;
                int i = 0;
                for (; i < 3; ++i) {
                    if (cum + h[i] >= rem) break;
                    cum += h[i];
                }
                const int bin = 255 - 4 * lane - i;
                sh_remaining = rem - cum;
                sh_prefix = prefix | ((uint32_t)bin << shift);
                sh_mask = mask | (255u << shift);
            }
        }
        __syncthreads();
    }
    const uint32_t tau = sh_prefix;
    const uint32_t remaining = sh_remaining;  // ties to take, lowest index first (>= 1)
    // Compaction: thread t owns candidates [t*per, (t+1)*per); index order is
    // thread order, so two block scans give every thread its output offset
    // and its share of the ties.
    const int per = (ncand + 1023) / 1024;
    const int j0 = min(tid * per, ncand), j1 = min(j0 + per, ncand);
    uint32_t ngt = 0, neq = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t x = rd(j);
        ngt += x > tau ? 1u : 0u;
        neq += x == tau ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t eq_base = block_excl_scan(neq, wsum, tot);
    const uint32_t take_eq = eq_base >= remaining ? 0u : min(neq, remaining - eq_base);
    uint32_t pos = block_excl_scan(ngt + take_eq, wsum, tot);
    uint32_t te = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t x = rd(j);
        if (x > tau) {
            sel[pos++] = j;
        } else if (x == tau && te < take_eq) {
            sel[pos++] = j;
            if (eq_base + te == remaining - 1) sh_jk = j;
            ++te;
        }
    }
    __syncthreads();
    if (tid == 0) {
        sel_count[bg] = k;
        thresh[bg] = hq_thresh{__uint_as_float(tau), sh_jk};
    }
}


struct ProbeWs {
    size_t part, rownorm, emap, total;
};
inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

struct ProbeShape {
    int NR, NRp, nrt, ngroups, waves, chunk, nchunk;
};
// Keys per pass-1 workgroup: 4,096, halved (down to 256) while the grid
// would have fewer than 256 workgroups. A pass-1 workgroup holds 109 KiB of
// LDS, so one runs per CU: 256 is one round of the chip's 256 CUs. Longer
// chunks convert each query tile to digits fewer times (32K decode shape,
// pass 1: 2.83 / 2.69 / 2.65 ms with 1,024 / 2,048 / 4,096 keys), and
// chunks that leave CUs idle or add rounds cost more (16K prefill probe:
// 512-key chunks 102 us, 256 123 us, 1,024 164 us).
ProbeShape probe_shape(int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, const hq_policy& pol) {
    ProbeShape s;
    s.NR = (Hq / Hkv) * pol.probe_rows;
    s.NRp = (s.NR + kRT - 1) / kRT * kRT;
    s.nrt = s.NRp / kRT;
    s.ngroups = (s.nrt + kTilesPerWg - 1) / kTilesPerWg;
    s.waves = s.nrt < kTilesPerWg ? s.nrt : kTilesPerWg;
    s.chunk = 4096;
    while (s.chunk > 256 && (int64_t)((Tmax + s.chunk - 1) / s.chunk) * Hkv * s.ngroups * B < 256) s.chunk /= 2;
    s.nchunk = (Tmax + s.chunk - 1) / s.chunk;
    return s;
}
// Row stride of the stored terms: the positions rounded up to a key tile,
// plus one tile so that rows are not a power of two apart (pass 2 reads a
// column block down all rows; at a 32K stride it streamed 4.3 GB at 6.1 TB/s,
// the re-probe's 34,816-position stride at 6.4 TB/s).
inline int probe_tp(int32_t Tmax) { return (Tmax + kKT - 1) / kKT * kKT + kKT; }
ProbeWs probe_ws(int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, const hq_policy& pol) {
    const ProbeShape s = probe_shape(B, Hq, Hkv, Tmax, pol);
    const size_t BG = (size_t)B * Hkv;
    ProbeWs w;
    w.part = 0;
    w.rownorm = al(BG * s.nchunk * s.NRp * 16);
    w.emap = w.rownorm + al(BG * s.NRp * 16);
    w.total = w.emap + al(BG * s.NRp * (size_t)probe_tp(Tmax) * 4);
    return w;
}

}  // namespace

bool probe_shape_supported(int32_t G, int32_t probe_rows) {
    const int64_t NR = (int64_t)G * probe_rows;
    return NR % 16 == 0 && NR <= 512;
}
const char* probe_shape_rule() {
    return "query heads per KV head x probe_rows must be a multiple of 16 and at most 512";
}

size_t probe_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, const hq_policy& pol) {
    return probe_ws(B, Hq, Hkv, Tmax, pol).total;
}

hipError_t launch_probe(const void* q_probe, const void* k, const int32_t* seq_lens, int32_t B, int32_t Hq,
                        int32_t Hkv, int32_t Tmax, bool f16, const hq_policy& pol, float sm_scale,
                        float* col_scores, int32_t* sel_idx, int32_t* sel_count, hq_thresh* thresh, void* ws,
                        hipStream_t s) {
    // probe_shape_supported(G, probe_rows) holds (host check)
    const ProbeShape sh = probe_shape(B, Hq, Hkv, Tmax, pol);
    const ProbeWs w = probe_ws(B, Hq, Hkv, Tmax, pol);
    ProbeParams p;
    p.q = static_cast<const uint16_t*>(q_probe);
    p.k = static_cast<const uint16_t*>(k);
    p.seq_lens = seq_lens;
    p.part = reinterpret_cast<double2*>(static_cast<char*>(ws) + w.part);
    p.rownorm = reinterpret_cast<double2*>(static_cast<char*>(ws) + w.rownorm);
    p.emap = reinterpret_cast<float*>(static_cast<char*>(ws) + w.emap);
    p.col_scores = col_scores;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Tmax = Tmax;
    p.Tp = probe_tp(Tmax);
    p.R = pol.probe_rows;
    p.G = Hq / Hkv;
    p.NR = sh.NR;
    p.NRp = sh.NRp;
    p.ngroups = sh.ngroups;
    p.nchunk = sh.nchunk;
    p.chunk = sh.chunk;
    p.sc2 = (double)sm_scale * 1.4426950408889634074;
    const int threads = 64 * kTilesPerWg;  // 8 waves; waves past the last row tile only move key tiles
    dim3 g1(sh.nchunk, Hkv * sh.ngroups, B);
    if (f16) k_probe_rowstats<true><<<g1, threads, 0, s>>>(p);
    else k_probe_rowstats<false><<<g1, threads, 0, s>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_probe_rowfinal<<<dim3(Hkv, B), 256, 0, s>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_probe_colsum<<<dim3((Tmax + kColCols - 1) / kColCols, Hkv, B), 256, 0, s>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_topk_select<<<dim3(Hkv, B), 1024, 0, s>>>(col_scores, seq_lens, Hkv, Tmax, pol, sel_stride(Tmax, pol),
                                                  sel_idx, sel_count, thresh);
    return hipGetLastError();
}

}  // namespace hq
