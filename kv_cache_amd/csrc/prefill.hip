// hq_prefill_attn: causal hybrid-precision prefill attention (gfx950).
//
// HyQuant pages: the HyQuant abstract (Prefill stage: the vertical-line
// tokens and a local sliding window stay in full precision, the remaining
// context is quantized); "How HyQuant uses hybrid-precision attention to cut
// decode compute", "What hybrid-precision attention changes" (compute the
// selected positions and the window in full precision, the rest in low
// precision); "HyQuant: Hybrid-Precision Quantization for LLM Attention",
// "How this relates to prior wiki pages" (two precision paths updating one
// online-softmax state).
//
// Score of query row i and key j <= i (window W, selected set S of the KV head):
//   j in S or i - j < W : (q_i . k_j) * sm_scale                 bf16 MFMA
//   otherwise           : (Q8_i . K8_j) * sQ * sK * sm_scale      int8 or fp8 MFMA
// The low-precision codes are symmetric per 64-token block over all 128
// channels, INT8: s = fp32(max|x| / 127), code = clamp(rint(x / s), -127, 127);
// or OCP FP8 E4M3 (the policy's choice; the pages leave FP8 as an open third
// precision point): s = fp32(max|x| / 448), code = E4M3 of fp32(x / s),
// rounded to nearest even. Both are one byte per element, so the two
// formats share the layout and the kernels differ only in the conversion and
// the matrix instruction (v_mfma_i32_32x32x32_i8, or gfx950's
// v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands: the same throughput, and
// float scores that need no integer conversion).
//
// Pre-pass (k_pf_quant_q, k_pf_quant_kv, k_pf_gather_sel): Q8/sQ, K8/sK, V
// converted to fp16 and transposed per 64-key block (the PV operand
// layout), a second copy of it with the selected columns zeroed and per-block
// row-sum weights (0 for a selected key) for the INT8 blocks, a 64-bit
// selected-column mask per key block, and gathered tiles of the selected
// columns (16-bit K rows and transposed fp16 V).
//
// Attention (k_pf_attn): one workgroup = 4 waves = 128 query rows of one head;
// each wave owns 32 queries. S^T = K Q^T is computed with 32x32 MFMA tiles so
// a lane holds one query column (16 keys per tile); row maxima need one
// cross-half exchange. Key blocks of 64:
//   * blocks entirely below the window band: int8 MFMA, selected columns
//     dropped through the zeroed V^T copy and zero row-sum weights;
//   * the 4 blocks that touch the band/diagonal: int8 and bf16 MFMA, the
//     score picked per element (band or selected -> bf16), causal mask;
//   * gathered selected columns below the band: bf16 MFMA, no mask needed.
// P goes to fp16 straight from the S^T registers (same key order as the V^T
// operand) for the fp16 PV MFMA; O^T accumulates in fp32. Online softmax in
// log2 units.
// The output and the fp16 V^T tensors, written in whole 128-byte lines, use
// streaming (non-temporal) stores: the output is not read again here and the
// V^T copies are larger than the caches, so keeping them there buys little,
// while dirty lines left behind would be written back during the kernels
// that run after this call (a decode step, in mixed serving). The output is
// staged through LDS so that each store instruction writes whole rows:
// partial lines written this way are not merged before they reach memory.
#include "hq_internal.h"

namespace hq {
namespace {

typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per block

struct PfLayout {
    size_t q8, sq, k8, sk, vt, mask, ksel, vtsel, vt0, wsel, l1q, l1k, route, total;
    int nblk, nsel_tiles, nqb, nw;
};
inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
PfLayout pf_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, const hq_policy& pol) {
    PfLayout w;
    w.nblk = (T + kBN - 1) / kBN;
    const int kmax = sel_stride(T, pol);
    w.nsel_tiles = (kmax + kBN - 1) / kBN;
    const size_t Tp = (size_t)w.nblk * kBN;
    w.q8 = 0;
    w.sq = w.q8 + al((size_t)B * Hq * Tp * kD);
    w.k8 = w.sq + al((size_t)B * Hq * w.nblk * 4);
    w.sk = w.k8 + al((size_t)B * Hkv * Tp * kD);
    w.vt = w.sk + al((size_t)B * Hkv * w.nblk * 4);
    w.mask = w.vt + al((size_t)B * Hkv * Tp * kD * 2);
    w.ksel = w.mask + al((size_t)B * Hkv * w.nblk * 8);
    w.vtsel = w.ksel + al((size_t)B * Hkv * w.nsel_tiles * kBN * kD * 2);
    w.vt0 = w.vtsel + al((size_t)B * Hkv * w.nsel_tiles * kBN * kD * 2);
    w.wsel = w.vt0 + al((size_t)B * Hkv * Tp * kD * 2);
    // tile routing: per-block maxima of the rows' code L1 norms, and per
    // (b, h, 128-row query block) a bit per key block
    w.nqb = (T + kBM - 1) / kBM;
    w.nw = (w.nblk + 63) / 64;
    w.l1q = w.wsel + al((size_t)B * Hkv * w.nblk * 32 * 4);
    w.l1k = w.l1q + al((size_t)B * Hq * w.nblk * 4);
    w.route = w.l1k + al((size_t)B * Hkv * w.nblk * 4);
    w.total = w.route + al((size_t)B * Hq * w.nqb * w.nw * 8);
    return w;
}

__device__ inline float block_max256(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

#pragma clang fp contract(off)
// Symmetric INT8 of one 64 x 128 block (rows beyond T are zero); 256 threads,
// thread t owns row t/4, channels 32*(t%4) .. +31. RECIP: quotients from the
// reciprocal and FMA residual steps (fewer instructions, more registers: the
// Q kernel gains, the K/V kernel, which also writes V^T, runs slower with it).
template <bool F16, bool RECIP, bool FP8>
__device__ __attribute__((always_inline)) inline void quant_block_i8(const uint16_t* src, int rows_valid, int8_t* dst,
                                                                    float* scale, int32_t* l1max) {
    __shared__ float red[4];
    const int t = threadIdx.x, r = t >> 2, c0 = (t & 3) * 32;
    float x[32];
    if (r < rows_valid) {
        const uint4* s4 = reinterpret_cast<const uint4*>(src + (size_t)r * kD + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 u = s4[i];
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[8 * i + 2 * j] = h16_to_f32<F16>(w[j] & 0xFFFFu);
                x[8 * i + 2 * j + 1] = h16_to_f32<F16>(w[j] >> 16);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = 0.f;
    }
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(x[i]));
    am = block_max256(am, red);
    const float s = am / (FP8 ? 448.0f : 127.0f);
    uint32_t packed[8];
    auto pack = [&](auto quot) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t w = 0;
            if constexpr (FP8) {
                // E4M3, round to nearest even; |x / s| <= 448 (1 + 2^-23), so
                // nothing reaches the overflow range; element j in byte j.
                // E4M3 keeps the sign of zero, which the residual steps of the
                // reciprocal route lose (-0 - (+0) = +0): the quotient takes
                // the dividend's sign, as the IEEE divide gives it (s > 0).
                auto qs = [&](float v) { return __builtin_copysignf(quot(v), v); };
                if (s > 0.f) {
                    int v = __builtin_amdgcn_cvt_pk_fp8_f32(qs(x[4 * i]), qs(x[4 * i + 1]), 0, false);
                    v = __builtin_amdgcn_cvt_pk_fp8_f32(qs(x[4 * i + 2]), qs(x[4 * i + 3]), v, true);
                    w = (uint32_t)v;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float c = 0.f;
                    if (s > 0.f) c = fminf(fmaxf(rintf(quot(x[4 * i + j])), -127.f), 127.f);
                    w |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * j);
                }
            }
            packed[i] = w;
        }
    };
    // x / s correctly rounded without a divide per element: y = RN(1/s), then
    // q0 = x * y and two FMA residual steps; by Markstein's theorem the second
    // step gives RN(x / s) once the first has made the quotient faithful. The
    // scale is uniform over the block; tiny, huge or non-finite scales (where
    // a residual could underflow or the reciprocal overflow) take the IEEE
    // divide.
    if (RECIP && s >= 0x1p-100f && s < 0x1p100f) {
        const float y = 1.0f / s;
        pack([&](float v) {
            const float q0 = v * y;
            const float q1 = fmaf(fmaf(-q0, s, v), y, q0);
            return fmaf(fmaf(-q1, s, v), y, q1);
        });
    } else {
        pack([&](float v) { return v / s; });
    }
    uint4* d4 = reinterpret_cast<uint4*>(dst + (size_t)r * kD + c0);
    d4[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    d4[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
    if (t == 0) *scale = s;
    if constexpr (!FP8) {
        if (l1max != nullptr) {  // tile routing: the block's largest row sum of |code| (uniform branch)
            int a = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) a += abs((int)(int8_t)(packed[i] >> (8 * j)));
            a += __shfl_xor(a, 1);  // the four threads of row r
            a += __shfl_xor(a, 2);
            const float mx = block_max256((float)a, red);  // exact: a <= 128 * 127
            if (t == 0) *l1max = (int32_t)mx;
        }
    }
}
#pragma clang fp contract(on)

// Key held at position s of a 64-key V^T row: each 16-key group is stored as
// keys 0-3, 8-11, 4-7, 12-15 (the order one lane half of the PV MFMA reads).
__device__ constexpr int vt_key(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }

struct PfParams {
    const uint16_t* q;   // [B][Hq][T][D]
    const uint16_t* k;   // [B][Hkv][T][D]
    const uint16_t* v;
    const int32_t* sel_idx;
    const int32_t* sel_count;
    int8_t* q8;          // [B][Hq][Tp][D]
    float* sq;           // [B][Hq][nblk]
    int8_t* k8;          // [B][Hkv][Tp][D]
    float* sk;           // [B][Hkv][nblk]
    uint16_t* vt;        // [B][Hkv][nblk][D][64] fp16 V^T per key block, keys in vt_key order
    uint64_t* mask;      // [B][Hkv][nblk] selected-column bits
    uint16_t* ksel;      // [B][Hkv][nsel_tiles][64][D] 16-bit K rows of selected columns
    uint16_t* vtsel;     // [B][Hkv][nsel_tiles][D][64] fp16 V^T of selected columns, vt_key order
    uint16_t* vt0;       // as vt, with the columns of selected keys zero (the INT8 blocks' PV operand)
    uint32_t* wsel;      // [B][Hkv][nblk][2][16] fp16 pairs: 1 for an unselected key, 0 for a selected
                         // one, in the order of the P^T words of lane half 0 / 1
    float* out;
    int out_dt;
    int32_t* l1q;        // [B][Hq][nblk] max row sum |Q8| per 64-row block (tile routing; else null)
    int32_t* l1k;        // [B][Hkv][nblk]
    uint64_t* route;     // [B][Hq][nqb][nw] routed key blocks of each 128-row query block (or null)
    int B, Hq, Hkv, G, T, nblk, nsel_tiles, sel_stride, W, nqb, nw, tile_num, tile_den;
    float c16;           // sm_scale * log2(e)
};

template <bool F16, bool FP8>
__global__ __launch_bounds__(256) void k_pf_quant_q(PfParams p) {
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const size_t Tp = (size_t)p.nblk * kBN;
    const uint16_t* src = p.q + (((size_t)b * p.Hq + h) * p.T + (size_t)blk * kBN) * kD;
    int8_t* dst = p.q8 + (((size_t)b * p.Hq + h) * Tp + (size_t)blk * kBN) * kD;
    quant_block_i8<F16, true, FP8>(src, min(kBN, p.T - blk * kBN), dst, p.sq + ((size_t)b * p.Hq + h) * p.nblk + blk,
                                   p.l1q ? p.l1q + ((size_t)b * p.Hq + h) * p.nblk + blk : nullptr);
}

// K8 + sK, V^T in fp16, and the selected-column mask of one key block.
template <bool F16, bool FP8>
__global__ __launch_bounds__(256) void k_pf_quant_kv(PfParams p) {
    __shared__ uint16_t vs[kBN][kD + 8];
    const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int bg = b * p.Hkv + g;
    const size_t Tp = (size_t)p.nblk * kBN;
    const int rows = min(kBN, p.T - blk * kBN);
    const uint16_t* ksrc = p.k + ((size_t)bg * p.T + (size_t)blk * kBN) * kD;
    quant_block_i8<F16, false, FP8>(ksrc, rows, p.k8 + ((size_t)bg * Tp + (size_t)blk * kBN) * kD, p.sk + (size_t)bg * p.nblk + blk,
                                    p.l1k ? p.l1k + (size_t)bg * p.nblk + blk : nullptr);
    // V -> fp16 -> transposed
    const int t = threadIdx.x, r = t >> 2, c0 = (t & 3) * 32;
    const uint16_t* vsrc = p.v + ((size_t)bg * p.T + (size_t)blk * kBN) * kD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint4 u = make_uint4(0, 0, 0, 0);
        if (r < rows) u = reinterpret_cast<const uint4*>(vsrc + (size_t)r * kD + c0)[i];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            vs[r][c0 + 8 * i + 2 * j] = (uint16_t)f32_to_f16_bits(h16_to_f32<F16>(w[j] & 0xFFFFu));
            vs[r][c0 + 8 * i + 2 * j + 1] = (uint16_t)f32_to_f16_bits(h16_to_f32<F16>(w[j] >> 16));
        }
    }
    // selected-column bits of this block
    __shared__ uint64_t sbits;
    if (t == 0) {
        const int32_t* S = p.sel_idx + (size_t)bg * p.sel_stride;
        const int k = min(max(p.sel_count[bg], 0), p.sel_stride);
        int lo = 0, hi = k;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (S[mid] < blk * kBN) lo = mid + 1;
            else hi = mid;
        }
        uint64_t bits = 0;
        for (int i = lo; i < k && S[i] < blk * kBN + kBN; ++i)
            if (S[i] >= blk * kBN) bits |= 1ull << (S[i] - blk * kBN);
        p.mask[(size_t)bg * p.nblk + blk] = bits;
        sbits = bits;
    }
    __syncthreads();
    const uint64_t bits = sbits;
    uint16_t* vdst = p.vt + ((size_t)bg * p.nblk + blk) * kD * kBN;
    uint16_t* v0dst = p.vt0 + ((size_t)bg * p.nblk + blk) * kD * kBN;
    for (int e = t; e < kD * 8; e += 256) {   // (channel, 8-key segment)
        const int ch = e >> 3, k0 = (e & 7) * 8;
        uint32_t w[4], w0[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ka = vt_key(k0 + 2 * j), kb = vt_key(k0 + 2 * j + 1);
            w[j] = (uint32_t)vs[ka][ch] | ((uint32_t)vs[kb][ch] << 16);
            w0[j] = w[j] & (((bits >> ka) & 1ull) ? 0xFFFF0000u : 0xFFFFFFFFu) &
                    (((bits >> kb) & 1ull) ? 0x0000FFFFu : 0xFFFFFFFFu);
        }
        st_nt(vdst + (size_t)ch * kBN + k0, make_uint4(w[0], w[1], w[2], w[3]));
        st_nt(v0dst + (size_t)ch * kBN + k0, make_uint4(w0[0], w0[1], w0[2], w0[3]));
    }
    // row-sum weights: word 4j + e of lane half hf pairs the keys of P^T
    // operand j, elements 2e and 2e + 1 (S^T tile j/2, registers
    // 8(j%2) + 2e and + 1, i.e. keys 32(j/2) + 8(2(j%2) + e/2) + 4hf + 2(e%2) and + 1)
    if (t < 32) {
        const int hf = t >> 4, j = (t >> 2) & 3, e = t & 3;
        const int ka = 32 * (j >> 1) + 8 * (2 * (j & 1) + (e >> 1)) + 4 * hf + 2 * (e & 1);
        const uint32_t one = 0x3C00u;  // fp16 1.0
        p.wsel[((size_t)bg * p.nblk + blk) * 32 + t] =
            (((bits >> ka) & 1ull) ? 0u : one) | (((bits >> (ka + 1)) & 1ull) ? 0u : (one << 16));
    }
}

// Tile routing: for one (b, h, 128-row query block), rank its candidate key
// blocks (below the window band for every row of the block) by the INT8
// score error bound's shape E = sK (A + B + 5D/2) and set the bits of the
// floor(tile_num * n / tile_den) largest, ties to the lower block. The keys
// (E bits, ~kb) are sorted in LDS (bitonic, ascending; E >= 0 so its bit
// pattern orders like its value, and every real key is above the zero
// padding).
__global__ __launch_bounds__(256) void k_pf_route(PfParams p) {
    __shared__ uint64_t key[kRouteMaxT / kBN];
    __shared__ unsigned long long bits[kRouteMaxT / kBN / 64];
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
    const int bg = b * p.Hkv + h / p.G;
    const int i0 = qb * kBM;
    const int nkb = min(p.nblk, (i0 + kBM + kBN - 1) / kBN);
    const int kb_band = min(nkb, max(0, (i0 - p.W + 1) / kBN));
    const int n = (int)((int64_t)p.tile_num * kb_band / p.tile_den);
    for (int w = t; w < p.nw; w += 256) bits[w] = 0ull;
    if (n > 0) {
        const int32_t* lq = p.l1q + ((size_t)b * p.Hq + h) * p.nblk;
        const int A = max(lq[2 * qb], 2 * qb + 1 < p.nblk ? lq[2 * qb + 1] : 0);
        const int32_t* lk = p.l1k + (size_t)bg * p.nblk;
        const float* sk = p.sk + (size_t)bg * p.nblk;
        int P = 1;
        while (P < kb_band) P <<= 1;
        for (int i = t; i < P; i += 256) {
            uint64_t kv = 0;
            if (i < kb_band) {
                const float e = sk[i] * (float)(A + lk[i] + 5 * kD / 2);
                kv = ((uint64_t)__float_as_uint(e) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
            }
            key[i] = kv;
        }
        __syncthreads();
        for (int k = 2; k <= P; k <<= 1)
            for (int j = k >> 1; j > 0; j >>= 1) {
                for (int i = t; i < P; i += 256) {
                    const int ixj = i ^ j;
                    if (ixj > i) {
                        const uint64_t a = key[i], c = key[ixj];
                        if (((i & k) == 0) ? (a > c) : (a < c)) {
                            key[i] = c;
                            key[ixj] = a;
                        }
                    }
                }
                __syncthreads();
            }
        for (int i = t; i < n; i += 256) {
            const uint32_t kb = 0xFFFFFFFFu - (uint32_t)key[P - 1 - i];
            atomicOr(&bits[kb >> 6], 1ull << (kb & 63));
        }
    }
    __syncthreads();
    uint64_t* out = p.route + (((size_t)b * p.Hq + h) * p.nqb + qb) * p.nw;
    for (int w = t; w < p.nw; w += 256) out[w] = bits[w];
}

// Gathered tiles of selected columns: 16-bit K rows and fp16 V^T.
template <bool F16>
__global__ __launch_bounds__(256) void k_pf_gather_sel(PfParams p) {
    __shared__ uint16_t vs[kBN][kD + 8];
    const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int bg = b * p.Hkv + g;
    const int k = min(max(p.sel_count[bg], 0), p.sel_stride);
    if (tile * kBN >= k) return;
    const int32_t* S = p.sel_idx + (size_t)bg * p.sel_stride;
    const int t = threadIdx.x, r = t >> 2, c0 = (t & 3) * 32;
    const int i = tile * kBN + r;
    const bool ok = i < k && S[i] >= 0 && S[i] < p.T;
    const int pos = ok ? S[i] : 0;
    const uint4* ks = reinterpret_cast<const uint4*>(p.k + ((size_t)bg * p.T + pos) * kD + c0);
    const uint4* vsrc = reinterpret_cast<const uint4*>(p.v + ((size_t)bg * p.T + pos) * kD + c0);
    uint4* kd = reinterpret_cast<uint4*>(p.ksel + (((size_t)bg * p.nsel_tiles + tile) * kBN + r) * kD + c0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint4 kk = ok ? ks[j] : make_uint4(0, 0, 0, 0);
        kd[j] = kk;
        const uint4 u = ok ? vsrc[j] : make_uint4(0, 0, 0, 0);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vs[r][c0 + 8 * j + 2 * e] = (uint16_t)f32_to_f16_bits(h16_to_f32<F16>(w[e] & 0xFFFFu));
            vs[r][c0 + 8 * j + 2 * e + 1] = (uint16_t)f32_to_f16_bits(h16_to_f32<F16>(w[e] >> 16));
        }
    }
    __syncthreads();
    uint16_t* vdst = p.vtsel + ((size_t)bg * p.nsel_tiles + tile) * kD * kBN;
    for (int e = t; e < kD * 8; e += 256) {
        const int ch = e >> 3, k0 = (e & 7) * 8;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)vs[vt_key(k0 + 2 * j)][ch] | ((uint32_t)vs[vt_key(k0 + 2 * j + 1)][ch] << 16);
        st_nt(vdst + (size_t)ch * kBN + k0, make_uint4(w[0], w[1], w[2], w[3]));
    }
}

// ---------------------------------------------------------------- attention

// LDS row strides (bytes), padded so that the 8 lanes of one 128-bit LDS
// access phase read 8 different rows in disjoint banks.
constexpr int kK8Stride = kD + 16;        // int8 K rows (128 B + pad)
constexpr int kK16Stride = 2 * kD + 16;   // 16-bit K rows (256 B + pad)
constexpr int kVtStride = 2 * kBN + 16;   // fp16 V^T rows (one channel, 64 keys)
constexpr float kLazy = 8.0f;             // log2-domain growth that triggers a rescale

// Output staging at the end of the kernel (the tiles are dead by then): per
// wave 32 rows of 128 values, rows padded by 16 bytes.
constexpr int kOutRowF32 = 4 * kD + 16;
constexpr int kOutRow16 = 2 * kD + 16;

struct Smem {
    int8_t k8[2][kBN * kK8Stride];
    uint8_t vt[2][kD * kVtStride];
    uint8_t k16[kBN * kK16Stride];
    uint4 wt[2][8];  // row-sum weights of the INT8 blocks (two slots, like vt)
};
static_assert(4 * 32 * kOutRowF32 <= sizeof(Smem), "output staging must fit in the tile LDS");

// S^T register r of lane half hf in a 32-key MFMA tile holds key
// 8*(r/4) + 4*hf + r%4 (the 32x32 MFMA output layout, M = keys).
__device__ constexpr int st_key(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// Cooperative copies into LDS (256 threads).
// A [64][128] 16-bit K tile in two halves, so that a block's loads can all
// be issued before any store: rows at or beyond rows_valid repeat the last
// valid row (their scores are masked; the reads stay inside the tensor).
struct K16Regs {
    uint4 v[4];
};
__device__ inline K16Regs load_k16(const uint16_t* src, int rows_valid) {
    const int t = threadIdx.x;
    K16Regs k;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = t + 256 * i, r = min(e >> 4, rows_valid - 1), c = (e & 15) * 16;
        k.v[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(src) + (size_t)r * 2 * kD + c);
    }
    return k;
}
__device__ inline void store_k16(uint8_t* dst, const K16Regs& k) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = t + 256 * i, r = e >> 4, c = (e & 15) * 16;
        *reinterpret_cast<uint4*>(dst + r * kK16Stride + c) = k.v[i];
    }
}

template <int N>
struct IConst {
    static constexpr int value = N;
};

// Register staging of one INT8 K block (8 KB) and one fp16 V^T block (16 KB):
// thread t moves 16-byte chunks e = t + 256 i (row e / 8, column chunk e % 8).
struct Stage {
    uint4 k0, k1, v0, v1, v2, v3;
};
__device__ inline const uint4& ld16(const void* base, int e, int row_bytes) {
    return *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(base) + (e >> 3) * row_bytes + (e & 7) * 16);
}
__device__ inline void st16(void* base, int e, int row_bytes, const uint4& v) {
    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(base) + (e >> 3) * row_bytes + (e & 7) * 16) = v;
}
__device__ inline Stage stage_load(const int8_t* k8, const uint16_t* vt) {
    const int t = threadIdx.x;
    Stage s;
    s.k0 = ld16(k8, t, kD);
    s.k1 = ld16(k8, t + 256, kD);
    s.v0 = ld16(vt, t, 2 * kBN);
    s.v1 = ld16(vt, t + 256, 2 * kBN);
    s.v2 = ld16(vt, t + 512, 2 * kBN);
    s.v3 = ld16(vt, t + 768, 2 * kBN);
    return s;
}
__device__ inline void stage_store(Smem& sm, int buf, const Stage& s) {
    const int t = threadIdx.x;
    st16(sm.k8[buf], t, kK8Stride, s.k0);
    st16(sm.k8[buf], t + 256, kK8Stride, s.k1);
    st16(sm.vt[buf], t, kVtStride, s.v0);
    st16(sm.vt[buf], t + 256, kVtStride, s.v1);
    st16(sm.vt[buf], t + 512, kVtStride, s.v2);
    st16(sm.vt[buf], t + 768, kVtStride, s.v3);
}

// Accumulators of the low-precision scores: exact int32 sums for INT8,
// fp32 for FP8 (E4M3 products are exact in fp32; the sums round).
template <bool FP8> struct LowAcc { typedef intx16 type; };
template <> struct LowAcc<true> { typedef floatx16 type; };

// One 32-key S^T tile (keys 32tt..32tt+31) of the low-precision products.
// INT8: K = 128 in 4 steps of 32; lane l supplies row l % 32, bytes
// 32 ks + 16 (l / 32) .. + 15 of each operand. FP8: 2 steps of 64; the lane
// supplies the two 16-byte pieces of the INT8 steps 2 k2 and 2 k2 + 1 as one
// 32-byte operand. Both operands are assembled the same way, so every
// channel meets its partner once whatever order the instruction sums in.
template <bool FP8>
__device__ inline typename LowAcc<FP8>::type st_low_tile(const int8_t* k8, const intx4 (&qb)[4], int tt) {
    const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
    typename LowAcc<FP8>::type acc = {};
    const int8_t* row = k8 + (32 * tt + m) * kK8Stride + 16 * hf;
    if constexpr (FP8) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const intx4 a0 = *reinterpret_cast<const intx4*>(row + 64 * k2);
            const intx4 a1 = *reinterpret_cast<const intx4*>(row + 64 * k2 + 32);
            const intx8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const intx4 b0 = qb[2 * k2], b1 = qb[2 * k2 + 1];
            const intx8 bq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            // format 0 (E4M3) for both operands, no block scaling
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bq, acc, 0, 0, 0, 0, 0, 0);
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const intx4 a = *reinterpret_cast<const intx4*>(row + 32 * ks);
            acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qb[ks], acc, 0, 0, 0);
        }
    }
    return acc;
}
// S^T (64 keys x 32 queries) of the low-precision products: two 32x32 tiles.
template <bool FP8>
__device__ inline void st_low(const int8_t* k8, const intx4 (&qb)[4], typename LowAcc<FP8>::type (&s)[2]) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) s[tt] = st_low_tile<FP8>(k8, qb, tt);
}
// S^T in 16-bit (bf16 or fp16 inputs), K = 128 in 8 steps.
template <bool F16>
__device__ inline void st_16(const uint8_t* k16, const intx4 (&qb)[8], floatx16 (&s)[2]) {
    const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        floatx16 acc = {};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const intx4 a = *reinterpret_cast<const intx4*>(k16 + (32 * tt + m) * kK16Stride + 2 * (16 * ks + 8 * hf));
            if constexpr (F16)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, qb[ks]),
                                                             acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, qb[ks]), acc, 0, 0, 0);
        }
        s[tt] = acc;
    }
}

// One 32-key S^T tile (keys 32tt..32tt+31) of the 16-bit products.
template <bool F16>
__device__ inline floatx16 st_16_tile(const uint8_t* k16, const intx4 (&qb)[8], int tt) {
    const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
    floatx16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const intx4 a = *reinterpret_cast<const intx4*>(k16 + (32 * tt + m) * kK16Stride + 2 * (16 * ks + 8 * hf));
        if constexpr (F16)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), __builtin_bit_cast(halfx8, qb[ks]),
                                                         acc, 0, 0, 0);
        else
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                          __builtin_bit_cast(bf16x8, qb[ks]), acc, 0, 0, 0);
    }
    return acc;
}

// O^T += V^T P^T for one 64-key block. Step j covers keys 16j..16j+15: the
// P^T operand is registers 8*(j%2)..+7 of S^T tile j/2 (keys 16j + 4hf +
// {0..3, 8..11}); the V^T block stores each 16-key group in the order
// (0-3, 8-11, 4-7, 12-15) so lane half hf reads its 8 keys with one 128-bit load.
__device__ inline void pv_block(const uint8_t* vt, const halfx8 (&pb)[4], floatx16 (&o)[4]) {
    const int lane = threadIdx.x & 63, m = lane & 31, hf = lane >> 5;
    // key step outer, channel tile inner: consecutive MFMAs write different
    // accumulators
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const intx4 a = *reinterpret_cast<const intx4*>(vt + (32 * ct + m) * kVtStride + 16 * hf + 32 * j);
            o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8, a), pb[j], o[ct], 0, 0, 0);
        }
    }
}

__device__ inline float swap_max(float v) {
    auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ inline int swap_max_i(int v) {
    auto sw = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v, false, false);
    return max((int)sw[0], (int)sw[1]);
}

// Lazy online-softmax reference: p = 2^(x - m_ref) is used as long as the
// block maximum stays within 2^kLazy of m_ref (p < 2^8 fits fp16); when it
// grows further the reference moves to the new maximum and l, o are rescaled
// (a wave-uniform branch taken rarely after the first blocks).
__device__ inline void lazy_rescale(float bm, float& m_ref, float& l, floatx16 (&o)[4]) {
    const bool grow = bm > m_ref + kLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? bm : m_ref;
        const float alpha = (!grow) ? 1.0f : (m_ref == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_ref - mn));
        m_ref = mn;
        l *= alpha;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
    }
}

__device__ inline uint32_t pack_h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, half2_t{(_Float16)a, (_Float16)b});
}

// p (fp32, >= 0) -> fp16 P^T operands; l += sum of the rounded values.
__device__ inline void pack_p(const float (&p)[2][16], halfx8 (&pb)[4], float& l) {
    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] = pack_h2(p[j >> 1][8 * (j & 1) + 2 * e], p[j >> 1][8 * (j & 1) + 2 * e + 1]);
            l = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[e]), ones, l, false);
        }
        const intx4 v = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        pb[j] = __builtin_bit_cast(halfx8, v);
    }
}

// As pack_p, with the row sum weighted per key (fp16 pairs: 0 drops a key).
__device__ inline void pack_p_w(const float (&p)[2][16], halfx8 (&pb)[4], float& l, const uint4 (&wt)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t w[4];
        const uint32_t ww[4] = {wt[j].x, wt[j].y, wt[j].z, wt[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] = pack_h2(p[j >> 1][8 * (j & 1) + 2 * e], p[j >> 1][8 * (j & 1) + 2 * e + 1]);
            l = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, w[e]), __builtin_bit_cast(half2_t, ww[e]), l, false);
        }
        const intx4 v = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        pb[j] = __builtin_bit_cast(halfx8, v);
    }
}

// Softmax step of a block given log2-domain scores x (-inf = masked).
__device__ inline void softmax_x(float (&x)[2][16], float& m_ref, float& l, floatx16 (&o)[4], halfx8 (&pb)[4]) {
    float bm = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) bm = fmaxf(bm, x[tt][r]);
    bm = swap_max(bm);
    lazy_rescale(bm, m_ref, l, o);
    const float mr = m_ref == -INFINITY ? 0.0f : m_ref;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[tt][r] = __builtin_amdgcn_exp2f(x[tt][r] - mr);
    pack_p(x, pb, l);
}

// As softmax_x for unscaled scores: x = raw * scale in log2 units (scale > 0,
// so the block maximum is taken on the raw values), one FMA per element.
__device__ inline void softmax_scaled(float (&x)[2][16], float scale, float& m_ref, float& l, floatx16 (&o)[4],
                                      halfx8 (&pb)[4]) {
    float bm = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) bm = fmaxf(bm, x[tt][r]);
    bm = swap_max(bm) * scale;
    lazy_rescale(bm, m_ref, l, o);
    const float nmr = m_ref == -INFINITY ? 0.0f : -m_ref;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[tt][r] = __builtin_amdgcn_exp2f(fmaf(x[tt][r], scale, nmr));
    pack_p(x, pb, l);
}

// Wave64 lane mask of the lanes whose S^T element r = 4a + b (tile tt)
// holds a selected key: lane half 0 holds key 32tt + 8a + b, half 1 key
// 32tt + 8a + 4 + b; `byte` = the 8 selection bits of keys 32tt + 8a ... +7.
__device__ inline uint64_t elem_lanes(uint32_t byte, int b) {
    return (((byte >> b) & 1u) ? 0x00000000FFFFFFFFull : 0ull) | (((byte >> (4 + b)) & 1u) ? 0xFFFFFFFF00000000ull : 0ull);
}

// v = sentinel on the elements of selected keys. The tests on the selection
// bits are scalar, so only 8-key groups that hold a selected key cost VALU
// work (one v_cndmask per element with a scalar lane mask).
template <typename V, typename A>
__device__ inline void mask_selected(uint64_t selbits, A (&v)[2], V sentinel) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const uint32_t byte = (uint32_t)(selbits >> (32 * tt + 8 * a)) & 0xFFu;
            if (byte) {
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4)
                    v[tt][4 * a + b4] = __builtin_amdgcn_inverse_ballot_w64(elem_lanes(byte, b4)) ? sentinel
                                                                                                  : v[tt][4 * a + b4];
            }
        }
}

template <bool F16, bool FP8>
__global__ __launch_bounds__(256, 2) void k_pf_attn(PfParams p) {
    __shared__ Smem sm;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m_ = lane & 31, hf = lane >> 5;
    // Workgroup order: consecutive ids cycle over (b, KV head) first, so the
    // XCD that a workgroup lands on (id mod 8) sees one KV head's key
    // blocks; query blocks are taken latest (heaviest) first.
    const int nqb = (p.T + kBM - 1) / kBM;
    const int BG = p.B * p.Hkv;
    const int id = blockIdx.x;
    const int bg = id % BG;
    const int rest = id / BG;
    const int hh = rest % p.G;
    const int qb = nqb - 1 - rest / p.G;
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int h = g * p.G + hh;
    const int i0 = qb * kBM;
    const int W = p.W;
    const size_t Tp = (size_t)p.nblk * kBN;
    const int qrow0 = i0 + 32 * wave;
    const int qi = qrow0 + m_;
    const bool qvalid = qi < p.T;
    const float c16 = p.c16;
    const float sq = p.sq[((size_t)b * p.Hq + h) * p.nblk + min(qrow0 >> 6, p.nblk - 1)];

    float m_ref = -INFINITY, l = 0.f;
    floatx16 o[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) o[ct] = floatx16{};
    halfx8 pb[4];

    intx4 q8b[4];
    {
        const int8_t* q8 = p.q8 + (((size_t)b * p.Hq + h) * Tp + (size_t)(qvalid ? qi : 0)) * kD;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) q8b[ks] = *reinterpret_cast<const intx4*>(q8 + 32 * ks + 16 * hf);
    }

    const int nkb = min(p.nblk, (i0 + kBM + kBN - 1) / kBN);  // key blocks holding keys <= last row
    const int kb_band = min(nkb, max(0, (i0 - W + 1) / kBN));  // blocks below it miss every row's band
    const int32_t* S = p.sel_idx + (size_t)bg * p.sel_stride;
    int nsel = 0;  // selected columns below kb_band * 64
    {
        const int k = min(max(p.sel_count[bg], 0), p.sel_stride);
        const int lim = kb_band * kBN;
        int lo = 0, hi = k;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (S[mid] < lim) lo = mid + 1;
            else hi = mid;
        }
        nsel = lo;
    }

    // ---- phase A: the blocks touching the window band / diagonal, and
    // ---- phase B: gathered selected columns below the band (16-bit scores)
    {
        intx4 q16b[8];
        {
            const uint16_t* q16 = p.q + (((size_t)b * p.Hq + h) * p.T + (size_t)(qvalid ? qi : 0)) * kD;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const intx4 z = {0, 0, 0, 0};
                q16b[ks] = qvalid ? *reinterpret_cast<const intx4*>(q16 + 16 * ks + 8 * hf) : z;
            }
        }
        // routed tiles (below the band, chosen by k_pf_route): 16-bit scores
        // for every key of the block except the selected ones, which phase B
        // covers (their p is 0 here)
        if (p.route != nullptr) {
            const uint64_t* rw = p.route + (((size_t)b * p.Hq + h) * p.nqb + qb) * p.nw;
            for (int w = 0; w < (kb_band + 63) / 64; ++w) {
                uint64_t mw = rw[w];
                while (mw) {
                    const int kb = 64 * w + __builtin_ctzll(mw);
                    mw &= mw - 1;
                    __syncthreads();
                    {
                        const int t = threadIdx.x;
                        const uint16_t* vsrc = p.vt + ((size_t)bg * p.nblk + kb) * kD * kBN;
                        const uint4 v0 = ld16(vsrc, t, 2 * kBN), v1 = ld16(vsrc, t + 256, 2 * kBN);
                        const uint4 v2 = ld16(vsrc, t + 512, 2 * kBN), v3 = ld16(vsrc, t + 768, 2 * kBN);
                        const K16Regs kr = load_k16(p.k + ((size_t)bg * p.T + (size_t)kb * kBN) * kD, kBN);
                        st16(sm.vt[0], t, kVtStride, v0);
                        st16(sm.vt[0], t + 256, kVtStride, v1);
                        st16(sm.vt[0], t + 512, kVtStride, v2);
                        st16(sm.vt[0], t + 768, kVtStride, v3);
                        store_k16(sm.k16, kr);
                    }
                    __syncthreads();
                    const uint64_t selbits = p.mask[(size_t)bg * p.nblk + kb];
                    float x[2][16];
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        const floatx16 sb = st_16_tile<F16>(sm.k16, q16b, tt);
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
                            const uint32_t byte = (uint32_t)(selbits >> (32 * tt + 8 * a)) & 0xFFu;
#pragma unroll
                            for (int b4 = 0; b4 < 4; ++b4) {
                                const bool sel = __builtin_amdgcn_inverse_ballot_w64(elem_lanes(byte, b4));
                                x[tt][4 * a + b4] = sel ? -INFINITY : sb[4 * a + b4] * c16;
                            }
                        }
                    }
                    softmax_x(x, m_ref, l, o, pb);
                    pv_block(sm.vt[0], pb, o);
                }
            }
        }
        for (int kb = kb_band; kb < nkb; ++kb) {
            __syncthreads();
            {
                const Stage st = stage_load(p.k8 + ((size_t)bg * Tp + (size_t)kb * kBN) * kD,
                                            p.vt + ((size_t)bg * p.nblk + kb) * kD * kBN);
                const K16Regs kr = load_k16(p.k + ((size_t)bg * p.T + (size_t)kb * kBN) * kD, min(kBN, p.T - kb * kBN));
                stage_store(sm, 0, st);
                store_k16(sm.k16, kr);
            }
            __syncthreads();
            const float c8 = sq * p.sk[(size_t)bg * p.nblk + kb] * c16;
            const uint64_t selbits = p.mask[(size_t)bg * p.nblk + kb];
            // Key kl = 32tt + 8a + b4 + 4hf of element r = 4a + b4 (tile tt) is
            // in the window band when kl > qi - 64kb - W and masked when
            // kl > qi - 64kb (which also covers keys at or beyond T: qi < T).
            // The compares are against per-lane bounds, with the lane half's
            // 4hf folded in; the selection test is a scalar lane mask. Rows
            // at or beyond T are computed with a zero query and not stored.
            const int lc = qi - kb * kBN - 4 * hf, lw = lc - W;
            float x[2][16];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                const auto si = st_low_tile<FP8>(sm.k8[0], q8b, tt);
                const floatx16 sb = st_16_tile<F16>(sm.k16, q16b, tt);
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const uint32_t byte = (uint32_t)(selbits >> (32 * tt + 8 * a)) & 0xFFu;
#pragma unroll
                    for (int b4 = 0; b4 < 4; ++b4) {
                        const int r = 4 * a + b4, k0 = 32 * tt + 8 * a + b4;
                        const bool sel = __builtin_amdgcn_inverse_ballot_w64(elem_lanes(byte, b4));
                        float val = (sel || k0 > lw) ? sb[r] * c16 : (float)si[r] * c8;
                        if (k0 > lc) val = -INFINITY;
                        x[tt][r] = val;
                    }
                }
            }
            softmax_x(x, m_ref, l, o, pb);
            pv_block(sm.vt[0], pb, o);
        }
        // Gathered tiles, double-buffered: tile n+1's K and V^T loads are
        // in flight while tile n is computed (K slots: sm.k16 and the INT8 K
        // area, free until phase C; V^T slots: sm.vt[0..1]).
        const int ntile = (nsel + kBN - 1) / kBN;
        if (ntile > 0) {
            const int t = threadIdx.x;
            auto kbuf = [&](int slot) { return slot ? reinterpret_cast<uint8_t*>(&sm.k8[0][0]) : sm.k16; };
            auto load_sel = [&](int tile, K16Regs& kr, uint4 (&vv)[4]) {
                kr = load_k16(p.ksel + ((size_t)bg * p.nsel_tiles + tile) * kBN * kD, kBN);
                const uint16_t* src = p.vtsel + ((size_t)bg * p.nsel_tiles + tile) * kD * kBN;
#pragma unroll
                for (int i = 0; i < 4; ++i) vv[i] = ld16(src, t + 256 * i, 2 * kBN);
            };
            auto store_sel = [&](int slot, const K16Regs& kr, const uint4 (&vv)[4]) {
                store_k16(kbuf(slot), kr);
#pragma unroll
                for (int i = 0; i < 4; ++i) st16(sm.vt[slot], t + 256 * i, kVtStride, vv[i]);
            };
            __syncthreads();  // the band blocks are done with LDS
            {
                K16Regs kr;
                uint4 vv[4];
                load_sel(0, kr, vv);
                store_sel(0, kr, vv);
            }
            __syncthreads();
            for (int tile = 0; tile < ntile; ++tile) {
                const int slot = tile & 1;
                const bool more = tile + 1 < ntile;
                K16Regs kr;
                uint4 vv[4];
                load_sel(more ? tile + 1 : tile, kr, vv);
                floatx16 sb[2];
                st_16<F16>(kbuf(slot), q16b, sb);
                float x[2][16];
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[tt][r] = sb[tt][r];
                if ((tile + 1) * kBN > nsel) {  // the last, partial tile: mask its unused columns
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            if (tile * kBN + 32 * tt + st_key(r, hf) >= nsel) x[tt][r] = -INFINITY;
                }
                softmax_scaled(x, c16, m_ref, l, o, pb);
                pv_block(sm.vt[slot], pb, o);
                if (more) store_sel(slot ^ 1, kr, vv);
                __syncthreads();
            }
        }
    }

    // ---- phase C: INT8 blocks below the band (selected columns dropped).
    // Software pipeline per wave: the QK MFMAs of block kb+1 are issued
    // before the softmax of block kb, so the matrix cores and the VALU work
    // of one wave overlap. LDS: K8 of block kb in K slot kb%2, V^T of block
    // kb in V slot kb%2; iteration kb loads K8[kb+2] and V^T[kb+1] into
    // registers (buffer loads with scalar offsets) and stores them into the
    // slots freed by the previous iteration; one barrier per iteration.
    // Selected columns are dropped without per-element work: their V^T
    // columns are zero (vt0) and their row-sum weights are zero (wsel), so
    // p of a selected key is computed but contributes nothing. (Its p stays
    // finite: phase B has seen the key's exact score, so the reference is at
    // most 2^8 below it, and the INT8 score differs from it by far less than
    // the 2^7 headroom left to fp16.)
    if (kb_band > 0) {
        const int t = threadIdx.x;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.k8 + (size_t)bg * Tp * kD), (short)0, kb_band * kBN * kD, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.vt0 + (size_t)bg * p.nblk * kD * kBN), (short)0, kb_band * kD * kBN * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.wsel + (size_t)bg * p.nblk * 32), (short)0, kb_band * 128, 0x00020000);
        const int voff = 16 * t;  // chunk t of a block; rows of K8 and V^T are both 128 bytes
        auto ld = [&](const __amdgpu_buffer_rsrc_t& r, int soff) {
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
        };
        // the 128-byte weight record of a block: every thread loads chunk t % 8
        auto ldw = [&](int soff) {
            return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * (t & 7), soff, 0));
        };
        __syncthreads();  // the band phases are done with LDS
        {
            const uint4 w0 = ldw(0);
            if (t < 8) sm.wt[0][t] = w0;
            stage_store(sm, 0, Stage{ld(rk, 0), ld(rk, 4096), ld(rv, 0), ld(rv, 4096), ld(rv, 8192), ld(rv, 12288)});
            if (kb_band > 1) {
                st16(sm.k8[1], t, kK8Stride, ld(rk, 8192));
                st16(sm.k8[1], t + 256, kK8Stride, ld(rk, 8192 + 4096));
            }
        }
        __syncthreads();
        typename LowAcc<FP8>::type sA[2], sB[2];
        st_low<FP8>(sm.k8[0], q8b, sA);
        const uint64_t* rwc = p.route ? p.route + (((size_t)b * p.Hq + h) * p.nqb + qb) * p.nw : nullptr;
        __syncthreads();  // every wave has read K slot 0 before iteration 0 refills it

        auto step = [&](auto P, typename LowAcc<FP8>::type (&sc)[2], typename LowAcc<FP8>::type (&sn)[2], int kb) {
            constexpr int cur = decltype(P)::value;
            const int kn2 = min(kb + 2, kb_band - 1), kn1 = min(kb + 1, kb_band - 1);
            const uint4 k0 = ld(rk, kn2 * 8192), k1 = ld(rk, kn2 * 8192 + 4096);
            const uint4 v0 = ld(rv, kn1 * 16384), v1 = ld(rv, kn1 * 16384 + 4096);
            const uint4 v2 = ld(rv, kn1 * 16384 + 8192), v3 = ld(rv, kn1 * 16384 + 12288);
            const uint4 wn = ldw(kn1 * 128);
            // QK of the next block (on the last block: of stale LDS data, unused),
            // unconditional so that it shares the softmax's basic block
            st_low<FP8>(sm.k8[cur ^ 1], q8b, sn);
            const float c8 = sq * p.sk[(size_t)bg * p.nblk + kb] * c16;
            uint4 wt[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) wt[j] = sm.wt[cur][4 * hf + j];
            // No block maximum on the common path: p = 2^(s - m_ref) with the
            // reference from the earlier blocks (the band and the selected
            // columns come first, so it is normally the row maximum already).
            // Only if some p of the block reaches 2^15 (the block sum shows
            // it, and catches inf) is the maximum taken and the state rescaled.
            float x[2][16];
            float lb = 0.0f;
            {
                // a routed block was scored in 16 bits in phase A: p = 2^-inf = 0 here
                const bool routed = rwc != nullptr && ((rwc[kb >> 6] >> (kb & 63)) & 1ull);
                const float nmr = routed ? -INFINITY : (m_ref == -INFINITY ? 0.0f : -m_ref);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) x[tt][r] = __builtin_amdgcn_exp2f(fmaf((float)sc[tt][r], c8, nmr));
                pack_p_w(x, pb, lb, wt);
                // interleave: the loads first, then each of the next block's
                // QK MFMAs followed by a share of this block's softmax VALU work
                __builtin_amdgcn_sched_group_barrier(0x0020, 7, 0);  // buffer loads
                __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);  // LDS reads
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // LDS read
                    __builtin_amdgcn_sched_group_barrier(0x0002, 14, 0); // VALU
                }
            }
            if (__builtin_amdgcn_ballot_w64(!(lb <= 32768.0f))) {
                const uint64_t selbits = p.mask[(size_t)bg * p.nblk + kb];
                float bm;
                if constexpr (FP8) {
                    mask_selected(selbits, sc, -INFINITY);
                    float fmx = -INFINITY;
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) fmx = fmaxf(fmx, sc[tt][r]);
                    fmx = swap_max(fmx);
                    bm = fmx == -INFINITY ? -INFINITY : fmx * c8;
                } else {
                    mask_selected(selbits, sc, (int)INT_MIN);
                    int imax = INT_MIN;
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int r = 0; r < 16; ++r) imax = max(imax, sc[tt][r]);
                    imax = swap_max_i(imax);
                    bm = imax == INT_MIN ? -INFINITY : (float)imax * c8;
                }
                lazy_rescale(bm, m_ref, l, o);
                const float nmr = m_ref == -INFINITY ? 0.0f : -m_ref;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        bool masked;
                        if constexpr (FP8) masked = sc[tt][r] == -INFINITY;
                        else masked = sc[tt][r] == INT_MIN;
                        x[tt][r] = masked ? 0.0f : __builtin_amdgcn_exp2f(fmaf((float)sc[tt][r], c8, nmr));
                    }
                lb = 0.0f;
                pack_p(x, pb, lb);
            }
            l += lb;
            pv_block(sm.vt[cur], pb, o);
            st16(sm.k8[cur], t, kK8Stride, k0);
            st16(sm.k8[cur], t + 256, kK8Stride, k1);
            st16(sm.vt[cur ^ 1], t, kVtStride, v0);
            st16(sm.vt[cur ^ 1], t + 256, kVtStride, v1);
            st16(sm.vt[cur ^ 1], t + 512, kVtStride, v2);
            st16(sm.vt[cur ^ 1], t + 768, kVtStride, v3);
            if (t < 8) sm.wt[cur ^ 1][t] = wn;
            __syncthreads();
        };
        for (int kb = 0; kb < kb_band; kb += 2) {
            step(IConst<0>{}, sA, sB, kb);
            if (kb + 1 >= kb_band) break;
            step(IConst<1>{}, sB, sA, kb + 1);
        }
    }

    // combine the two lane halves of each query and write. Each wave stages
    // its 32 x 128 output tile in LDS (rows padded by 16 bytes), then writes
    // it out with streaming stores, 1 KiB of whole rows per instruction.
    {
        auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
        l = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float inv = 1.0f / l;  // rows beyond T: unused
    const bool f32 = p.out_dt == HQ_F32;
    uint8_t* stg = reinterpret_cast<uint8_t*>(&sm) + wave * (32 * kOutRowF32);
    __syncthreads();  // every wave is done with the LDS tiles
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int ch = 32 * ct + 8 * r4 + 4 * hf;
            const float vv[4] = {o[ct][4 * r4] * inv, o[ct][4 * r4 + 1] * inv, o[ct][4 * r4 + 2] * inv,
                                 o[ct][4 * r4 + 3] * inv};
            if (f32) {
                *reinterpret_cast<float4*>(stg + m_ * kOutRowF32 + 4 * ch) = make_float4(vv[0], vv[1], vv[2], vv[3]);
            } else {
                uint32_t hb[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (p.out_dt == HQ_F16) hb[e] = f32_to_f16_bits(vv[e]);
                    else {
                        uint32_t xb = __float_as_uint(vv[e]);
                        xb += 0x7FFFu + ((xb >> 16) & 1u);
                        hb[e] = xb >> 16;
                    }
                }
                *reinterpret_cast<uint2*>(stg + m_ * kOutRow16 + 2 * ch) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
            }
        }
    }
    __syncthreads();
    // 1 KiB per instruction: 2 rows (fp32) or 4 rows (16-bit) of the wave's tile
    if (f32) {
        float* ob = p.out + (((size_t)b * p.Hq + h) * p.T + qrow0) * kD;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 2 * i + (lane >> 5), ck = lane & 31;
            if (qrow0 + row < p.T)
                st_nt(ob + (size_t)row * kD + 4 * ck, *reinterpret_cast<const uint4*>(stg + row * kOutRowF32 + 16 * ck));
        }
    } else {
        uint16_t* ob = reinterpret_cast<uint16_t*>(p.out) + (((size_t)b * p.Hq + h) * p.T + qrow0) * kD;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 4 * i + (lane >> 4), ck = lane & 15;
            if (qrow0 + row < p.T)
                st_nt(ob + (size_t)row * kD + 8 * ck, *reinterpret_cast<const uint4*>(stg + row * kOutRow16 + 16 * ck));
        }
    }
}

template <bool F16, bool FP8>
void launch_pf(const PfParams& p, const PfLayout& w, int32_t B, int32_t Hq, int32_t Hkv, int32_t T, hipStream_t s) {
    k_pf_quant_q<F16, FP8><<<dim3(w.nblk, Hq, B), 256, 0, s>>>(p);
    k_pf_quant_kv<F16, FP8><<<dim3(w.nblk, Hkv, B), 256, 0, s>>>(p);
    k_pf_gather_sel<F16><<<dim3(w.nsel_tiles, Hkv, B), 256, 0, s>>>(p);
    if (p.route != nullptr) k_pf_route<<<dim3(w.nqb, Hq, B), 256, 0, s>>>(p);
    k_pf_attn<F16, FP8><<<dim3(((T + kBM - 1) / kBM) * Hq * B), 256, 0, s>>>(p);
}

}  // namespace

size_t prefill_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, const hq_policy& pol) {
    return pf_layout(B, Hq, Hkv, T, pol).total;
}

hipError_t launch_prefill(const void* q, const void* k, const void* v, int32_t B, int32_t Hq, int32_t Hkv,
                          int32_t T, bool f16, const hq_policy& pol, const int32_t* sel_idx,
                          const int32_t* sel_count, int32_t sel_stride_, float sm_scale, void* out,
                          hq_dtype out_dt, void* ws, hipStream_t s) {
    const PfLayout w = pf_layout(B, Hq, Hkv, T, pol);
    char* base = static_cast<char*>(ws);
    PfParams p;
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.sel_idx = sel_idx;
    p.sel_count = sel_count;
    p.q8 = reinterpret_cast<int8_t*>(base + w.q8);
    p.sq = reinterpret_cast<float*>(base + w.sq);
    p.k8 = reinterpret_cast<int8_t*>(base + w.k8);
    p.sk = reinterpret_cast<float*>(base + w.sk);
    p.vt = reinterpret_cast<uint16_t*>(base + w.vt);
    p.mask = reinterpret_cast<uint64_t*>(base + w.mask);
    p.ksel = reinterpret_cast<uint16_t*>(base + w.ksel);
    p.vtsel = reinterpret_cast<uint16_t*>(base + w.vtsel);
    p.vt0 = reinterpret_cast<uint16_t*>(base + w.vt0);
    p.wsel = reinterpret_cast<uint32_t*>(base + w.wsel);
    const bool route = pol.tile_num > 0;
    p.l1q = route ? reinterpret_cast<int32_t*>(base + w.l1q) : nullptr;
    p.l1k = route ? reinterpret_cast<int32_t*>(base + w.l1k) : nullptr;
    p.route = route ? reinterpret_cast<uint64_t*>(base + w.route) : nullptr;
    p.nqb = w.nqb;
    p.nw = w.nw;
    p.tile_num = pol.tile_num;
    p.tile_den = pol.tile_den > 0 ? pol.tile_den : 1;
    p.out = static_cast<float*>(out);
    p.out_dt = (int)out_dt;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.G = Hq / Hkv;
    p.T = T;
    p.nblk = w.nblk;
    p.nsel_tiles = w.nsel_tiles;
    p.sel_stride = sel_stride_;
    p.W = pol.window;
    p.c16 = sm_scale * 1.4426950408889634f;
    const bool fp8 = pol.low_fmt == HQ_LOW_FP8;
    if (f16) {
        if (fp8) launch_pf<true, true>(p, w, B, Hq, Hkv, T, s);
        else launch_pf<true, false>(p, w, B, Hq, Hkv, T, s);
    } else {
        if (fp8) launch_pf<false, true>(p, w, B, Hq, Hkv, T, s);
        else launch_pf<false, false>(p, w, B, Hq, Hkv, T, s);
    }
    return hipGetLastError();
}

}  // namespace hq
