// hq_probe_select: vertical-line probe and top-k column selection (gfx950).
//
// HyQuant pages: "HyQuant: Hybrid-Precision Quantization for LLM
// Attention", TL;DR and "What problem it solves" (a small number of key
// columns are attended to by almost every query row; a lightweight pattern
// signal finds them without calibration), "Gaps" (the probe must not
// materialise the attention map); "How HyQuant uses hybrid-precision
// attention to cut decode compute", "Why preserve selected positions?" (keep
// the top 5% high-score positions).
//
// Column score c[j] = sum over the G query heads and the last R probe rows of
// the row-normalised causal softmax. The map is never stored: pass 1
// computes each row's normaliser over key chunks (relative to a reference
// logit per chunk), a combine kernel merges the chunks, pass 2 recomputes the
// logits and sums the normalised probabilities per column.
//
// Precision: the selection is a ranking of scores whose top-k gap is often
// only ~1e-5..1e-4 relative on long contexts, so the logits are formed
// exactly (bf16/fp16 inputs converted to fp64, v_mfma_f64_16x16x4 with fp64
// accumulation), exponentials use an fp64 polynomial, and normalisers and
// column sums accumulate in fp64. The scores are rounded once to fp32.
//
// Top-k: one workgroup per (b, g); 4-pass 8-bit radix select on the fp32 bit
// patterns (scores are >= 0, so bit order = value order) with LDS histograms
// and a wave-parallel scan over the bins, then an index-ordered compaction
// (each thread a contiguous run of candidates, two block scans) that takes
// all scores above the threshold and the lowest-index ties.
#include "hq_internal.h"

namespace hq {
namespace {

typedef double double4_t __attribute__((ext_vector_type(4)));

// Keys per pass-1 workgroup: 1,024, or 512 when 1,024-key chunks would give
// fewer than 1,024 workgroups (four per CU of the chip), so that short or
// small-batch calls still spread over every CU. A multiple of 16.
inline int probe_key_chunk(int32_t B, int32_t Hkv, int32_t Tmax) {
    const int64_t wg = (int64_t)((Tmax + 1023) / 1024) * Hkv * B;
    return wg >= 1024 ? 1024 : 512;
}

// 2^x in fp64 (x finite or very negative): 2^n * e^(f ln2), |f| <= 1/2,
// Taylor series to degree 14 (truncation < 1e-17 relative). The coefficients
// 1/14! .. 1/2! come in the kernel arguments (c): uniform values in scalar
// registers that the FMAs read directly (as literals the compiler keeps them
// in vector registers and copies one into place before every FMA).
constexpr int kExpCoefs = 13;
__device__ inline double exp2_f64(double x, const double (&c)[kExpCoefs]) {
    if (x < -1000.0) return 0.0;
    const double n = rint(x);
    const double y = (x - n) * 0.69314718055994530942;
    double e = c[0];
#pragma unroll
    for (int i = 1; i < kExpCoefs; ++i) e = fma(e, y, c[i]);
    e = fma(e, y, 1.0);
    e = fma(e, y, 1.0);
    return ldexp(e, (int)n);
}

// 32 consecutive 16-bit values (one lane's share of a row), loaded raw so
// that the next tile's loads can be in flight while this tile is computed.
struct Raw32 {
    uint4 u[4];
};
__device__ inline Raw32 load_raw32(const uint16_t* src, bool ok) {
    const uint4* s4 = reinterpret_cast<const uint4*>(src);
    Raw32 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.u[i] = ok ? s4[i] : make_uint4(0, 0, 0, 0);
    return r;
}
template <bool F16>
__device__ inline void cvt32_f64(const Raw32& r, double* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {r.u[i].x, r.u[i].y, r.u[i].z, r.u[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[8 * i + 2 * j] = (double)h16_to_f32<F16>(w[j] & 0xFFFFu);
            out[8 * i + 2 * j + 1] = (double)h16_to_f32<F16>(w[j] >> 16);
        }
    }
}
template <bool F16>
__device__ inline void load32_f64(const uint16_t* src, bool ok, double* out) {
    cvt32_f64<F16>(load_raw32(src, ok), out);
}

// Exact 16 x 16 block of dot products over 128 channels. Lane l supplies row
// (l % 16) of A and column (l % 16) of B for channels 32*(l/16) .. +31; the
// result element i of lane l is D[4*i + l/16][l % 16] (rows interleave across
// the four 16-lane groups).
__device__ inline double4_t mfma_dot128(const double* a, const double* b) {
    double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 32; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], b[s], acc, 0, 0, 0);
    return acc;
}

// As mfma_dot128 with the B operand given as raw 16-bit values, each
// converted to fp64 just before the MFMA that reads it.
template <bool F16>
__device__ inline double raw_elem(const Raw32& r, int s) {
    const uint4& u = r.u[s >> 3];
    const uint32_t w = ((s >> 1) & 3) == 0 ? u.x : ((s >> 1) & 3) == 1 ? u.y : ((s >> 1) & 3) == 2 ? u.z : u.w;
    return (double)h16_to_f32<F16>((s & 1) ? (w >> 16) : (w & 0xFFFFu));
}
template <bool F16>
__device__ inline double4_t mfma_dot128_rb(const double* a, const Raw32& br) {
    double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 32; ++s) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], raw_elem<F16>(br, s), acc, 0, 0, 0);
    return acc;
}
struct ProbeParams {
    const uint16_t* q;     // [B][Hq][R][D]
    const uint16_t* k;     // [B][Hkv][Tmax][D]
    const int32_t* seq_lens;
    double2* part;         // [B][Hkv][nchunk][NR] (m, l) per key chunk: l = sum of 2^(x - m), m a reference
    double2* rows;         // [B][Hkv][NR] (M, 1/L) over all chunks, M = the largest chunk reference
    float* col_scores;     // [B][Hkv][Tmax]
    int32_t B, Hq, Hkv, Tmax, R, G, NR, nchunk, chunk;  // chunk: keys per pass-1 workgroup
    double sc2;            // sm_scale * log2(e)
    double ec[kExpCoefs];  // 1/14!, 1/13!, ..., 1/2!: the exp2_f64 series
};

__device__ inline const uint16_t* qrow(const ProbeParams& p, int b, int g, int row) {
    const int h = row / p.R, r = row % p.R;
    return p.q + (((size_t)b * p.Hq + g * p.G + h) * p.R + r) * kD;
}
__device__ inline int row_pos(const ProbeParams& p, int T, int row) { return T - p.R + (row % p.R); }

// Pass 1: per (key chunk, g, b), online reference / sum of 2^x per probe
// row. A workgroup of 16 waves, one 16-row tile of probe rows per wave (its
// queries held in fp64), streams the chunk's keys 16 at a time: each key tile
// is converted to fp64 once into LDS (double-buffered; the next tile's raw
// values are loaded while this one is computed) and read by every wave.
constexpr int kPW = 16;          // waves per pass-1 workgroup
constexpr int kKRow = kD + 2;    // LDS row stride in doubles (16-byte pad: no bank conflicts across rows)
template <bool F16>
__device__ inline double4_t mfma_dot128_lds(const double* a, const double* brow) {
    double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 32; s += 2) {
        const double2 bb = *reinterpret_cast<const double2*>(brow + s);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s], bb.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a[s + 1], bb.y, acc, 0, 0, 0);
        if ((s & 7) == 6) asm volatile("" ::: "memory");  // bound the LDS reads in flight
    }
    return acc;
}
template <bool F16>
__global__ __launch_bounds__(1024) void k_probe_rowstats(ProbeParams p) {
    __shared__ __align__(16) double kt[2][16][kKRow];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int T = p.seq_lens[b];
    const int key_lo = chunk * p.chunk;
    const int bg = b * p.Hkv + g;
    const int li = lane & 15, kq = lane >> 4;
    const uint16_t* kbase = p.k + (size_t)bg * p.Tmax * kD;
    const int nrt = p.NR / 16;
    double2* part = p.part + ((size_t)bg * p.nchunk + chunk) * p.NR;
    if (key_lo >= T) {  // no key of this chunk exists: empty statistics
        for (int r = tid; r < p.NR; r += 1024) part[r] = make_double2(-INFINITY, 0.0);
        return;
    }
    const int key_hi = min(key_lo + p.chunk, T);
    const int ntile = (key_hi - key_lo + 15) / 16;
    // staging: thread t < 256 moves 8 channels (16 bytes) of key t / 16 of a tile
    const int srow = (tid >> 4) & 15, sc0 = (tid & 15) * 8;
    auto stage_load = [&](int t) {
        const int key = key_lo + 16 * t + srow;
        const bool ok = tid < 256 && key < key_hi;
        return ok ? *reinterpret_cast<const uint4*>(kbase + (size_t)key * kD + sc0) : make_uint4(0, 0, 0, 0);
    };
    auto stage_store = [&](int buf, const uint4& raw) {
        if (tid < 256) {
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
            double* dst = &kt[buf][srow][sc0];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<double2*>(dst + 2 * j) =
                    make_double2((double)h16_to_f32<F16>(w[j] & 0xFFFFu), (double)h16_to_f32<F16>(w[j] >> 16));
        }
    };
    for (int rt0 = 0; rt0 < nrt; rt0 += kPW) {
        const int rt = rt0 + wave;
        const bool active = rt < nrt;  // wave-uniform
        stage_store(0, stage_load(0));
        __syncthreads();
        double m[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[i] = -INFINITY;
            l[i] = 0.0;
        }
        double a[32];
        int pos[4];
        if (active) {
            load32_f64<F16>(qrow(p, b, g, rt * 16 + li) + 32 * kq, true, a);
#pragma unroll
            for (int i = 0; i < 4; ++i) pos[i] = row_pos(p, T, rt * 16 + 4 * i + kq);
        }
        // m is a reference, not the running maximum: l = sum of 2^(x - m)
        // with m moved only when a logit exceeds it by more than 2^9 (and on
        // the first one), so the common path takes one exp per element and
        // no divergent branch. Terms up to 2^512 are exact in fp64 range; the
        // chunk merge and the normalisation accept any reference.
        for (int t = 0; t < ntile; ++t) {
            const int cur = t & 1;
            const bool more = t + 1 < ntile;
            const uint4 nraw = more ? stage_load(t + 1) : make_uint4(0, 0, 0, 0);
            if (active) {
                const int key = key_lo + 16 * t + li;
                const bool kok = key < key_hi;
                const double4_t acc = mfma_dot128_lds<F16>(a, &kt[cur][li][32 * kq]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (kok && pos[i] >= 0 && key <= pos[i]) {
                        const double x = acc[i] * p.sc2;
                        if (x > m[i] + 512.0) {
                            l[i] = l[i] * exp2_f64(m[i] - x, p.ec);
                            m[i] = x;
                        }
                        l[i] += exp2_f64(x - m[i], p.ec);
                    }
                }
            }
            if (more) stage_store(cur ^ 1, nraw);
            __syncthreads();
        }
        if (active) {
            // merge the 16 lanes that hold the same rows (different keys)
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const double m2 = __shfl_xor(m[i], off), l2 = __shfl_xor(l[i], off);
                    const double M = fmax(m[i], m2);
                    double L = 0.0;
                    if (m[i] != -INFINITY) L += l[i] * exp2_f64(m[i] - M, p.ec);
                    if (m2 != -INFINITY) L += l2 * exp2_f64(m2 - M, p.ec);
                    m[i] = M;
                    l[i] = L;
                }
            }
            if (li == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) part[rt * 16 + kq + 4 * i] = make_double2(m[i], l[i]);
            }
        }
    }
}

// Merge the chunk statistics of every probe row: (M, 1/L), with M the
// largest chunk reference and L = sum of l * 2^(m - M).
__global__ __launch_bounds__(256) void k_probe_rowfinal(ProbeParams p) {
    const int g = blockIdx.x, b = blockIdx.y;
    const int bg = b * p.Hkv + g;
    const int T = p.seq_lens[b];
    const int nch = (T + p.chunk - 1) / p.chunk;
    for (int row = threadIdx.x; row < p.NR; row += 256) {
        double M = -INFINITY;
        for (int c = 0; c < nch; ++c) M = fmax(M, p.part[((size_t)bg * p.nchunk + c) * p.NR + row].x);
        double L = 0.0;
        for (int c = 0; c < nch; ++c) {
            const double2 v = p.part[((size_t)bg * p.nchunk + c) * p.NR + row];
            if (v.x != -INFINITY) L += v.y * exp2_f64(v.x - M, p.ec);
        }
        p.rows[(size_t)bg * p.NR + row] = make_double2(M, L > 0.0 ? 1.0 / L : 0.0);
    }
}

// Pass 2: per (256-key block, g, b), column sums of the normalised softmax.
// Each of the 16 waves holds 16 keys in fp64; the probe rows stream through
// LDS 16 at a time, converted to fp64 once per workgroup (double-buffered,
// the next tile's raw values loaded while this one is computed).
__device__ inline double4_t mfma_dot128_lda(const double* arow, const double* b) {
    double4_t acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 32; s += 2) {
        const double2 aa = *reinterpret_cast<const double2*>(arow + s);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(aa.x, b[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(aa.y, b[s + 1], acc, 0, 0, 0);
        if ((s & 7) == 6) asm volatile("" ::: "memory");  // bound the LDS reads in flight
    }
    return acc;
}
constexpr int kColKeys = 16 * kPW;  // keys per pass-2 workgroup
template <bool F16>
__global__ __launch_bounds__(1024) void k_probe_colsum(ProbeParams p) {
    __shared__ __align__(16) double qt[2][16][kKRow];
    __shared__ double2 rs[512];
    __shared__ int rpos[512];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int T = p.seq_lens[b];
    const int bg = b * p.Hkv + g;
    const int li = lane & 15, kq = lane >> 4;
    const int key = blk * kColKeys + wave * 16 + li;
    if (blk * kColKeys >= T) {
        if (tid < kColKeys && blk * kColKeys + tid < p.Tmax)
            p.col_scores[(size_t)bg * p.Tmax + blk * kColKeys + tid] = 0.0f;
        return;
    }
    // staging: thread t < 256 moves 8 channels (16 bytes) of probe row t / 16 of a tile
    const int srow = (tid >> 4) & 15, sc0 = (tid & 15) * 8;
    auto stage_load = [&](int rt) {
        return tid < 256 ? *reinterpret_cast<const uint4*>(qrow(p, b, g, rt * 16 + srow) + sc0) : make_uint4(0, 0, 0, 0);
    };
    auto stage_store = [&](int buf, const uint4& raw) {
        if (tid < 256) {
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
            double* dst = &qt[buf][srow][sc0];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<double2*>(dst + 2 * j) =
                    make_double2((double)h16_to_f32<F16>(w[j] & 0xFFFFu), (double)h16_to_f32<F16>(w[j] >> 16));
        }
    };
    for (int row = tid; row < p.NR; row += 1024) {
        rs[row] = p.rows[(size_t)bg * p.NR + row];
        rpos[row] = row_pos(p, T, row);
    }
    stage_store(0, stage_load(0));
    __syncthreads();
    const bool kok = key < T;
    double bv[32];
    load32_f64<F16>(p.k + ((size_t)bg * p.Tmax + (kok ? key : 0)) * kD + 32 * kq, kok, bv);
    double colacc = 0.0;
    const int nrt = p.NR / 16;
    for (int rt = 0; rt < nrt; ++rt) {
        const int cur = rt & 1;
        const bool more = rt + 1 < nrt;
        const uint4 nraw = more ? stage_load(rt + 1) : make_uint4(0, 0, 0, 0);
        const double4_t acc = mfma_dot128_lda(&qt[cur][li][32 * kq], bv);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = rt * 16 + 4 * i + kq;
            const int pr = rpos[row];
            if (kok && pr >= 0 && key <= pr) {
                const double2 st = rs[row];
                colacc += exp2_f64(acc[i] * p.sc2 - st.x, p.ec) * st.y;
            }
        }
        if (more) stage_store(cur ^ 1, nraw);
        __syncthreads();
    }
    colacc += __shfl_xor(colacc, 16);
    colacc += __shfl_xor(colacc, 32);
    if (kq == 0 && key < p.Tmax) p.col_scores[(size_t)bg * p.Tmax + key] = kok ? (float)colacc : 0.0f;
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
    __shared__ uint32_t hist[256];
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
        for (int i = tid; i < 256; i += 1024) hist[i] = 0;
        __syncthreads();
        const uint32_t prefix = sh_prefix, mask = sh_mask;
        for (int j = tid; j < ncand; j += 1024) {
            const uint32_t x = xs[j];
            if ((x & mask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 64) {
            // the highest bin at which the count from the top reaches the
            // remaining number: lane l holds bins 255 - 4l .. 252 - 4l
            const uint32_t rem = sh_remaining;
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = hist[255 - 4 * lane - i];
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
        const uint32_t x = xs[j];
        ngt += x > tau ? 1u : 0u;
        neq += x == tau ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t eq_base = block_excl_scan(neq, wsum, tot);
    const uint32_t take_eq = eq_base >= remaining ? 0u : min(neq, remaining - eq_base);
    uint32_t pos = block_excl_scan(ngt + take_eq, wsum, tot);
    uint32_t te = 0;
    for (int j = j0; j < j1; ++j) {
        const uint32_t x = xs[j];
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
    size_t part, rows, total;
};
inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
ProbeWs probe_ws(int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, const hq_policy& pol) {
    const int G = Hq / Hkv;
    const size_t NR = (size_t)G * pol.probe_rows;
    const int kc = probe_key_chunk(B, Hkv, Tmax);
    const size_t nchunk = (Tmax + kc - 1) / kc;
    ProbeWs w;
    w.part = 0;
    w.rows = al((size_t)B * Hkv * nchunk * NR * 16);
    w.total = w.rows + al((size_t)B * Hkv * NR * 16);
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
    const int G = Hq / Hkv;
    const int NR = G * pol.probe_rows;  // probe_shape_supported(G, probe_rows) holds (host check)
    const ProbeWs w = probe_ws(B, Hq, Hkv, Tmax, pol);
    ProbeParams p;
    p.q = static_cast<const uint16_t*>(q_probe);
    p.k = static_cast<const uint16_t*>(k);
    p.seq_lens = seq_lens;
    p.part = reinterpret_cast<double2*>(static_cast<char*>(ws) + w.part);
    p.rows = reinterpret_cast<double2*>(static_cast<char*>(ws) + w.rows);
    p.col_scores = col_scores;
    p.B = B;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.Tmax = Tmax;
    p.R = pol.probe_rows;
    p.G = G;
    p.NR = NR;
    p.chunk = probe_key_chunk(B, Hkv, Tmax);
    p.nchunk = (Tmax + p.chunk - 1) / p.chunk;
    p.sc2 = (double)sm_scale * 1.4426950408889634074;
    {
        double f = 1.0;  // 14! .. 2!
        for (int k = 2; k <= 14; ++k) f *= k;
        for (int i = 0; i < kExpCoefs; ++i) {
            p.ec[i] = 1.0 / f;
            f /= 14 - i;
        }
    }
    dim3 g1(p.nchunk, Hkv, B);
    if (f16) k_probe_rowstats<true><<<g1, 1024, 0, s>>>(p);
    else k_probe_rowstats<false><<<g1, 1024, 0, s>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_probe_rowfinal<<<dim3(Hkv, B), 256, 0, s>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    dim3 g2((Tmax + kColKeys - 1) / kColKeys, Hkv, B);
    if (f16) k_probe_colsum<true><<<g2, 1024, 0, s>>>(p);
    else k_probe_colsum<false><<<g2, 1024, 0, s>>>(p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_topk_select<<<dim3(Hkv, B), 1024, 0, s>>>(col_scores, seq_lens, Hkv, Tmax, pol, sel_stride(Tmax, pol),
                                                  sel_idx, sel_count, thresh);
    return hipGetLastError();
}

}  // namespace hq
