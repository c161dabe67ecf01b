// Re-probing the hybrid cache from decode-time queries (gfx950).
//
// Pages: "HyQuant: Hybrid-Precision Quantization for LLM Attention", "Gaps"
// (whether the vertical-line columns found on the prompt stay the heavy
// columns through decoding is left open, notably under heavy batching); TL;DR
// (the columns are found with a lightweight signal of the attention pattern).
// The re-probe runs the prompt probe's statistic again, over the keys the
// cache now holds and the last R decode queries, then counts how many of the
// newly selected columns are already in the kept store.
//
// The probe's kernels take dense 16-bit keys in position order, so the cache
// is first expanded into the workspace: kept and window rows are copied,
// INT4 rows are dequantized (fp32 code*s + z, one rounding, then rounded to
// the cache's 16-bit type, half to even). The expansion moves ~80 bytes in
// and 256 out per token; the probe that follows costs ~(G*R/16) int8 matrix
// instructions per 64 keys and bounds the call, so a fused dequantizing probe
// would save little.
#include "hq_internal.h"

namespace hq {
namespace {

struct ExpandParams {
    hq_cache c;
    uint8_t* kx;         // [B][Hkv][tcap][D] 16-bit
    int32_t* seq_lens;   // [B]
    uint8_t* kept;       // [B][Hkv][tcap]: 1 where the position is in the kept store
    int32_t tcap;
    int32_t nq_tiles, nk_tiles;  // INT4 tiles, kept tiles; window tiles follow
};

__device__ inline uint32_t bf16_rne_bits(float x) {  // finite x
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One workgroup per 64-slot tile of one store of one (b, g); thread task
// id = 256*it + tid covers slot id/16, 16-byte chunk id%16 (channels
// 8*chunk .. 8*chunk+7), so the 16 threads of a slot write its 256-byte row
// contiguously. Every position below seq_len sits in exactly one store, so
// every row and flag below seq_len is written once.
template <bool F16>
__global__ __launch_bounds__(256) void k_reprobe_expand(ExpandParams p) {
    const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int Hkv = p.c.Hkv, W = p.c.window;
    const int bg = b * Hkv + g;
    const Counts cn = reinterpret_cast<const Counts*>(p.c.counts)[bg];
    const int T = min(cn.seq_len, p.tcap);
    if (tile == 0 && g == 0 && threadIdx.x == 0) p.seq_lens[b] = max(T, 1);
    uint8_t* dst = p.kx + (size_t)bg * p.tcap * (kD * 2);
    uint8_t* kflag = p.kept + (size_t)bg * p.tcap;
    const int kind = tile < p.nq_tiles ? 0 : tile < p.nq_tiles + p.nk_tiles ? 1 : 2;
    const int lt = kind == 0 ? tile : kind == 1 ? tile - p.nq_tiles : tile - p.nq_tiles - p.nk_tiles;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int id = it * 256 + threadIdx.x, s = id >> 4, ch = id & 15;
        const int i = lt * kTile + s;
        int pos;
        uint4 val;
        uint8_t flag = 0;
        if (kind == 0) {
            const QSpan qs = q_span(p.c, bg);
            if (i >= min(cn.n_q, qs.tiles * kTile)) continue;
            pos = p.c.q_pos[(size_t)qs.tile0 * kTile + i];
            const size_t tb = (size_t)qs.tile0 + lt;
            const uint32_t w =
                *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.c.k_codes) + tb * kTileBytesQ +
                                                   kq_word(s, 8 * ch));
            const uint32_t sz = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(p.c.k_meta) +
                                                                   tb * 1024 + kmeta_word(s, ch >> 2));
            const float sc = f16_to_f32(sz & 0xFFFFu), zc = f16_to_f32(sz >> 16);
            uint32_t h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // code*s is exact in fp32 (4 bits times an 11-bit significand): one rounding
                const float x = fmaf((float)((w >> mf_nib(e)) & 15u), sc, zc);
                h[e] = F16 ? f32_to_f16_bits(x) : bf16_rne_bits(x);
            }
            val = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        } else if (kind == 1) {
            if (i >= min(cn.n_keep, p.c.cap_keep)) continue;
            pos = p.c.keep_pos[(size_t)bg * p.c.cap_keep + i];
            val = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.c.k_keep) +
                                                  ((size_t)bg * (p.c.cap_keep / kTile) + lt) * kTileBytes16 +
                                                  k16_off(s, ch));
            flag = 1;
        } else {
            // ring slot i holds the position in [T - W, T) congruent to i mod W
            const int base = T - W;
            if (base < 0) {
                if (i >= T) continue;
                pos = i;
            } else {
                pos = base + (i - base % W + W) % W;
            }
            val = *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(p.c.k_win) +
                                                  ((size_t)bg * (W / kTile) + lt) * kTileBytes16 + k16_off(s, ch));
        }
        if (pos < 0 || pos >= T) continue;
        *reinterpret_cast<uint4*>(dst + (size_t)pos * (kD * 2) + ch * 16) = val;
        if (ch == 0) kflag[pos] = flag;
    }
}

// n_persist[b][g] = number of selected columns whose position is in the
// kept store. One workgroup per (b, g).
__global__ __launch_bounds__(256) void k_reprobe_persist(const int32_t* sel_idx, const int32_t* sel_count,
                                                         int32_t stride, const uint8_t* kept, int32_t tcap,
                                                         int32_t* n_persist) {
    const int bg = blockIdx.y * gridDim.x + blockIdx.x;
    const int n = min(sel_count[bg], stride);
    int cnt = 0;
    for (int i = threadIdx.x; i < n; i += 256) {
        const int j = sel_idx[(size_t)bg * stride + i];
        if (j >= 0 && j < tcap) cnt += kept[(size_t)bg * tcap + j];
    }
    __shared__ int red[4];
    float v = wave_sum((float)cnt);  // exact: counts stay far below 2^24
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = (int)v;
    __syncthreads();
    if (threadIdx.x == 0) n_persist[bg] = red[0] + red[1] + red[2] + red[3];
}

inline size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

struct ReprobeWs {
    size_t kx, seq_lens, kept, probe, total;
};
ReprobeWs reprobe_ws(const hq_cache& c, int32_t Hq, const hq_policy& pol) {
    const int32_t tcap = reprobe_tcap(c);
    const size_t BG = (size_t)c.B * c.Hkv;
    ReprobeWs w;
    w.kx = 0;
    w.seq_lens = al(BG * tcap * kD * 2);
    w.kept = w.seq_lens + al((size_t)c.B * 4);
    w.probe = w.kept + al(BG * tcap);
    w.total = w.probe + probe_ws_bytes(c.B, Hq, c.Hkv, tcap, pol);
    return w;
}

}  // namespace

int32_t reprobe_tcap(const hq_cache& c) { return c.cap_q + c.cap_keep + c.window; }

size_t reprobe_ws_bytes(const hq_cache& c, int32_t Hq, const hq_policy& pol) {
    return reprobe_ws(c, Hq, pol).total;
}

hipError_t launch_reprobe(const hq_cache& c, const void* q_recent, int32_t Hq, const hq_policy& pol, float sm_scale,
                          float* col_scores, int32_t* sel_idx, int32_t* sel_count, hq_thresh* thresh,
                          int32_t* n_persist, void* ws, hipStream_t s) {
    const ReprobeWs w = reprobe_ws(c, Hq, pol);
    const int32_t tcap = reprobe_tcap(c);
    uint8_t* base = static_cast<uint8_t*>(ws);
    ExpandParams e;
    e.c = c;
    e.kx = base + w.kx;
    e.seq_lens = reinterpret_cast<int32_t*>(base + w.seq_lens);
    e.kept = base + w.kept;
    e.tcap = tcap;
    e.nq_tiles = c.cap_q / kTile;
    e.nk_tiles = c.cap_keep / kTile;
    const dim3 grid(e.nq_tiles + e.nk_tiles + c.window / kTile, c.Hkv, c.B);
    if (c.dt == HQ_F16) k_reprobe_expand<true><<<grid, 256, 0, s>>>(e);
    else k_reprobe_expand<false><<<grid, 256, 0, s>>>(e);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = launch_probe(q_recent, e.kx, e.seq_lens, c.B, Hq, c.Hkv, tcap, c.dt == HQ_F16, pol, sm_scale, col_scores,
                       sel_idx, sel_count, thresh, base + w.probe, s);
    if (err != hipSuccess) return err;
    k_reprobe_persist<<<dim3(c.Hkv, c.B), 256, 0, s>>>(sel_idx, sel_count, sel_stride(tcap, pol), e.kept, tcap,
                                                        n_persist);
    return hipGetLastError();
}

}  // namespace hq
