// hq_quantize_kv: build the hybrid KV cache of a prompt (gfx950).
//
// HyQuant pages: "HyQuant: Hybrid-Precision Quantization for LLM
// Attention", flowchart (persistently attended columns and the recent local
// window go to high precision, everything else low-bit); "How HyQuant uses
// hybrid-precision attention to cut decode compute", "What the authors
// tested" (Key-4bit / Value-4bit for the rest) and "Memory and runtime
// costs" (retained tokens held only in 16 bits).
//
// One workgroup per destination tile of 64 slots of one (b, g): INT4 tiles
// gather the n-th non-selected position (binary search on the selected set),
// quantize K and V per 32-channel group (4 threads per slot) and write the
// codes in the decode kernel's tile layouts; kept tiles copy the selected
// rows; ring tiles copy the last `window` rows into slot = position % window.
// Writes are full 64-slot tiles, contiguous across the workgroup.
#include "int4_quant.h"

namespace hq {
namespace {

// The cache is written once here and read by later calls: every write is a
// streaming store (st_nt).

struct QuantParams {
    const uint16_t* k;
    const uint16_t* v;
    const int32_t* seq_lens;
    const int32_t* sel_idx;
    const int32_t* sel_count;
    const float* col_scores;
    const hq_thresh* thresh;
    hq_cache c;
    int32_t Tmax, sel_stride;
};

// Position of the n-th (0-based) non-selected token: n + #{i : S[i] - i <= n}.
__device__ inline int32_t nth_unselected(const int32_t* S, int32_t k, int32_t n) {
    int32_t lo = 0, hi = k;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (S[mid] - mid <= n) lo = mid + 1;
        else hi = mid;
    }
    return n + lo;
}

template <bool F16>
__global__ __launch_bounds__(256) void k_quantize(QuantParams p) {
    const int tid = threadIdx.x;
    const int g = blockIdx.y, b = blockIdx.z;
    const int Hkv = p.c.Hkv, W = p.c.window;
    const int bg = b * Hkv + g;
    const int T = p.seq_lens[b];
    const int32_t* S = p.sel_idx + (size_t)bg * p.sel_stride;
    int k = p.sel_count[bg];
    const int nwin = T < W ? T : W;
    const bool bad = k < 0 || k > p.c.cap_keep || k > p.sel_stride || k > T - nwin || T > p.Tmax || T < 1;
    if (bad) {
        if (tid == 0) atomicOr(p.c.err_flag, 1);
        return;
    }
    const int n_q = T - k - nwin;
    const QSpan qs = q_span(p.c, bg);
    if (n_q > qs.tiles * kTile) {  // the (b, g)'s INT4 capacity (ragged layout)
        if (tid == 0) atomicOr(p.c.err_flag, 1);
        return;
    }
    const int qt = p.c.cap_q / kTile, kt = p.c.cap_keep / kTile;
    int tile = blockIdx.x;
    const uint16_t* krows = p.k + (size_t)bg * p.Tmax * kD;
    const uint16_t* vrows = p.v + (size_t)bg * p.Tmax * kD;

    if (tile == 0 && tid == 0) {
        int4 cnt = {T, n_q, k, T};
        *reinterpret_cast<int4*>(p.c.counts + 4 * bg) = cnt;
        p.c.thresh[bg] = p.thresh[bg];
    }

    if (tile < qt) {
        // ---------------- INT4 tile
        // the probe scores of positions tile*64 + 64*qt*r + lane (cap_probe
        // may exceed cap_q by up to the window)
        if (tid < kTile) {
            for (int j = tile * kTile + tid; j < p.c.cap_probe; j += qt * kTile)
                p.c.col_scores[(size_t)bg * p.c.cap_probe + j] = j < T ? p.col_scores[(size_t)bg * p.Tmax + j] : 0.0f;
        }
        const int t = tid >> 2, grp = tid & 3;
        const int n = tile * kTile + t;
        const bool valid = n < n_q;
        if (tile * kTile >= n_q) return;  // uniform: whole tile empty
        const int pos = valid ? nth_unselected(S, k, n) : 0;
        float x[kGroup];
        uint32_t kp[4], vp[4], ks, kz, vs, vz;
        {
            const uint4* src = reinterpret_cast<const uint4*>(krows + (size_t)pos * kD + grp * kGroup);
#pragma unroll
            for (int i = 0; i < 4; ++i) unpack8<F16>(src[i], x + 8 * i);
            int4_quant_group(x, kp, ks, kz);
        }
        {
            const uint4* src = reinterpret_cast<const uint4*>(vrows + (size_t)pos * kD + grp * kGroup);
#pragma unroll
            for (int i = 0; i < 4; ++i) unpack8<F16>(src[i], x + 8 * i);
            int4_quant_group(x, vp, vs, vz);
        }
        // V words gather 8 slots of one channel: stage the canonical words in LDS
        __shared__ uint32_t vstage[kTile][4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) vstage[t][grp][i] = valid ? vp[i] : 0u;
        const size_t tile_base = ((size_t)qs.tile0 + tile) * kTileBytesQ;
        const size_t meta_base = ((size_t)qs.tile0 + tile) * (kTile * 16);
        uint8_t* kc = reinterpret_cast<uint8_t*>(p.c.k_codes) + tile_base;
        uint8_t* vc = reinterpret_cast<uint8_t*>(p.c.v_codes) + tile_base;
        if (valid) {
#pragma unroll
            for (int w = 0; w < 4; ++w)
                st_nt(kc + kq_word(t, kGroup * grp + 8 * w), to_mf_order(kp[w]));
            // (K metadata and positions: a quarter line per instruction, default policy)
            *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(p.c.k_meta) + meta_base + kmeta_word(t, grp)) =
                ks | (kz << 16);
            st_nt(reinterpret_cast<uint8_t*>(p.c.v_meta) + meta_base + vmeta_word(t, grp), (uint32_t)(vs | (vz << 16)));
            if (grp == 0) p.c.q_pos[(size_t)qs.tile0 * kTile + n] = pos;
        }
        __syncthreads();
        // 1024 V words per tile: word (channel ch, slot octet o) holds slots
        // 8o..8o+7. Thread tid assembles the four words of one 16-byte record
        // (channels ch, ch + 16 x octets o, o + 4), so each wave stores 1 KiB
        // of whole lines.
        {
            const int cb = tid >> 6, oq = (tid >> 4) & 3, c16 = tid & 15;
            uint32_t wd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ch = 32 * cb + 16 * (j >> 1) + c16, o = oq + 4 * (j & 1);
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t code = (vstage[8 * o + e][ch >> 5][(ch >> 3) & 3] >> (4 * (ch & 7))) & 0xFu;
                    w |= code << mf_nib(e);
                }
                wd[j] = w;
            }
            st_nt(vc + vq_word(8 * oq, 32 * cb + c16), make_uint4(wd[0], wd[1], wd[2], wd[3]));
        }
        return;
    }
    tile -= qt;
    // 16-bit tiles: item e = tid + 256 r (r < 4) is the 16 bytes at byte 16e
    // of the K tile and of the V tile, so each wave stores 1 KiB of whole
    // lines. K byte 16e holds slot e % 64, chunk e / 64 (k16_off); V byte 16e
    // holds slot e / 64 + 16 ((e / 16) % 4), chunk e % 16 (v16_off).
    auto k_slot = [](int e) { return e & 63; };
    auto k_chunk = [](int e) { return e >> 6; };
    auto v_slot = [](int e) { return (e >> 6) + 16 * ((e >> 4) & 3); };
    auto v_chunk = [](int e) { return e & 15; };
    if (tile < kt) {
        // ---------------- kept tile
        if (tile * kTile >= k) return;
        // position of slot s, or -1 past the count or for an invalid entry
        auto kept_pos = [&](int s) {
            const int i = tile * kTile + s;
            if (i >= k) return -1;
            const int pos = S[i];
            return (pos < 0 || pos >= T - nwin || (i > 0 && S[i - 1] >= pos)) ? -1 : pos;
        };
        if (tid < kTile) {
            const int i = tile * kTile + tid;
            if (i < k) {
                const int pos = kept_pos(tid);
                if (pos < 0) atomicOr(p.c.err_flag, 4);  // selected positions must be ascending candidates
                else p.c.keep_pos[(size_t)bg * p.c.cap_keep + i] = pos;
            }
        }
        const size_t tb = ((size_t)bg * kt + tile) * kTileBytes16;
        uint8_t* kd = reinterpret_cast<uint8_t*>(p.c.k_keep) + tb;
        uint8_t* vd = reinterpret_cast<uint8_t*>(p.c.v_keep) + tb;
        int kp[4], vp[4];
        uint4 kv[4], vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = tid + 256 * r;
            kp[r] = kept_pos(k_slot(e));
            vp[r] = kept_pos(v_slot(e));
            kv[r] = reinterpret_cast<const uint4*>(krows + (size_t)max(kp[r], 0) * kD)[k_chunk(e)];
            vv[r] = reinterpret_cast<const uint4*>(vrows + (size_t)max(vp[r], 0) * kD)[v_chunk(e)];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = tid + 256 * r;
            if (kp[r] >= 0) st_nt(kd + 16 * e, kv[r]);
            if (vp[r] >= 0) st_nt(vd + 16 * e, vv[r]);
        }
        return;
    }
    tile -= kt;
    {
        // ---------------- ring tile (slot = position % W)
        const size_t tb = ((size_t)bg * (W / kTile) + tile) * kTileBytes16;
        uint8_t* kd = reinterpret_cast<uint8_t*>(p.c.k_win) + tb;
        uint8_t* vd = reinterpret_cast<uint8_t*>(p.c.v_win) + tb;
        // position of ring slot s, or -1 for a slot no token has reached
        auto ring_pos = [&](int s) {
            const int slot = tile * kTile + s;
            if (T >= W) return T - 1 - ((T - 1 - slot) % W);
            return slot < T ? slot : -1;
        };
        int kp[4], vp[4];
        uint4 kv[4], vv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = tid + 256 * r;
            kp[r] = ring_pos(k_slot(e));
            vp[r] = ring_pos(v_slot(e));
            kv[r] = reinterpret_cast<const uint4*>(krows + (size_t)max(kp[r], 0) * kD)[k_chunk(e)];
            vv[r] = reinterpret_cast<const uint4*>(vrows + (size_t)max(vp[r], 0) * kD)[v_chunk(e)];
        }
        const uint4 zero = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = tid + 256 * r;
            st_nt(kd + 16 * e, kp[r] >= 0 ? kv[r] : zero);
            st_nt(vd + 16 * e, vp[r] >= 0 ? vv[r] : zero);
        }
    }
}

}  // namespace

hipError_t launch_quantize(const void* k, const void* v, const int32_t* seq_lens, int32_t Tmax,
                           const int32_t* sel_idx, const int32_t* sel_count, int32_t sel_stride_,
                           const float* col_scores, const hq_thresh* thresh, const hq_cache& c,
                           hipStream_t s) {
    QuantParams p;
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.seq_lens = seq_lens;
    p.sel_idx = sel_idx;
    p.sel_count = sel_count;
    p.col_scores = col_scores;
    p.thresh = thresh;
    p.c = c;
    p.Tmax = Tmax;
    p.sel_stride = sel_stride_;
    const int tiles = c.cap_q / kTile + c.cap_keep / kTile + c.window / kTile;
    dim3 grid(tiles, c.Hkv, c.B);
    if (c.dt == HQ_F16)
        k_quantize<true><<<grid, 256, 0, s>>>(p);
    else
        k_quantize<false><<<grid, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace hq
