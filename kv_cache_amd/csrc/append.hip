// hq_append_kv: one decode-time append per (b, g) (gfx950).
//
// HyQuant pages: "HyQuant: Hybrid-Precision Quantization for LLM
// Attention", flowchart (the recent local sliding window stays in high
// precision); "How HyQuant uses hybrid-precision attention to cut decode
// compute", "What hybrid-precision attention changes" (during decode most of
// the cache is low-bit, selected positions stay high precision).
//
// The new token at position T enters ring slot T % W. The token leaving the
// window, d = T - W, sits in that same slot; it is staged in LDS first, then
// copied to the kept store when it was probed and its probe score ranks
// above the k-th selected candidate, and INT4-quantized into the next INT4
// slot otherwise. Launch-latency bound: one 64-lane workgroup per (b, g).
#include "int4_quant.h"

namespace hq {
namespace {

template <bool F16>
__global__ __launch_bounds__(64) void k_append(hq_cache c, const uint16_t* k_new, const uint16_t* v_new) {
    __shared__ uint4 stage_k[16], stage_v[16];
    const int lane = threadIdx.x;
    const int g = blockIdx.x, b = blockIdx.y;
    const int bg = b * c.Hkv + g;
    const int W = c.window;
    const int4 cnt = *reinterpret_cast<const int4*>(c.counts + 4 * bg);
    const int T = cnt.x;
    int n_q = cnt.y, n_keep = cnt.z;
    const int probe_len = cnt.w;

    // the departing token (or, with no window, the new token itself)
    bool depart = false;
    int d = -1;
    if (W == 0) {
        depart = true;
        d = T;
        if (lane < 16) {
            stage_k[lane] = reinterpret_cast<const uint4*>(k_new + (size_t)bg * kD)[lane];
            stage_v[lane] = reinterpret_cast<const uint4*>(v_new + (size_t)bg * kD)[lane];
        }
    } else if (T >= W) {
        depart = true;
        d = T - W;
        const int slot = T % W, tile = slot / kTile, ts = slot % kTile;
        const uint8_t* kt = reinterpret_cast<const uint8_t*>(c.k_win) + ((size_t)bg * (W / kTile) + tile) * kTileBytes16;
        const uint8_t* vt = reinterpret_cast<const uint8_t*>(c.v_win) + ((size_t)bg * (W / kTile) + tile) * kTileBytes16;
        if (lane < 16) {
            stage_k[lane] = *reinterpret_cast<const uint4*>(kt + k16_off(ts, lane));
            stage_v[lane] = *reinterpret_cast<const uint4*>(vt + v16_off(ts, lane));
        }
    }
    __syncthreads();

    bool to_keep = false;
    if (depart && d < probe_len) {
        const float cd = c.col_scores[(size_t)bg * c.cap_probe + d];
        const hq_thresh th = c.thresh[bg];
        to_keep = (cd > th.tau) || (cd == th.tau && d < th.j_k);
    }
    bool overflow = false;
    if (depart) {
        if (to_keep) {
            overflow = n_keep >= c.cap_keep;
            if (!overflow) {
                const int i = n_keep, tile = i / kTile, ts = i % kTile;
                const size_t tb = ((size_t)bg * (c.cap_keep / kTile) + tile) * kTileBytes16;
                if (lane < 16) {
                    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(c.k_keep) + tb + k16_off(ts, lane)) = stage_k[lane];
                    *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(c.v_keep) + tb + v16_off(ts, lane)) = stage_v[lane];
                }
                if (lane == 0) c.keep_pos[(size_t)bg * c.cap_keep + i] = d;
                n_keep += 1;
            }
        } else {
            const QSpan qs = q_span(c, bg);
            overflow = n_q >= qs.tiles * kTile;
            if (!overflow) {
                const int n = n_q, tile = n / kTile, ts = n % kTile;
                const size_t tb = ((size_t)qs.tile0 + tile) * kTileBytesQ;
                const size_t mb = ((size_t)qs.tile0 + tile) * (kTile * 16);
                __shared__ uint32_t vwords[4][4];  // canonical V words of the departing token
                if (lane < 8) {
                    const bool isv = lane >= 4;
                    const int grp = lane & 3;
                    const uint4* src = isv ? stage_v : stage_k;
                    float x[kGroup];
#pragma unroll
                    for (int i = 0; i < 4; ++i) unpack8<F16>(src[4 * grp + i], x + 8 * i);
                    uint32_t pk[4], sb, zb;
                    int4_quant_group(x, pk, sb, zb);
                    if (!isv) {
                        uint8_t* kc = reinterpret_cast<uint8_t*>(c.k_codes) + tb;
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            *reinterpret_cast<uint32_t*>(kc + kq_word(ts, kGroup * grp + 8 * w)) = to_mf_order(pk[w]);
                        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(c.k_meta) + mb + kmeta_word(ts, grp)) =
                            sb | (zb << 16);
                    } else {
#pragma unroll
                        for (int w = 0; w < 4; ++w) vwords[grp][w] = pk[w];
                        *reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(c.v_meta) + mb + vmeta_word(ts, grp)) =
                            sb | (zb << 16);
                    }
                }
                __syncthreads();
                // each V word holds 8 slots of one channel: replace this slot's nibble
                uint8_t* vc = reinterpret_cast<uint8_t*>(c.v_codes) + tb;
                const int sh = mf_nib(ts & 7);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int ch = lane + 64 * i;
                    const uint32_t code = (vwords[ch >> 5][(ch >> 3) & 3] >> (4 * (ch & 7))) & 0xFu;
                    uint32_t* wp = reinterpret_cast<uint32_t*>(vc + vq_word(ts, ch));
                    *wp = (*wp & ~(0xFu << sh)) | (code << sh);
                }
                if (lane == 0) c.q_pos[(size_t)qs.tile0 * kTile + n] = d;
                n_q += 1;
            }
        }
    }
    if (overflow) {
        if (lane == 0) atomicOr(c.err_flag, 2);
        return;  // leave the cache unchanged
    }
    if (W > 0) {
        const int slot = T % W, tile = slot / kTile, ts = slot % kTile;
        const size_t tb = ((size_t)bg * (W / kTile) + tile) * kTileBytes16;
        if (lane < 16) {
            *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(c.k_win) + tb + k16_off(ts, lane)) =
                reinterpret_cast<const uint4*>(k_new + (size_t)bg * kD)[lane];
            *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(c.v_win) + tb + v16_off(ts, lane)) =
                reinterpret_cast<const uint4*>(v_new + (size_t)bg * kD)[lane];
        }
    }
    if (lane == 0) {
        int4 out = {T + 1, n_q, n_keep, probe_len};
        *reinterpret_cast<int4*>(c.counts + 4 * bg) = out;
    }
}

}  // namespace

hipError_t launch_append(const hq_cache& c, const void* k_new, const void* v_new, hipStream_t s) {
    dim3 grid(c.Hkv, c.B);
    if (c.dt == HQ_F16)
        k_append<true><<<grid, 64, 0, s>>>(c, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new));
    else
        k_append<false><<<grid, 64, 0, s>>>(c, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new));
    return hipGetLastError();
}

}  // namespace hq
