// Internal declarations shared by the libhyquant translation units (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hq.h"

namespace hq {

constexpr int kD = 128;          // head_dim (the only supported value)
constexpr int kTile = 64;        // tokens per cache tile == wavefront size
constexpr int kGroup = 32;       // INT4 quantization group (channels)
constexpr int kTileBytesQ = 4096;        // packed INT4 codes of one tile (K or V)
constexpr int kTileBytes16 = kTile * kD * 2;  // one tile of 16-bit rows
// Cache-policy operand of the buffer loads that stream the INT4 store: the
// non-temporal hint (each byte is read once per call, so it is not kept in
// the caches at the expense of other data; measured faster than the default).
constexpr int kLoadNT = 2;

// Streaming (non-temporal) stores, for results that this call does not read
// back: they are not kept dirty in the caches, where their later write-back
// would take bandwidth from the kernels that run next.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline void st_nt(void* ptr, uint32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(ptr)); }
__device__ inline void st_nt(void* ptr, int32_t v) { __builtin_nontemporal_store(v, reinterpret_cast<int32_t*>(ptr)); }
__device__ inline void st_nt(void* ptr, uint32_t a, uint32_t b) {
    const u32x2_t x = {a, b};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(ptr));
}
__device__ inline void st_nt(void* ptr, const uint4& v) {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(ptr));
}
constexpr int kInt8Block = 64;   // prefill INT8 block (tokens)
constexpr int kRouteMaxT = 1 << 18;  // longest prefill with tile routing (4,096 key blocks sorted in LDS)
// Largest cache capacity in slots: the decode kernel addresses one (b, g)'s
// INT4 codes (64 bytes per slot) with 32-bit buffer offsets.
constexpr int32_t kMaxCapTokens = 1 << 24;

// ---------------------------------------------------------------------------
// INT4 tile layouts (per (b, g), tile of 64 slots). The decode kernel feeds
// the codes straight into 16x16x32 fp16 MFMA operands, so every 32-bit word
// holds the 8 codes of one operand lane: element e (0..7) of the lane's
// 8-element k-slice sits in the nibble at bit mf_nib(e) = 16*(e%2) + 4*(e/2),
// so that register k of the operand (elements 2k, 2k+1 in its low / high
// 16 bits) is the word's nibbles at bits (4(k/2)+..., 16+...) after at most
// one shift, and a single and-or turns them into fp16 "1024 + c" (nibble at
// bits 0..3 of a half) or "64 + c" (nibble at bits 4..7) values.
__host__ __device__ constexpr int mf_nib(int e) { return 16 * (e & 1) + 4 * (e >> 1); }

// K codes: slot t, channel c. Operand lane l = t%16 + 16*((c%32)/8) (token
// t%16 of 16-token block t/16, channel octet (c%32)/8), element c%8; the word
// of (block nb = t/16, group c/32) is at byte nb*1024 + l*16 + (c/32)*4.
__host__ __device__ inline int kq_word(int slot, int ch) {
    return (slot >> 4) * 1024 + ((slot & 15) + 16 * ((ch >> 3) & 3)) * 16 + (ch >> 5) * 4;
}
// V codes: slot t, channel c. Operand lane l = c%16 + 16*((t%32)/8) (channel
// c%16 of 16-channel block c/16, token octet (t%32)/8 of token half t/32),
// element t%8; the word of (channel block mb = c/16, token half ks = t/32) is
// at byte (mb/2)*1024 + l*16 + ((mb%2)*2 + ks)*4.
__host__ __device__ inline int vq_word(int slot, int ch) {
    return (ch >> 5) * 1024 + ((ch & 15) + 16 * ((slot >> 3) & 3)) * 16 + ((((ch >> 4) & 1) << 1) | (slot >> 5)) * 4;
}
// K scale/zero (fp16 pair, one dword) of slot t, group j inside the tile's
// 1024-byte metadata block: byte (t%16 + 16*j)*16 + (t/16)*4, so lane
// l = t%16 + 16j reads the four 16-token blocks with one 16-byte load.
__host__ __device__ inline int kmeta_word(int slot, int group) {
    return ((slot & 15) + 16 * group) * 16 + (slot >> 4) * 4;
}
// V scale/zero: slot t, group j at byte t*16 + j*4 (one 16-byte record per slot).
__host__ __device__ inline int vmeta_word(int slot, int group) { return slot * 16 + group * 4; }

// Canonical packed word (nibble n = channel/slot 8w+n at bits 4n) -> the
// operand nibble order above.
__host__ __device__ inline uint32_t to_mf_order(uint32_t w) {
    uint32_t r = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) r |= ((w >> (4 * n)) & 0xFu) << mf_nib(n);
    return r;
}

// 16-bit tiles. K (token phase): 16-byte chunk c (channels 8c..8c+7) of slot
// t at c*1024 + t*16. V (channel phase): chunk c8 of slot t = 16u + i at
// i*1024 + (16u + c8)*16.
__host__ __device__ inline int k16_off(int slot, int chunk) { return chunk * 1024 + slot * 16; }
__host__ __device__ inline int v16_off(int slot, int chunk) {
    return (slot & 15) * 1024 + (16 * (slot >> 4) + chunk) * 16;
}

// INT4 store of one (b, g): its first tile in the pools and its capacity in
// tiles. Uniform layout: tiles [bg cap_q/64, (bg + 1) cap_q/64). Ragged
// layout: the span q_tile_off[bg] .. q_tile_off[bg + 1], empty if it is not
// ascending, leaves [0, q_tiles_total) or exceeds cap_q/64 tiles.
struct QSpan {
    int64_t tile0;
    int32_t tiles;
};
__host__ __device__ inline QSpan q_span(const hq_cache& c, int bg) {
    const int32_t qt = c.cap_q / kTile;
    if (c.q_tile_off == nullptr) return {(int64_t)bg * qt, qt};
    const int64_t a = c.q_tile_off[bg], b = c.q_tile_off[bg + 1];
    if (a < 0 || b < a || b > c.q_tiles_total || b - a > qt) return {0, 0};
    return {a, (int32_t)(b - a)};
}

// Device-side counters of one (b, g).
struct Counts {
    int32_t seq_len, n_q, n_keep, probe_len;
};

// ---------------------------------------------------------------------------
// Scalar conversions.
__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ inline float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ inline uint32_t f32_to_f16_bits(float x) {  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
template <bool F16>
__device__ inline float h16_to_f32(uint32_t bits16) {
    if constexpr (F16) return f16_to_f32(bits16);
    else return bf16_to_f32(bits16);
}

// ---------------------------------------------------------------------------
// Wavefront reductions (wave64).
__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ inline double wave_sum_d(double v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ inline double wave_max_d(double v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v = fmax(v, __shfl_xor(v, o));
    return v;
}

// ---------------------------------------------------------------------------
// Policy helpers (host and device).
__host__ __device__ inline int32_t keep_count(int32_t T, const hq_policy& p) {
    int32_t n_cand = T > p.window ? T - p.window : 0;
    int64_t k = (int64_t)p.keep_num * T / p.keep_den;
    return (int32_t)(k < n_cand ? k : n_cand);
}
inline int32_t sel_stride(int32_t T, const hq_policy& p) {
    int64_t k = (int64_t)p.keep_num * T / p.keep_den;
    return (int32_t)(k > 1 ? k : 1);
}
inline int32_t round_up(int32_t x, int32_t m) { return (x + m - 1) / m * m; }

// ---------------------------------------------------------------------------
// Launchers (each defined next to its kernels). Return hipSuccess or the
// launch error.
hipError_t launch_quantize(const void* k, const void* v, const int32_t* seq_lens, int32_t Tmax,
                           const int32_t* sel_idx, const int32_t* sel_count, int32_t sel_stride,
                           const float* col_scores, const hq_thresh* thresh, const hq_cache& c,
                           hipStream_t s);
hipError_t launch_append(const hq_cache& c, const void* k_new, const void* v_new, hipStream_t s);

struct DecodeLaunch {
    int32_t Hq, G, nsplit, tiles_per_split;
    float sm_scale_log2;
    void* ws;
};
hipError_t launch_decode(const hq_cache& c, const void* q, void* out, hq_dtype out_dt,
                         const DecodeLaunch& d, hipStream_t s);
size_t decode_ws_bytes(const hq_cache& c, int32_t Hq, int32_t nsplit);
// hq_decode_attn_noalloc: the static scratch array (HQ_DECODE_NOALLOC_SCRATCH_BYTES)
// that replaces the workspace; *out = its address on the current device
// (looked up once per device, never allocated).
constexpr size_t kDecodeScratchBytes = HQ_DECODE_NOALLOC_SCRATCH_BYTES;
hipError_t decode_scratch(void** out);
int32_t decode_nsplit(const hq_cache& c, int32_t tps);
int32_t decode_nsq(const hq_cache& c, int32_t tps);  // INT4 splits of a (b, g)

// Streaming read of the INT4 store in the decode kernel's access pattern
// (measurement helper, not a step of the method).
size_t diag_sink_bytes(const hq_cache& c, int32_t tps);
hipError_t launch_diag_read_int4(const hq_cache& c, void* sink, int32_t tps, hipStream_t s);
hipError_t launch_diag_exp2_error(int32_t k0, int64_t n, double* out, int nblocks, hipStream_t s);

// Shapes the probe kernels support: G query heads per KV head times
// probe_rows rows. probe_shape_rule() states the rule for error messages.
bool probe_shape_supported(int32_t G, int32_t probe_rows);
const char* probe_shape_rule();
hipError_t launch_probe(const void* q_probe, const void* k, const int32_t* seq_lens, int32_t B,
                        int32_t Hq, int32_t Hkv, int32_t Tmax, bool f16, const hq_policy& pol,
                        float sm_scale, float* col_scores, int32_t* sel_idx, int32_t* sel_count,
                        hq_thresh* thresh, void* ws, hipStream_t s);
size_t probe_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, const hq_policy& pol);

// Re-probe of a hybrid cache: positions the probe covers (every slot of the
// three stores), workspace bytes, and the launch (expand, probe, persistence).
int32_t reprobe_tcap(const hq_cache& c);
size_t reprobe_ws_bytes(const hq_cache& c, int32_t Hq, const hq_policy& pol);
hipError_t launch_reprobe(const hq_cache& c, const void* q_recent, int32_t Hq, const hq_policy& pol,
                          float sm_scale, float* col_scores, int32_t* sel_idx, int32_t* sel_count,
                          hq_thresh* thresh, int32_t* n_persist, void* ws, hipStream_t s);

hipError_t launch_prefill(const void* q, const void* k, const void* v, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t T, bool f16, const hq_policy& pol,
                          const int32_t* sel_idx, const int32_t* sel_count, int32_t sel_stride,
                          float sm_scale, void* out, hq_dtype out_dt, void* ws, hipStream_t s);
size_t prefill_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, const hq_policy& pol);

}  // namespace hq
