// Host side of libhyquant: argument validation, sizing and launches.
// Every check runs before anything is enqueued; on error nothing is launched.
#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "hq_internal.h"
#include "../../include/hq_diag.h"

namespace {

thread_local char g_err[512] = "";

hq_status fail(hq_status code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}
void clear_err() { g_err[0] = '\0'; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQ_PTR(p)                                                                           \
    do {                                                                                     \
        if ((p) == nullptr) return fail(HQ_ERR_INVALID_ARG, "%s: %s is null", fn, #p);        \
        if (!aligned16(p)) return fail(HQ_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
    } while (0)

hq_status check_policy(const char* fn, const hq_policy* p) {
    if (!p) return fail(HQ_ERR_INVALID_ARG, "%s: policy is null", fn);
    if (p->keep_den <= 0 || p->keep_num < 0 || p->keep_num > p->keep_den)
        return fail(HQ_ERR_INVALID_ARG, "%s: retained fraction %d/%d must satisfy 0 <= num <= den, den > 0", fn,
                    p->keep_num, p->keep_den);
    if (p->window < 0 || p->window % hq::kTile != 0 || p->window > (1 << 20))
        return fail(HQ_ERR_INVALID_ARG, "%s: window %d must be a non-negative multiple of 64", fn, p->window);
    if (p->probe_rows < 1 || p->probe_rows > 256)
        return fail(HQ_ERR_INVALID_ARG, "%s: probe_rows %d must be in [1, 256]", fn, p->probe_rows);
    if (p->low_fmt != HQ_LOW_INT8 && p->low_fmt != HQ_LOW_FP8)
        return fail(HQ_ERR_UNSUPPORTED, "%s: low_fmt %d unsupported (HQ_LOW_INT8, HQ_LOW_FP8)", fn, p->low_fmt);
    if (p->tile_num < 0 || (p->tile_num > 0 && (p->tile_den <= 0 || p->tile_num > p->tile_den)))
        return fail(HQ_ERR_INVALID_ARG, "%s: tile fraction %d/%d must satisfy 0 <= num <= den, den > 0", fn,
                    p->tile_num, p->tile_den);
    if (p->tile_num > 0 && p->low_fmt != HQ_LOW_INT8)
        return fail(HQ_ERR_UNSUPPORTED, "%s: tile routing needs the INT8 low-precision path", fn);
    return HQ_OK;
}

hq_status check_heads(const char* fn, int32_t B, int32_t Hq, int32_t Hkv, int32_t D) {
    if (B < 1 || Hq < 1 || Hkv < 1) return fail(HQ_ERR_INVALID_ARG, "%s: B, Hq, Hkv must be >= 1", fn);
    if (D != hq::kD) return fail(HQ_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (only 128)", fn, D);
    if (Hq % Hkv != 0) return fail(HQ_ERR_UNSUPPORTED, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
    const int G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(HQ_ERR_UNSUPPORTED, "%s: query heads per KV head %d unsupported (1, 2, 4, 8)", fn, G);
    return HQ_OK;
}

hq_status check_dt(const char* fn, int dt) {
    if (dt != HQ_BF16 && dt != HQ_F16) return fail(HQ_ERR_UNSUPPORTED, "%s: dtype %d unsupported (bf16, f16)", fn, dt);
    return HQ_OK;
}

hq_status check_cache(const char* fn, const hq_cache* c) {
    if (!c) return fail(HQ_ERR_INVALID_ARG, "%s: cache is null", fn);
    if (c->B < 1 || c->Hkv < 1) return fail(HQ_ERR_INVALID_ARG, "%s: cache B/Hkv must be >= 1", fn);
    if (c->D != hq::kD) return fail(HQ_ERR_UNSUPPORTED, "%s: cache head_dim %d unsupported", fn, c->D);
    hq_status st = check_dt(fn, c->dt);
    if (st) return st;
    if (c->window < 0 || c->window % hq::kTile)
        return fail(HQ_ERR_INVALID_ARG, "%s: cache window %d must be a multiple of 64", fn, c->window);
    if (c->cap_q < hq::kTile || c->cap_q % hq::kTile || c->cap_keep < hq::kTile || c->cap_keep % hq::kTile)
        return fail(HQ_ERR_INVALID_ARG, "%s: cache capacities must be positive multiples of 64", fn);
    if (c->cap_q > hq::kMaxCapTokens || c->cap_keep > hq::kMaxCapTokens)
        return fail(HQ_ERR_CAPACITY, "%s: cache capacities %d / %d exceed %d slots (32-bit byte offsets)", fn,
                    c->cap_q, c->cap_keep, hq::kMaxCapTokens);
    if (c->cap_probe < 1 || c->cap_probe > c->cap_q + c->window)
        return fail(HQ_ERR_INVALID_ARG, "%s: cap_probe %d must be in [1, cap_q + window]", fn, c->cap_probe);
    REQ_PTR(c->k_codes);
    REQ_PTR(c->v_codes);
    REQ_PTR(c->k_meta);
    REQ_PTR(c->v_meta);
    REQ_PTR(c->k_keep);
    REQ_PTR(c->v_keep);
    if (c->window > 0) {
        REQ_PTR(c->k_win);
        REQ_PTR(c->v_win);
    }
    REQ_PTR(c->q_pos);
    REQ_PTR(c->keep_pos);
    REQ_PTR(c->counts);
    REQ_PTR(c->col_scores);
    REQ_PTR(c->thresh);
    if (c->err_flag == nullptr) return fail(HQ_ERR_INVALID_ARG, "%s: cache err_flag is null", fn);
    if (c->q_tile_off != nullptr) {
        REQ_PTR(c->q_tile_off);
        if (c->q_tiles_total < 1)
            return fail(HQ_ERR_INVALID_ARG, "%s: ragged layout needs q_tiles_total >= 1", fn);
    }
    return HQ_OK;
}

hq_status hip_fail(const char* fn, hipError_t e) {
    return fail(HQ_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
}

// Compute units of the current device (cached per device; 0 if unknown).
int32_t device_cus() {
    static std::atomic<int32_t> cached[64];  // zero-initialised (static storage)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int32_t c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    if (dev < 64 && n > 0) cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

// INT4 cache tiles per decode split. Start from 54 tiles per split and add
// splits until the grid fills whole rounds of the device's workgroup slots
// (two per CU): a partial last round leaves CUs idle at the end of the
// kernel. At least 4 tiles (one per wave) per split.
int32_t decode_tps(const hq_cache& c, int32_t G) {
    const int32_t tiles = c.cap_q / hq::kTile;
    if (tiles < 1) return 54;
    const int32_t base = (tiles + 53) / 54;
    const int32_t n16 = hq::decode_nsplit(c, 54) - base;
    // eight heads per KV head run as two four-head workgroups per split
    const int64_t bg = (int64_t)c.B * c.Hkv * (G > 4 ? 2 : 1);
    const int64_t slots = 2 * (int64_t)device_cus();
    if (slots <= 0 || bg <= 0) return 54;
    const int64_t total = (base + n16) * bg;
    const int64_t rounds = (total + slots - 1) / slots;
    const int64_t nsq = std::max<int64_t>(base, rounds * slots / bg - n16);
    return std::max<int32_t>(4, (int32_t)((tiles + nsq - 1) / nsq));  // at least one tile per wave
}

}  // namespace

extern "C" {

const char* hq_last_error(void) { return g_err; }

int32_t hq_sel_stride(int32_t T, const hq_policy* policy) {
    if (!policy || policy->keep_den <= 0 || T < 0) return 1;
    return hq::sel_stride(T, *policy);
}

hq_status hq_cache_layout(int32_t B, int32_t Hkv, int32_t D, int32_t cap_tokens, int32_t cap_probe, int32_t dt,
                          const hq_policy* policy, hq_cache_sizes* out) {
    static const char* fn = "hq_cache_layout";
    clear_err();
    hq_status st = check_policy(fn, policy);
    if (st) return st;
    if (!out) return fail(HQ_ERR_INVALID_ARG, "%s: out is null", fn);
    if (B < 1 || Hkv < 1) return fail(HQ_ERR_INVALID_ARG, "%s: B and Hkv must be >= 1", fn);
    if (D != hq::kD) return fail(HQ_ERR_UNSUPPORTED, "%s: head_dim %d unsupported (only 128)", fn, D);
    if ((st = check_dt(fn, dt))) return st;
    if (cap_tokens < 1) return fail(HQ_ERR_INVALID_ARG, "%s: cap_tokens %d out of range", fn, cap_tokens);
    if (cap_tokens > hq::kMaxCapTokens)
        return fail(HQ_ERR_CAPACITY, "%s: cap_tokens %d exceeds %d (32-bit byte offsets of the INT4 store)", fn,
                    cap_tokens, hq::kMaxCapTokens);
    if (cap_probe < 1 || cap_probe > cap_tokens)
        return fail(HQ_ERR_INVALID_ARG, "%s: cap_probe %d must be in [1, cap_tokens]", fn, cap_probe);
    const int32_t kmax = hq::keep_count(cap_probe, *policy);
    const int32_t w = policy->window < cap_probe ? policy->window : cap_probe;
    // INT4 store: every token outside the window can land there. The top-k
    // count is not subtracted: a shorter sequence of a ragged batch keeps
    // fewer columns and may be appended up to cap_tokens.
    const int32_t wq = policy->window < cap_tokens ? policy->window : cap_tokens;
    out->cap_q = std::max(hq::kTile, hq::round_up(cap_tokens - wq, hq::kTile));
    // kept store: the k selected columns plus, during appends, departures
    // flagged by the probe scores; those were window positions at probe
    // time, so at most w of them.
    int32_t ck = hq::round_up(kmax + w, hq::kTile);
    out->cap_keep = ck < hq::kTile ? hq::kTile : ck;
    out->cap_probe = cap_probe;
    const size_t BG = (size_t)B * Hkv;
    out->k_codes = out->v_codes = BG * (size_t)out->cap_q / 2 * hq::kD;  // 64 B per token
    out->k_meta = out->v_meta = BG * (size_t)out->cap_q * 16;
    out->k_keep = out->v_keep = BG * (size_t)out->cap_keep * hq::kD * 2;
    out->k_win = out->v_win = BG * (size_t)policy->window * hq::kD * 2;
    out->q_pos = BG * (size_t)out->cap_q * 4;
    out->keep_pos = BG * (size_t)out->cap_keep * 4;
    out->counts = BG * 16;
    out->col_scores = BG * (size_t)cap_probe * 4;
    out->thresh = BG * sizeof(hq_thresh);
    out->err_flag = 4;
    return HQ_OK;
}

hq_status hq_cache_layout_ragged(int32_t B, int32_t Hkv, int32_t D, const int32_t* cap_tokens, int32_t cap_probe,
                                 int32_t dt, const hq_policy* policy, int64_t* q_tile_off, hq_cache_sizes* out) {
    static const char* fn = "hq_cache_layout_ragged";
    clear_err();
    hq_status st = check_policy(fn, policy);
    if (st) return st;
    if (!out || !cap_tokens || !q_tile_off) return fail(HQ_ERR_INVALID_ARG, "%s: null argument", fn);
    if (B < 1 || Hkv < 1) return fail(HQ_ERR_INVALID_ARG, "%s: B and Hkv must be >= 1", fn);
    int32_t cmax = 0;
    for (int32_t b = 0; b < B; ++b) {
        if (cap_tokens[b] < 1) return fail(HQ_ERR_INVALID_ARG, "%s: cap_tokens[%d] = %d out of range", fn, b, cap_tokens[b]);
        if (cap_tokens[b] > hq::kMaxCapTokens)
            return fail(HQ_ERR_CAPACITY, "%s: cap_tokens[%d] = %d exceeds %d", fn, b, cap_tokens[b], hq::kMaxCapTokens);
        cmax = std::max(cmax, cap_tokens[b]);
    }
    // every buffer but the INT4 pools as for the uniform layout of the longest
    // sequence (or of the probe's positions, when the prompts were probed
    // padded to a longer length than any sequence's capacity)
    if (cap_probe < 1) return fail(HQ_ERR_INVALID_ARG, "%s: cap_probe %d out of range", fn, cap_probe);
    if ((st = hq_cache_layout(B, Hkv, D, std::max(cmax, cap_probe), cap_probe, dt, policy, out))) return st;
    int64_t off = 0;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t wq = std::min(policy->window, cap_tokens[b]);
        const int64_t tiles = std::max(hq::kTile, hq::round_up(cap_tokens[b] - wq, hq::kTile)) / hq::kTile;
        for (int32_t g = 0; g < Hkv; ++g) {
            q_tile_off[(size_t)b * Hkv + g] = off;
            off += tiles;
        }
    }
    q_tile_off[(size_t)B * Hkv] = off;
    out->k_codes = out->v_codes = (size_t)off * hq::kTileBytesQ;
    out->k_meta = out->v_meta = (size_t)off * 1024;
    out->q_pos = (size_t)off * hq::kTile * 4;
    return HQ_OK;
}

size_t hq_probe_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, int32_t D, const hq_policy* policy) {
    if (!policy || B < 1 || Hq < 1 || Hkv < 1 || Tmax < 1 || D != hq::kD || Hq % Hkv) return 0;
    if (!hq::probe_shape_supported(Hq / Hkv, policy->probe_rows)) return 0;
    return hq::probe_ws_bytes(B, Hq, Hkv, Tmax, *policy);
}

hq_status hq_probe_select(const void* q_probe, const void* k, const int32_t* seq_lens, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t Tmax, int32_t D, int32_t dt, const hq_policy* policy,
                          float sm_scale, float* col_scores, int32_t* sel_idx, int32_t* sel_count,
                          hq_thresh* thresh, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "hq_probe_select";
    clear_err();
    hq_status st;
    if ((st = check_policy(fn, policy))) return st;
    if ((st = check_heads(fn, B, Hq, Hkv, D))) return st;
    if ((st = check_dt(fn, dt))) return st;
    if (Tmax < 1 || Tmax > (1 << 24)) return fail(HQ_ERR_INVALID_ARG, "%s: Tmax %d out of range", fn, Tmax);
    if (!(sm_scale > 0.0f) || sm_scale > 1e6f) return fail(HQ_ERR_INVALID_ARG, "%s: sm_scale must be positive", fn);
    if (!hq::probe_shape_supported(Hq / Hkv, policy->probe_rows))
        return fail(HQ_ERR_UNSUPPORTED, "%s: %s (query heads per KV head %d, probe_rows %d)", fn,
                    hq::probe_shape_rule(), Hq / Hkv, policy->probe_rows);
    REQ_PTR(q_probe);
    REQ_PTR(k);
    REQ_PTR(seq_lens);
    REQ_PTR(col_scores);
    REQ_PTR(sel_idx);
    REQ_PTR(sel_count);
    REQ_PTR(thresh);
    const size_t need = hq::probe_ws_bytes(B, Hq, Hkv, Tmax, *policy);
    if (need > 0) REQ_PTR(ws);
    if (ws_bytes < need)
        return fail(HQ_ERR_CAPACITY, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    hipError_t e = hq::launch_probe(q_probe, k, seq_lens, B, Hq, Hkv, Tmax, dt == HQ_F16, *policy, sm_scale,
                                    col_scores, sel_idx, sel_count, thresh, ws, (hipStream_t)stream);
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

hq_status hq_quantize_kv(const void* k, const void* v, const int32_t* seq_lens, int32_t Tmax, const int32_t* sel_idx,
                         const int32_t* sel_count, const float* col_scores, const hq_thresh* thresh,
                         const hq_policy* policy, const hq_cache* cache, void* stream) {
    static const char* fn = "hq_quantize_kv";
    clear_err();
    hq_status st;
    if ((st = check_policy(fn, policy))) return st;
    if ((st = check_cache(fn, cache))) return st;
    if (policy->window != cache->window)
        return fail(HQ_ERR_INVALID_ARG, "%s: policy window %d != cache window %d", fn, policy->window, cache->window);
    if (Tmax < 1 || Tmax > cache->cap_probe)
        return fail(HQ_ERR_CAPACITY, "%s: Tmax %d exceeds the cache capacity (cap_probe %d)", fn, Tmax,
                    cache->cap_probe);
    if (hq::keep_count(Tmax, *policy) > cache->cap_keep)
        return fail(HQ_ERR_CAPACITY, "%s: kept store capacity %d < %d", fn, cache->cap_keep,
                    hq::keep_count(Tmax, *policy));
    REQ_PTR(k);
    REQ_PTR(v);
    REQ_PTR(seq_lens);
    REQ_PTR(sel_idx);
    REQ_PTR(sel_count);
    REQ_PTR(col_scores);
    REQ_PTR(thresh);
    hipError_t e = hq::launch_quantize(k, v, seq_lens, Tmax, sel_idx, sel_count, hq::sel_stride(Tmax, *policy),
                                       col_scores, thresh, *cache, (hipStream_t)stream);
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

hq_status hq_append_kv(const hq_cache* cache, const void* k_new, const void* v_new, void* stream) {
    static const char* fn = "hq_append_kv";
    clear_err();
    hq_status st;
    if ((st = check_cache(fn, cache))) return st;
    REQ_PTR(k_new);
    REQ_PTR(v_new);
    hipError_t e = hq::launch_append(*cache, k_new, v_new, (hipStream_t)stream);
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

size_t hq_decode_ws_bytes(const hq_cache* cache, int32_t Hq) {
    if (!cache || cache->Hkv < 1 || Hq < 1 || Hq % cache->Hkv) return 0;
    const int32_t tps = decode_tps(*cache, Hq / cache->Hkv);
    const int32_t nsplit = hq::decode_nsplit(*cache, tps);
    return hq::decode_ws_bytes(*cache, Hq, nsplit);
}

}  // extern "C"

namespace {

// Shared by hq_decode_attn (caller's workspace) and hq_decode_attn_noalloc
// (ws == nullptr: the library's static scratch array).
hq_status decode_call(const char* fn, const hq_cache* cache, const void* q, int32_t Hq, float sm_scale,
                      void* out, int32_t out_dt, void* ws, size_t ws_bytes, void* stream) {
    clear_err();
    hq_status st;
    if ((st = check_cache(fn, cache))) return st;
    if ((st = check_heads(fn, cache->B, Hq, cache->Hkv, cache->D))) return st;
    if (out_dt != HQ_F32 && out_dt != HQ_BF16 && out_dt != HQ_F16)
        return fail(HQ_ERR_UNSUPPORTED, "%s: out dtype %d unsupported", fn, out_dt);
    if (!(sm_scale > 0.0f) || sm_scale > 1e6f) return fail(HQ_ERR_INVALID_ARG, "%s: sm_scale must be positive", fn);
    REQ_PTR(q);
    REQ_PTR(out);
    const bool own_ws = ws != nullptr || ws_bytes != (size_t)-1;
    if (own_ws) REQ_PTR(ws);
    hq::DecodeLaunch d;
    d.Hq = Hq;
    d.G = Hq / cache->Hkv;
    d.tiles_per_split = decode_tps(*cache, d.G);
    d.nsplit = hq::decode_nsplit(*cache, d.tiles_per_split);
    d.sm_scale_log2 = sm_scale * 1.4426950408889634f;
    const size_t need = hq::decode_ws_bytes(*cache, Hq, d.nsplit);
    if (own_ws) {
        if (ws_bytes < need)
            return fail(HQ_ERR_CAPACITY, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
        d.ws = ws;
    } else {
        if (need > hq::kDecodeScratchBytes)
            return fail(HQ_ERR_CAPACITY, "%s: this cache needs %zu bytes of split partials, more than the %zu-byte "
                        "static scratch holds (use hq_decode_attn with a workspace)", fn, need,
                        hq::kDecodeScratchBytes);
        hipError_t e = hq::decode_scratch(&d.ws);
        if (e != hipSuccess) return fail(HQ_ERR_HIP, "%s: scratch lookup failed: %s", fn, hipGetErrorString(e));
    }
    hipError_t e = hq::launch_decode(*cache, q, out, (hq_dtype)out_dt, d, (hipStream_t)stream);  // validated above
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

}  // namespace

extern "C" {

hq_status hq_decode_attn(const hq_cache* cache, const void* q, int32_t Hq, float sm_scale, void* out,
                         int32_t out_dt, void* ws, size_t ws_bytes, void* stream) {
    if (ws == nullptr) {
        clear_err();
        return fail(HQ_ERR_INVALID_ARG, "hq_decode_attn: ws is null");
    }
    return decode_call("hq_decode_attn", cache, q, Hq, sm_scale, out, out_dt, ws, ws_bytes, stream);
}

hq_status hq_decode_attn_noalloc(const hq_cache* cache, const void* q, int32_t Hq, float sm_scale, void* out,
                                 int32_t out_dt, void* stream) {
    return decode_call("hq_decode_attn_noalloc", cache, q, Hq, sm_scale, out, out_dt, nullptr, (size_t)-1,
                       stream);
}

size_t hq_reprobe_ws_bytes(const hq_cache* cache, int32_t Hq, const hq_policy* policy) {
    if (!cache || !policy || cache->B < 1 || cache->Hkv < 1 || Hq < 1 || Hq % cache->Hkv) return 0;
    if (cache->cap_q < hq::kTile || cache->cap_keep < hq::kTile || cache->window < 0) return 0;
    if ((int64_t)cache->cap_q + cache->cap_keep + cache->window > (1 << 24)) return 0;
    if (!hq::probe_shape_supported(Hq / cache->Hkv, policy->probe_rows)) return 0;
    return hq::reprobe_ws_bytes(*cache, Hq, *policy);
}

hq_status hq_reprobe(const hq_cache* cache, const void* q_recent, int32_t Hq, const hq_policy* policy,
                     float sm_scale, float* col_scores, int32_t* sel_idx, int32_t* sel_count, hq_thresh* thresh,
                     int32_t* n_persist, void* ws, size_t ws_bytes, void* stream) {
    static const char* fn = "hq_reprobe";
    clear_err();
    hq_status st;
    if ((st = check_policy(fn, policy))) return st;
    if ((st = check_cache(fn, cache))) return st;
    if ((st = check_heads(fn, cache->B, Hq, cache->Hkv, cache->D))) return st;
    if (policy->window != cache->window)
        return fail(HQ_ERR_INVALID_ARG, "%s: policy window %d != cache window %d", fn, policy->window, cache->window);
    if (!hq::probe_shape_supported(Hq / cache->Hkv, policy->probe_rows))
        return fail(HQ_ERR_UNSUPPORTED, "%s: %s (query heads per KV head %d, probe_rows %d)", fn,
                    hq::probe_shape_rule(), Hq / cache->Hkv, policy->probe_rows);
    if ((int64_t)cache->cap_q + cache->cap_keep + cache->window > (1 << 24))
        return fail(HQ_ERR_CAPACITY, "%s: cap_q + cap_keep + window exceeds 2^24 positions", fn);
    if (!(sm_scale > 0.0f) || sm_scale > 1e6f) return fail(HQ_ERR_INVALID_ARG, "%s: sm_scale must be positive", fn);
    REQ_PTR(q_recent);
    REQ_PTR(col_scores);
    REQ_PTR(sel_idx);
    REQ_PTR(sel_count);
    REQ_PTR(thresh);
    REQ_PTR(n_persist);
    REQ_PTR(ws);
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return fail(HQ_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    const size_t need = hq::reprobe_ws_bytes(*cache, Hq, *policy);
    if (ws_bytes < need) return fail(HQ_ERR_CAPACITY, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    hipError_t e = hq::launch_reprobe(*cache, q_recent, Hq, *policy, sm_scale, col_scores, sel_idx, sel_count, thresh,
                                      n_persist, ws, (hipStream_t)stream);
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

size_t hq_prefill_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t D, const hq_policy* policy) {
    if (!policy || B < 1 || Hq < 1 || Hkv < 1 || T < 1 || D != hq::kD || Hq % Hkv) return 0;
    return hq::prefill_ws_bytes(B, Hq, Hkv, T, *policy);
}

hq_status hq_prefill_attn(const void* q, const void* k, const void* v, int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                          int32_t D, int32_t dt, const hq_policy* policy, const int32_t* sel_idx,
                          const int32_t* sel_count, float sm_scale, void* out, int32_t out_dt, void* ws,
                          size_t ws_bytes, void* stream) {
    static const char* fn = "hq_prefill_attn";
    clear_err();
    hq_status st;
    if ((st = check_policy(fn, policy))) return st;
    if ((st = check_heads(fn, B, Hq, Hkv, D))) return st;
    if ((st = check_dt(fn, dt))) return st;
    if (T < 1 || T > (1 << 22)) return fail(HQ_ERR_INVALID_ARG, "%s: T %d out of range", fn, T);
    if (policy->tile_num > 0 && T > hq::kRouteMaxT)
        return fail(HQ_ERR_UNSUPPORTED, "%s: tile routing supports T <= %d (T = %d)", fn, hq::kRouteMaxT, T);
    if (out_dt != HQ_F32 && out_dt != HQ_BF16 && out_dt != HQ_F16)
        return fail(HQ_ERR_UNSUPPORTED, "%s: out dtype %d unsupported", fn, out_dt);
    if (!(sm_scale > 0.0f) || sm_scale > 1e6f) return fail(HQ_ERR_INVALID_ARG, "%s: sm_scale must be positive", fn);
    REQ_PTR(q);
    REQ_PTR(k);
    REQ_PTR(v);
    REQ_PTR(sel_idx);
    REQ_PTR(sel_count);
    REQ_PTR(out);
    const size_t need = hq::prefill_ws_bytes(B, Hq, Hkv, T, *policy);
    REQ_PTR(ws);
    if (ws_bytes < need) return fail(HQ_ERR_CAPACITY, "%s: workspace %zu bytes < required %zu", fn, ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return fail(HQ_ERR_INVALID_ARG, "%s: workspace must be 256-byte aligned", fn);
    hipError_t e = hq::launch_prefill(q, k, v, B, Hq, Hkv, T, dt == HQ_F16, *policy, sel_idx, sel_count,
                                      hq::sel_stride(T, *policy), sm_scale, out, (hq_dtype)out_dt, ws, (hipStream_t)stream);
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

size_t hq_diag_read_int4_sink_bytes(const hq_cache* cache) {
    if (!cache || cache->B < 1 || cache->Hkv < 1 || cache->cap_q < hq::kTile) return 0;
    return hq::diag_sink_bytes(*cache, decode_tps(*cache, 4));
}

hq_status hq_diag_read_int4(const hq_cache* cache, void* sink, size_t sink_bytes, void* stream) {
    static const char* fn = "hq_diag_read_int4";
    clear_err();
    hq_status st;
    if ((st = check_cache(fn, cache))) return st;
    REQ_PTR(sink);
    const size_t need = hq::diag_sink_bytes(*cache, decode_tps(*cache, 4));
    if (sink_bytes < need) return fail(HQ_ERR_CAPACITY, "%s: sink %zu bytes < required %zu", fn, sink_bytes, need);
    hipError_t e = hq::launch_diag_read_int4(*cache, sink, decode_tps(*cache, 4), (hipStream_t)stream);
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

hq_status hq_diag_exp2_error(float lo, float hi, double* out, size_t out_count, void* stream) {
    static const char* fn = "hq_diag_exp2_error";
    clear_err();
    if (!(lo >= -64.0f && hi <= 64.0f && lo <= hi))
        return fail(HQ_ERR_INVALID_ARG, "%s: need -64 <= lo <= hi <= 64 (finite)", fn);
    if (out_count < 1 || out_count > 65536)
        return fail(HQ_ERR_INVALID_ARG, "%s: out_count must be in [1, 65536]", fn);
    REQ_PTR(out);
    auto key = [](float x) -> int64_t {
        uint32_t b;
        memcpy(&b, &x, 4);
        return (b & 0x80000000u) ? -(int64_t)(b & 0x7FFFFFFFu) : (int64_t)b;
    };
    const int64_t k0 = key(lo), n = key(hi) - k0 + 1;
    hipError_t e = hq::launch_diag_exp2_error((int32_t)k0, n, out, (int)out_count, (hipStream_t)stream);
    return e == hipSuccess ? HQ_OK : hip_fail(fn, e);
}

}  // extern "C"
