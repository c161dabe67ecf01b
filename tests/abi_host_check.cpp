// Host-layer check of libhyquant's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_abi.py (host code only; no GPU is
// needed: every call below is a size or layout query or is rejected by the
// host validation before anything is launched; no call here has arguments
// that pass validation, and the test hides every device from the process).
// Prints "host checks passed"
// and exits 0, or names the failing check and exits 1; a sanitizer report
// aborts the run.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string_view>
#include <vector>

#include "../include/hq.h"
#include "../include/hq_diag.h"

static int failures = 0;
#define EXPECT(cond)                                                            \
    do {                                                                        \
        if (!(cond)) {                                                          \
            std::printf("FAILED line %d: %s (%s)\n", __LINE__, #cond, hq_last_error()); \
            ++failures;                                                         \
        }                                                                       \
    } while (0)

int main() {
    void* const F = reinterpret_cast<void*>(0x100000);   // aligned, never dereferenced
    void* const M = reinterpret_cast<void*>(0x100004);   // misaligned
    hq_policy pol = {5, 100, 128, 64, HQ_LOW_INT8, 0, 100};

    // sizes and layouts (host arithmetic only)
    EXPECT(hq_sel_stride(32768, &pol) == 1638);
    EXPECT(hq_sel_stride(10, &pol) == 1);
    EXPECT(hq_sel_stride(100, nullptr) == 1);
    hq_cache_sizes sz;
    std::memset(&sz, 0, sizeof(sz));
    EXPECT(hq_cache_layout(2, 8, 128, 4096, 4096, HQ_BF16, &pol, &sz) == HQ_OK);
    EXPECT(sz.cap_q == 4096 - 128 && sz.k_codes == (size_t)16 * sz.cap_q * 64);
    EXPECT(hq_cache_layout(2, 8, 128, 0, 1, HQ_BF16, &pol, &sz) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_cache_layout(2, 8, 128, (1 << 24) + 1, 10, HQ_BF16, &pol, &sz) == HQ_ERR_CAPACITY);
    EXPECT(hq_cache_layout(2, 8, 96, 1000, 1000, HQ_BF16, &pol, &sz) == HQ_ERR_UNSUPPORTED);
    EXPECT(hq_cache_layout(2, 8, 128, 1000, 1000, HQ_F32, &pol, &sz) == HQ_ERR_UNSUPPORTED);
    EXPECT(hq_cache_layout(2, 8, 128, 1000, 1000, HQ_BF16, nullptr, &sz) == HQ_ERR_INVALID_ARG);
    const int32_t caps[3] = {700, 3000, 64};
    std::vector<int64_t> off(3 * 2 + 1, -1);
    EXPECT(hq_cache_layout_ragged(3, 2, 128, caps, 2000, HQ_BF16, &pol, off.data(), &sz) == HQ_OK);
    EXPECT(off[0] == 0 && off[6] == 2 * 9 + 2 * 45 + 2 * 1 && sz.k_codes == (size_t)off[6] * 4096);
    const int32_t bad_caps[3] = {700, -1, 64};
    EXPECT(hq_cache_layout_ragged(3, 2, 128, bad_caps, 2000, HQ_BF16, &pol, off.data(), &sz) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_cache_layout_ragged(3, 2, 128, nullptr, 2000, HQ_BF16, &pol, off.data(), &sz) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_probe_ws_bytes(1, 32, 8, 32768, 128, &pol) > 0);
    EXPECT(hq_probe_ws_bytes(1, 32, 8, 32768, 128, nullptr) == 0);
    EXPECT(hq_prefill_ws_bytes(1, 32, 8, 16384, 128, &pol) > 0);

    // probe validation
    hq_thresh* thr = reinterpret_cast<hq_thresh*>(F);
    float* fcol = reinterpret_cast<float*>(F);
    int32_t* iF = reinterpret_cast<int32_t*>(F);
    EXPECT(hq_probe_select(nullptr, F, iF, 1, 32, 8, 1024, 128, HQ_BF16, &pol, 0.088f, fcol, iF, iF, thr, F,
                           1ull << 40, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_probe_select(M, F, iF, 1, 32, 8, 1024, 128, HQ_BF16, &pol, 0.088f, fcol, iF, iF, thr, F, 1ull << 40,
                           nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_probe_select(F, F, iF, 1, 32, 7, 1024, 128, HQ_BF16, &pol, 0.088f, fcol, iF, iF, thr, F, 1ull << 40,
                           nullptr) == HQ_ERR_UNSUPPORTED);
    EXPECT(hq_probe_select(F, F, iF, 1, 32, 8, 1024, 128, HQ_BF16, &pol, -1.0f, fcol, iF, iF, thr, F, 1ull << 40,
                           nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_probe_select(F, F, iF, 1, 32, 8, 1024, 128, HQ_BF16, &pol, 0.088f, fcol, iF, iF, thr, F, 16,
                           nullptr) == HQ_ERR_CAPACITY);
    hq_policy odd = pol;
    odd.probe_rows = 10;  // 4 x 10 rows: not a multiple of 16
    EXPECT(hq_probe_select(F, F, iF, 1, 32, 8, 1024, 128, HQ_BF16, &odd, 0.088f, fcol, iF, iF, thr, F, 1ull << 40,
                           nullptr) == HQ_ERR_UNSUPPORTED);
    std::string_view msg = hq_last_error();
    EXPECT(msg.find("multiple of 16") != std::string_view::npos);

    // cache calls on malformed caches
    hq_cache c;
    std::memset(&c, 0, sizeof(c));
    EXPECT(hq_decode_attn(&c, F, 4, 0.088f, F, HQ_F32, F, 1ull << 40, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_append_kv(&c, F, F, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_append_kv(nullptr, F, F, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_decode_attn_noalloc(nullptr, F, 4, 0.088f, F, HQ_F32, nullptr) == HQ_ERR_INVALID_ARG);
    c.B = 1; c.Hkv = 1; c.D = 128; c.window = 128; c.cap_q = 960; c.cap_keep = 192; c.cap_probe = 1024; c.dt = HQ_BF16;
    c.k_codes = c.v_codes = c.k_meta = c.v_meta = c.k_keep = c.v_keep = c.k_win = c.v_win = F;
    c.q_pos = c.keep_pos = c.counts = iF;
    c.col_scores = fcol;
    c.thresh = thr;
    c.err_flag = iF;
    EXPECT(hq_decode_attn(&c, F, 6, 0.088f, F, HQ_F32, F, 1ull << 40, nullptr) == HQ_ERR_UNSUPPORTED);
    EXPECT(hq_decode_attn(&c, F, 4, 0.088f, F, 9, F, 1ull << 40, nullptr) == HQ_ERR_UNSUPPORTED);
    EXPECT(hq_decode_attn(&c, F, 4, 0.088f, F, -1, F, 1ull << 40, nullptr) == HQ_ERR_UNSUPPORTED);
    EXPECT(hq_cache_layout(2, 8, 128, 1000, 1000, 1 << 30, &pol, &sz) == HQ_ERR_UNSUPPORTED);
    EXPECT(hq_decode_attn(&c, F, 4, 0.088f, F, HQ_F32, F, 8, nullptr) == HQ_ERR_CAPACITY);
    EXPECT(hq_decode_attn(&c, F, 4, 0.088f, F, HQ_F32, nullptr, 1ull << 40, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_decode_ws_bytes(&c, 4) > 0 && hq_decode_ws_bytes(&c, 0) == 0 && hq_decode_ws_bytes(nullptr, 4) == 0);
    hq_cache r = c;
    r.q_tile_off = reinterpret_cast<const int64_t*>(F);
    r.q_tiles_total = 0;
    EXPECT(hq_append_kv(&r, F, F, nullptr) == HQ_ERR_INVALID_ARG);
    r.cap_q = 100;
    EXPECT(hq_quantize_kv(F, F, iF, 100, iF, iF, fcol, thr, &pol, &r, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_quantize_kv(F, F, iF, 4096, iF, iF, fcol, thr, &pol, &c, nullptr) == HQ_ERR_CAPACITY);
    hq_policy w64 = pol;
    w64.window = 64;
    EXPECT(hq_quantize_kv(F, F, iF, 512, iF, iF, fcol, thr, &w64, &c, nullptr) == HQ_ERR_INVALID_ARG);

    // re-probe validation
    const size_t need = hq_reprobe_ws_bytes(&c, 4, &pol);
    EXPECT(need > 0);
    EXPECT(hq_reprobe(&c, F, 4, &pol, 0.088f, fcol, iF, iF, thr, iF, F, need - 1, nullptr) == HQ_ERR_CAPACITY);
    EXPECT(hq_reprobe(&c, F, 4, &w64, 0.088f, fcol, iF, iF, thr, iF, F, need, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_reprobe(&c, F, 4, &pol, 0.088f, fcol, iF, iF, thr, nullptr, F, need, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_reprobe(&c, F, 4, &pol, 0.088f, fcol, iF, iF, thr, iF, reinterpret_cast<void*>(0x100010), need,
                      nullptr) == HQ_ERR_INVALID_ARG);

    // prefill validation, including the low-precision format and tile routing
    auto pre = [&](const hq_policy& p, int32_t T, int32_t D, int32_t odt, size_t wsb) {
        return hq_prefill_attn(F, F, F, 1, 32, 8, T, D, HQ_BF16, &p, iF, iF, 0.088f, F, odt, F, wsb, nullptr);
    };
    EXPECT(pre(pol, 0, 128, HQ_F32, 1ull << 40) == HQ_ERR_INVALID_ARG);
    EXPECT(pre(pol, 1024, 64, HQ_F32, 1ull << 40) == HQ_ERR_UNSUPPORTED);
    EXPECT(pre(pol, 1024, 128, 7, 1ull << 40) == HQ_ERR_UNSUPPORTED);   // any int32 is a valid argument
    EXPECT(pre(pol, 1024, 128, HQ_F32, 1) == HQ_ERR_CAPACITY);
    hq_policy lp = pol;
    lp.low_fmt = 3;
    EXPECT(pre(lp, 1024, 128, HQ_F32, 1ull << 40) == HQ_ERR_UNSUPPORTED);
    hq_policy tp = pol;
    tp.tile_num = 7;
    tp.tile_den = 5;
    EXPECT(pre(tp, 1024, 128, HQ_F32, 1ull << 40) == HQ_ERR_INVALID_ARG);
    tp.tile_den = 0;
    EXPECT(pre(tp, 1024, 128, HQ_F32, 1ull << 40) == HQ_ERR_INVALID_ARG);
    tp.tile_num = 5;
    tp.tile_den = 100;
    tp.low_fmt = HQ_LOW_FP8;
    EXPECT(pre(tp, 1024, 128, HQ_F32, 1ull << 40) == HQ_ERR_UNSUPPORTED);
    tp.low_fmt = HQ_LOW_INT8;
    EXPECT(pre(tp, (1 << 18) + 1, 128, HQ_F32, 1ull << 40) == HQ_ERR_UNSUPPORTED);

    // the measurement helper
    EXPECT(hq_diag_read_int4(nullptr, F, 1ull << 40, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_diag_read_int4_sink_bytes(nullptr) == 0);
    double* const D = reinterpret_cast<double*>(0x100000);
    EXPECT(hq_diag_exp2_error(0.5f, -0.5f, D, 16, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_diag_exp2_error(-65.f, 0.f, D, 16, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_diag_exp2_error(-0.5f, 0.5f, D, 0, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_diag_exp2_error(-0.5f, 0.5f, D, 65537, nullptr) == HQ_ERR_INVALID_ARG);
    EXPECT(hq_diag_exp2_error(-0.5f, 0.5f, nullptr, 16, nullptr) == HQ_ERR_INVALID_ARG);

    if (failures) return 1;
    std::printf("host checks passed\n");
    return 0;
}
