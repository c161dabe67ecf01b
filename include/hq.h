/* hq.h -- C ABI of libhyquant: HyQuant-style hybrid-precision attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (pages: "HyQuant: Hybrid-Precision Quantization for LLM
 * Attention", TL;DR and flowchart; "How HyQuant uses hybrid-precision
 * attention to cut decode compute", "What hybrid-precision attention
 * changes"; the HyQuant abstract on the ACL Anthology author page):
 * a cheap vertical-line-aware probe of the attention pattern picks the key
 * columns that nearly every query attends to; those columns plus a recent
 * local window stay in high precision and everything else is quantized to
 * low bit width. Prefill runs a hybrid-precision attention operator with
 * that split; decode keeps a hybrid KV cache and fuses dequantization into
 * the attention kernel so dequantized values never go back to memory.
 *
 * The five calls below follow that statement of the problem:
 *   hq_probe_select  -- the probe and the top-k column selection
 *   hq_quantize_kv   -- build the hybrid cache (INT4 rest + 16-bit kept/window)
 *   hq_append_kv     -- one decode-time token append (the window slides)
 *   hq_decode_attn   -- decode attention with fused INT4 dequantization
 *   hq_prefill_attn  -- the causal prefill hybrid-precision operator
 * and hq_reprobe runs the probe again over the cache during decoding.
 *
 * Conventions shared by every call
 *   - Device pointers unless stated otherwise. All work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the null stream) and is
 *     asynchronous; no call synchronizes, allocates device memory, frees, or
 *     changes the current device. Buffers are owned by the caller; the *_bytes
 *     and hq_cache_layout queries give their sizes.
 *   - Tensors are contiguous, row-major, in the shapes written next to each
 *     argument. Element types (`dt`, `out_dt`) are hq_dtype values passed as
 *     int32_t, so that any integer a caller passes is validated rather than
 *     being an out-of-range enum. 16-bit tensors use `dt` (HQ_BF16 or
 *     HQ_F16); head_dim D must
 *     be 128; Hq must be a multiple of Hkv (grouped-query attention: query
 *     head h reads KV head h / (Hq/Hkv)); Hq/Hkv must be 1, 2, 4 or 8.
 *   - All device pointers must be 16-byte aligned. Outputs must not alias
 *     inputs.
 *   - Every argument is validated on the host before anything is launched.
 *     On a validation error nothing is enqueued, no output is written, the
 *     call returns a negative status and hq_last_error() describes the
 *     problem. A failed kernel launch returns HQ_ERR_HIP with the HIP error
 *     string; calls that launch several kernels in sequence (probe, decode,
 *     prefill) may then leave the kernels launched before the failing one
 *     enqueued, so their outputs are undefined after HQ_ERR_HIP.
 *   - The library's only global state is a per-device cache of the compute
 *     unit count (read once with hipDeviceGetAttribute) and the per-device
 *     scratch array of hq_decode_attn_noalloc. It is safe to call from
 *     several threads (each thread has its own hq_last_error buffer).
 */
#ifndef HQ_H_
#define HQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int hq_status;
#define HQ_OK 0
#define HQ_ERR_INVALID_ARG (-1) /* null pointer, bad size, misalignment, bad policy */
#define HQ_ERR_UNSUPPORTED (-2) /* D != 128, Hq % Hkv != 0, group size, dtype      */
#define HQ_ERR_CAPACITY (-3)    /* workspace or cache capacity too small           */
#define HQ_ERR_HIP (-4)         /* kernel launch failed                            */

typedef enum { HQ_F16 = 0, HQ_BF16 = 1, HQ_F32 = 2 } hq_dtype;

/* Retention policy. Pages: "How HyQuant uses hybrid-precision attention to
 * cut decode compute", sections "Why preserve selected positions?" and "What
 * the authors tested": the top 5% of key positions plus a local window (128
 * tokens in the coverage analysis) stay in high precision.
 *   keep_num/keep_den : retained fraction; k = floor(keep_num*T/keep_den),
 *                       capped at the T - window candidates (default 5/100)
 *   window            : recent positions always kept; multiple of 64 (128)
 *   probe_rows        : last query rows the probe looks at (64)            */
typedef struct {
    int32_t keep_num;
    int32_t keep_den;
    int32_t window;
    int32_t probe_rows;
    int32_t low_fmt;   /* low-precision path of hq_prefill_attn: HQ_LOW_INT8
                          (0, the default) or HQ_LOW_FP8; ignored elsewhere */
    int32_t tile_num;  /* tile routing of hq_prefill_attn (INT8 path only):  */
    int32_t tile_den;  /* the fraction tile_num / tile_den of each 128-row
                          query block's key blocks below its window band is
                          also computed in 16 bits; tile_num = 0 (the
                          default) turns it off                            */
} hq_policy;
typedef enum { HQ_LOW_INT8 = 0, HQ_LOW_FP8 = 1 } hq_low_fmt;

/* Score and position of the k-th selected candidate (k > 0), or
 * {+inf, -1} when nothing was selected. */
typedef struct {
    float tau;
    int32_t j_k;
} hq_thresh;

/* Size in elements of the per-(batch, KV head) selected-index stride for a
 * context of up to T tokens: max(1, floor(keep_num*T/keep_den)). */
int32_t hq_sel_stride(int32_t T, const hq_policy* policy);

/* ------------------------------------------------------------------------
 * hq_probe_select -- vertical-line probe + top-k column selection.
 * Pages: "HyQuant: Hybrid-Precision Quantization for LLM Attention", TL;DR
 * and "What problem it solves" (a few key columns are attended by almost
 * every query, found with a lightweight pattern signal, no calibration);
 * "How HyQuant uses ...", "Why preserve selected positions?" (retain the
 * high-score positions, top 5%).
 * Computes, for each batch b and KV head g, with T = seq_lens[b]:
 *   col_scores[b][g][j] = sum over the Hq/Hkv query heads of g and the last
 *     R = min(probe_rows, T) rows r (at positions T-R..T-1) of
 *     softmax_{j' <= pos_r}(q_r . k_j' * sm_scale)[j],  for j < T
 *   sel_idx[b][g][0..k)  = the k candidates j in [0, T - window) with the
 *     largest score (ties: lower j first), in ascending order; k as in
 *     hq_policy. sel_count[b][g] = k; thresh[b][g] = the k-th one.
 * sm_scale is used as the fp32 value passed. Logits come from exact integer
 * products on the int8 matrix cores (each 16-bit value written as base-256
 * digits of a scaled integer); a per-tile a-posteriori bound on the digits
 * left out is checked and any tile above 1.0e-7 (log2 units) is recomputed
 * in fp64. Each logit is computed once: its softmax term (against a
 * per-row, per-key-chunk power-of-two reference) is stored in fp32 in the
 * workspace, the row normalisers and the column sums of the stored terms
 * accumulate in fp64, and the scores are rounded to fp32. Each score above
 * 1e-30 has a relative error below 2.9e-7 (with the observed bounds, ~1e-8
 * logit error, it is the two fp32 roundings); smaller scores are within
 * 1e-42 absolute.
 * Supported shapes: (Hq/Hkv) * probe_rows must be a multiple of 16 and at
 * most 512; other shapes return HQ_ERR_UNSUPPORTED before any launch.
 *   q_probe   [B][Hq][probe_rows][D] dt  row r is position T_b - probe_rows + r
 *   k         [B][Hkv][Tmax][D]      dt
 *   seq_lens  [B] int32, 1 <= T_b <= Tmax
 *   col_scores[B][Hkv][Tmax] fp32 out (entries >= T_b are set to 0)
 *   sel_idx   [B][Hkv][hq_sel_stride(Tmax)] int32 out (unused tail = -1)
 *   sel_count [B][Hkv] int32 out;  thresh [B][Hkv] out
 *   ws        workspace of hq_probe_ws_bytes(...) bytes: mostly the probe
 *             rows' stored terms, 4 * (Hq/Hkv) * probe_rows * Tp bytes
 *             (Tp = Tmax rounded up to 32, plus 32) per (b, KV head), the
 *             rows' count rounded up to 32; 4.3 GB for B = 16,
 *             8 KV heads, 4 heads each, 64 rows, Tmax = 32768             */
hq_status hq_probe_select(const void* q_probe, const void* k, const int32_t* seq_lens,
                          int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, int32_t D,
                          int32_t dt, const hq_policy* policy, float sm_scale,
                          float* col_scores, int32_t* sel_idx, int32_t* sel_count,
                          hq_thresh* thresh, void* ws, size_t ws_bytes, void* stream);
size_t hq_probe_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Tmax, int32_t D,
                         const hq_policy* policy);

/* ------------------------------------------------------------------------
 * The hybrid KV cache. Pages: "HyQuant: ...", flowchart and "Key results"
 * (decode keeps a hybrid cache; dequantization fused into attention);
 * "How HyQuant uses ...", "What the authors tested" (non-retained KV in
 * Key-4bit/Value-4bit) and "Memory and runtime costs" (retention costs about
 * 15% over strict 4-bit, i.e. retained tokens are held only in 16 bits).
 *
 * Per (batch b, KV head g) the cache holds
 *   INT4 store : every position that is neither selected nor in the window,
 *                ascending; per token and per 32-channel group of K and of
 *                V: asymmetric codes (0..15), fp16 scale s and zero z with
 *                x_hat = code*s + z, where s = fp16(fp32(max-min)/15),
 *                z = fp16(min), code = clamp(rint((x - z)/s), 0, 15) in fp32.
 *   kept store : the selected positions (and departures flagged by the append
 *                rule), 16-bit, in insertion order.
 *   ring       : the last `window` positions, 16-bit, slot = position % window.
 * Storage is tiled in 64-token tiles. The INT4 tiles are laid out as the
 * operands of the decode kernel's 16x16x32 fp16 matrix instructions: every
 * 32-bit word holds 8 codes, element e (0..7) in the nibble at bit
 * n(e) = 16*(e%2) + 4*(e/2), and every 128-bit load is contiguous across the
 * wavefront. For slot t and channel c of a tile (4096 bytes each for K, V):
 *   K code: element c%8 of the word at byte
 *       (t/16)*1024 + ((t%16) + 16*((c%32)/8))*16 + (c/32)*4;
 *   V code: element t%8 of the word at byte
 *       (c/32)*1024 + ((c%16) + 16*((t%32)/8))*16 + (2*((c/16)%2) + t/32)*4;
 *   K scale/zero of group j (one fp16 pair): byte ((t%16) + 16j)*16 + (t/16)*4
 *       of the tile's 1024-byte metadata block;
 *   V scale/zero of group j: byte t*16 + j*4 of the tile's metadata block;
 *   16-bit K rows, chunk c (channels 8c..8c+7) of slot t at c*1024 + t*16;
 *   16-bit V rows, chunk c of slot t at (t%16)*1024 + (16*(t/16) + c)*16.
 * Position tags give the canonical order. The struct is filled by the caller
 * with buffers of the sizes hq_cache_layout() returns; all counters live on
 * the device so no call needs a device-to-host copy.                       */
typedef struct {
    int32_t B, Hkv, D, window;
    int32_t cap_q;      /* INT4 slots per (b, g), multiple of 64              */
    int32_t cap_keep;   /* kept-store slots per (b, g), multiple of 64        */
    int32_t cap_probe;  /* probed positions per (b, g) (col_scores stride)    */
    int32_t dt;         /* hq_dtype of the 16-bit stores (HQ_BF16 or HQ_F16)  */
    void* k_codes;      /* [B][Hkv][cap_q/64][4096] bytes                     */
    void* v_codes;      /* [B][Hkv][cap_q/64][4096] bytes                     */
    void* k_meta;       /* [B][Hkv][cap_q/64][1024] bytes: (s,z) fp16 pairs    */
    void* v_meta;       /* [B][Hkv][cap_q/64][1024] bytes                      */
    void* k_keep;       /* [B][Hkv][cap_keep/64][64*D] 16-bit                 */
    void* v_keep;
    void* k_win;        /* [B][Hkv][window/64][64*D] 16-bit                   */
    void* v_win;
    int32_t* q_pos;     /* [B][Hkv][cap_q] position of each INT4 slot         */
    int32_t* keep_pos;  /* [B][Hkv][cap_keep] position of each kept slot      */
    int32_t* counts;    /* [B][Hkv][4]: seq_len, n_q, n_keep, probe_len       */
    float* col_scores;  /* [B][Hkv][cap_probe] probe scores kept for append   */
    hq_thresh* thresh;  /* [B][Hkv]                                           */
    int32_t* err_flag;  /* [1]: bits set by kernels, never cleared by them:
                           1 quantize: a count or length out of range (that
                             (b, g) is left unwritten); 2 append: a store full
                             (nothing stored); 4 quantize: selected positions
                             not ascending candidates (the entries before the
                             first bad one are stored)                      */
    /* Ragged INT4 layout (hq_cache_layout_ragged); NULL / 0 for the uniform
     * one above. q_tile_off: device [B*Hkv + 1] int64, ascending: the INT4
     * store of (b, g) is tiles [q_tile_off[bg], q_tile_off[bg+1]) of
     * k_codes / v_codes / k_meta / v_meta (4096 / 4096 / 1024 / 1024 bytes
     * per tile) and slots [64 q_tile_off[bg], ...) of q_pos; cap_q is the
     * largest per-(b, g) capacity. q_tiles_total: tiles in each of those
     * buffers. A span that is not ascending or leaves [0, q_tiles_total) is
     * treated as empty (nothing read or written there).                    */
    const int64_t* q_tile_off;
    int64_t q_tiles_total;
} hq_cache;

typedef struct {
    int32_t cap_q, cap_keep, cap_probe;
    size_t k_codes, v_codes, k_meta, v_meta, k_keep, v_keep, k_win, v_win;
    size_t q_pos, keep_pos, counts, col_scores, thresh, err_flag;
} hq_cache_sizes;

/* Byte sizes of every cache buffer for contexts of up to cap_tokens tokens
 * (prompt plus appends) whose probe covered at most cap_probe positions.
 *   cap_q    = round64(cap_tokens - min(window, cap_tokens)), at least 64:
 *              every position outside the window may be quantized (a short
 *              sequence of a ragged batch keeps few columns and may be
 *              appended up to cap_tokens, so the top-k is not subtracted);
 *   cap_keep = round64(k(cap_probe) + min(window, cap_probe)): the selected
 *              columns plus the departures the append rule may keep, which
 *              were window positions when the probe ran.
 * cap_tokens above 2^24 returns HQ_ERR_CAPACITY (one (b, g)'s INT4 store is
 * addressed with 32-bit byte offsets).                                     */
hq_status hq_cache_layout(int32_t B, int32_t Hkv, int32_t D, int32_t cap_tokens,
                          int32_t cap_probe, int32_t dt, const hq_policy* policy,
                          hq_cache_sizes* out);

/* The ragged INT4 layout: a host-side allocator for batches whose sequences
 * have different capacities (serving: each sequence sized for its own prompt
 * plus its own decode budget, instead of every (b, g) sized for the longest).
 * Pages: "How HyQuant uses ...", "Reported speedups: kernel gains are not
 * end-to-end gains" (the serving system around the kernel decides the end to
 * end gain) and "Memory and runtime costs" (the memory the cache takes).
 * Sequence b gets round64(cap_tokens[b] - min(window, cap_tokens[b])) INT4
 * slots (at least 64), for each of its Hkv heads, packed back to back in
 * (b, g) order: q_tile_off (host [B*Hkv + 1], written) holds the tile
 * offsets, to be copied to the device for hq_cache.q_tile_off. The kept
 * store, ring and per-(b, g) arrays keep the uniform layout of
 * max(max cap_tokens, cap_probe) (cap_probe may exceed every capacity when
 * the prompts were probed padded to a common length). out receives every
 * buffer's bytes (the INT4 pools sized by the total) and out->cap_q = that
 * uniform layout's INT4 capacity, at least every sequence's.
 * Errors as hq_cache_layout, checked for every cap_tokens[b].            */
hq_status hq_cache_layout_ragged(int32_t B, int32_t Hkv, int32_t D, const int32_t* cap_tokens,
                                 int32_t cap_probe, int32_t dt, const hq_policy* policy,
                                 int64_t* q_tile_off, hq_cache_sizes* out);

/* ------------------------------------------------------------------------
 * hq_quantize_kv -- build the hybrid cache from a prompt's K and V.
 * Kept set H = S u [T-W, T) with S = sel_idx[b][g][0..sel_count); every other
 * position is INT4-quantized (K and V alike); the probe scores and threshold
 * are copied into the cache for the append rule. Resets the cache counters.
 *   k, v       [B][Hkv][Tmax][D] dt;  seq_lens [B] int32
 *   sel_idx    [B][Hkv][hq_sel_stride(Tmax)] ascending; sel_count [B][Hkv]
 *   col_scores [B][Hkv][Tmax] fp32; thresh [B][Hkv]
 *   cache      host struct describing caller-owned buffers (Tmax <= cap_probe) */
hq_status hq_quantize_kv(const void* k, const void* v, const int32_t* seq_lens, int32_t Tmax,
                         const int32_t* sel_idx, const int32_t* sel_count,
                         const float* col_scores, const hq_thresh* thresh,
                         const hq_policy* policy, const hq_cache* cache, void* stream);

/* ------------------------------------------------------------------------
 * hq_append_kv -- append one token per (b, g) at position T = seq_len.
 * Pages: "HyQuant: ...", flowchart (the recent local sliding window stays in
 * high precision next to the vertical-line columns; the rest is low-bit);
 * "How HyQuant uses ...", "What hybrid-precision attention changes" (during
 * decode the cache keeps the selected positions in high precision and the
 * rest in low bit width). The pages do not say what happens to a token that
 * slides out of the window. Reading: it is treated as the selection would
 * have treated it.
 * The new token enters the ring. The token leaving the window, d = T - W
 * (when T >= W), goes to the kept store if it was probed (d < probe_len) and
 * its probe score ranks above the k-th selected candidate (it would have been
 * selected had it been a candidate), and is INT4-quantized otherwise; tokens
 * generated after the probe are always quantized when they leave.
 *   k_new, v_new [B][Hkv][D] cache->dt
 * A capacity overflow sets bit 1 of cache->err_flag and stores nothing.    */
hq_status hq_append_kv(const hq_cache* cache, const void* k_new, const void* v_new, void* stream);

/* ------------------------------------------------------------------------
 * hq_decode_attn -- one decode step of attention over the hybrid cache.
 * Pages: "HyQuant: ...", TL;DR and "Key results" (KV dequantization fused
 * with the attention computation); "How HyQuant uses ...", "What
 * hybrid-precision attention changes" (no full-precision copy of the cache
 * is ever expanded).
 *   out[b][h] = sum_j softmax_j(q[b][h] . k~_j * sm_scale) v~_j over all
 *   T = seq_len cached tokens of KV head h / (Hq/Hkv), with k~, v~ the 16-bit
 *   values on kept/window positions and code*s + z elsewhere.
 * INT4 codes are dequantized in registers; dot products accumulate in fp32;
 * split-K partial softmax states are merged by a second kernel.
 *   q   [B][Hq][D] cache->dt;  out [B][Hq][D] out_dt (HQ_F32 for parity)
 *   ws  workspace of hq_decode_ws_bytes(cache, Hq) bytes
 * Split size: the INT4 tiles (64 tokens) of a (b, g) are divided over
 * ceil(tiles / 54) splits, raised until the grid fills whole rounds of the
 * current device's workgroup slots (2 per CU; eight heads per KV head run
 * as two four-head workgroups per split), with
 * at least 4 tiles per split. The workspace query and the call compute it
 * alike for the current device. The result does not depend on it beyond
 * fp32 rounding. */
hq_status hq_decode_attn(const hq_cache* cache, const void* q, int32_t Hq, float sm_scale,
                         void* out, int32_t out_dt, void* ws, size_t ws_bytes, void* stream);
size_t hq_decode_ws_bytes(const hq_cache* cache, int32_t Hq);

/* ------------------------------------------------------------------------
 * hq_reprobe -- run the probe again over the hybrid cache, from the last
 * decode queries, to see whether the kept columns are still the heavy ones.
 * Pages: "HyQuant: ...", "Gaps" (whether the vertical-line columns found on
 * the prompt persist through decoding, notably under heavy batching, is left
 * open) and TL;DR (the columns are found with a lightweight signal of the
 * attention pattern).
 * Computes what hq_probe_select computes, with T = the cache's seq_len, over
 * the keys the cache now holds:
 *   k~_j = the stored 16-bit row for kept and window positions; for INT4
 *          positions code*s + z evaluated in fp32 with one rounding, then
 *          rounded to cache->dt (half to even),
 * and the last R = policy->probe_rows decode queries (row r at position
 * T - R + r: the query issued when the cache held T - R + r + 1 tokens);
 * and in addition
 *   n_persist[b][g] = how many of the newly selected columns are in the kept
 *                     store, i.e. already held in 16 bits.
 * The cache is only read; moving tokens between stores is left to the
 * caller. Tcap = cache->cap_q + cache->cap_keep + cache->window bounds every
 * seq_len and is the position stride of the outputs:
 *   q_recent   [B][Hq][probe_rows][D] cache->dt
 *   col_scores [B][Hkv][Tcap] fp32 out (entries >= seq_len are 0)
 *   sel_idx    [B][Hkv][hq_sel_stride(Tcap)] int32 out (unused tail = -1)
 *   sel_count, n_persist [B][Hkv] int32 out;  thresh [B][Hkv] out
 *   ws         hq_reprobe_ws_bytes(cache, Hq, policy) bytes, 256-byte aligned.
 *              After the call its first B*Hkv*Tcap*D*2 bytes hold the expanded
 *              keys k~ as [B][Hkv][Tcap][D] cache->dt (rows >= seq_len are
 *              not written).
 * policy->window must equal cache->window. The shape rule, error bound and
 * errors of hq_probe_select apply; Tcap above 2^24 returns HQ_ERR_CAPACITY.
 * All KV heads of one batch row hold the same seq_len (hq_quantize_kv and
 * hq_append_kv keep it so); the one of KV head 0 is used. */
hq_status hq_reprobe(const hq_cache* cache, const void* q_recent, int32_t Hq, const hq_policy* policy,
                     float sm_scale, float* col_scores, int32_t* sel_idx, int32_t* sel_count,
                     hq_thresh* thresh, int32_t* n_persist, void* ws, size_t ws_bytes, void* stream);
size_t hq_reprobe_ws_bytes(const hq_cache* cache, int32_t Hq, const hq_policy* policy);

/* ------------------------------------------------------------------------
 * hq_decode_attn_noalloc -- hq_decode_attn without a workspace argument, for
 * callers that cannot allocate device memory around the call (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, kernels and results as hq_decode_attn; the split partials
 * go to a fixed array inside the library (HQ_DECODE_NOALLOC_SCRATCH_BYTES
 * per device, held until the process ends) instead of `ws`. The call
 * allocates nothing: the first call on a device looks up that device's copy
 * of the array once (hipGetSymbolAddress).
 * Errors as hq_decode_attn, plus HQ_ERR_CAPACITY when the cache needs more
 * partials than the array holds (hq_decode_ws_bytes(cache, Hq) bytes must be
 * at most HQ_DECODE_NOALLOC_SCRATCH_BYTES), checked before any launch.
 * Every call on one device uses the same array: calls that overlap on one
 * device (concurrent streams, or host threads without ordering) race and
 * give undefined results. Calls on one stream are ordered and safe; nothing
 * in the array needs to be cleared between calls. */
#define HQ_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
hq_status hq_decode_attn_noalloc(const hq_cache* cache, const void* q, int32_t Hq, float sm_scale,
                                 void* out, int32_t out_dt, void* stream);

/* ------------------------------------------------------------------------
 * hq_prefill_attn -- causal hybrid-precision prefill attention.
 * Pages: HyQuant abstract (Prefill stage: vertical-line tokens and a local
 * sliding window in full precision, the remaining context quantized);
 * "HyQuant: ...", "How this relates to prior wiki pages" (two precision
 * paths updating one online-softmax state).
 * For query row i of head h (KV head g) and key j <= i:
 *   j in S_g or i - j < window : score = (q_i . k_j) * sm_scale   (bf16 MFMA)
 *   otherwise : score = (Q8_i . K8_j) * sQ * sK * sm_scale  (INT8 or FP8 MFMA)
 * with symmetric codes per 64-token block over all channels, by
 * policy->low_fmt: HQ_LOW_INT8, s = max|x|/127 in fp32, code = rint(x/s)
 * (exact int32 products); or HQ_LOW_FP8 (HyQuant page "Gaps": FP8 as a third
 * precision point), s = max|x|/448 in fp32, code = OCP E4M3 of fp32(x/s),
 * round to nearest even (fp32 sums of exact products). out_i = sum_j
 * softmax(score)_j v_j. P and V enter the PV product as fp16.
 * Tile routing (policy->tile_num > 0, INT8 only; HyQuant page "How this
 * relates to prior wiki pages" and "Gaps": TileMix's tile-level FP16/INT8
 * dispatch, and whether it composes with the token routing): for every
 * 128-row query block (rows i0 .. i0+127, i0 = 128 qb) the candidate key
 * blocks kb < kb_band = min(nkb, max(0, (i0 - window + 1) / 64)) are ranked
 * by E(kb) = fp32(sK(kb) * (A + B(kb) + 5D/2)), A = max over the block's rows
 * of sum_c |Q8_ic|, B(kb) = max over the key block of sum_c |K8_jc| (the
 * INT8 score error bound's shape), and the floor(tile_num * kb_band /
 * tile_den) largest (ties: lower kb) are scored in 16 bits for every row of
 * the query block. T must then be at most 262,144.
 *   q [B][Hq][T][D], k, v [B][Hkv][T][D] dt (values within fp16 range for
 *   V); sel_idx [B][Hkv][hq_sel_stride(T)] int32, the first sel_count[b][g]
 *   entries ascending, distinct and in [0, T) (as hq_probe_select returns
 *   them for Tmax = T; any such set is accepted, including an empty one);
 *   out [B][Hq][T][D] out_dt; ws of hq_prefill_ws_bytes() bytes, 256-byte
 *   aligned. Entries outside the documented range are ignored, never read
 *   out of bounds.
 * Workspace after the call (the low-precision stage, readable for
 * inspection; one code byte per element, INT8 or E4M3 bits), with
 * nb = ceil(T / 64), Tp = 64 nb and A(x) = x rounded up to a multiple of 256:
 *   offset 0                      Q8 int8 [B][Hq][Tp][D] (rows >= T are 0)
 *   o1 = A(B Hq Tp D)             sQ fp32 [B][Hq][nb]
 *   o2 = o1 + A(4 B Hq nb)        K8 int8 [B][Hkv][Tp][D]
 *   o3 = o2 + A(B Hkv Tp D)       sK fp32 [B][Hkv][nb]
 * the rest is staging (fp16 V^T blocks, with and without the selected
 * columns, selected-column masks and row-sum weights, gathered selected K / V
 * tiles) and, with tile routing, the per-block code norms; the workspace
 * ends with the routed tiles' masks: its last A(8 B Hq nqb nw) bytes,
 * nqb = ceil(T / 128), nw = ceil(nb / 64), hold uint64 [B][Hq][nqb][nw]
 * with bit kb % 64 of word kb / 64 set for a routed key block kb.
 * Errors: HQ_ERR_UNSUPPORTED for D != 128, Hq % Hkv != 0, G = Hq / Hkv not
 * in {1, 2, 4, 8} or an unsupported dtype; HQ_ERR_CAPACITY if ws_bytes is
 * too small; HQ_ERR_INVALID_ARG for null pointers or T outside [1, 2^22]. */
hq_status hq_prefill_attn(const void* q, const void* k, const void* v, int32_t B, int32_t Hq,
                          int32_t Hkv, int32_t T, int32_t D, int32_t dt,
                          const hq_policy* policy, const int32_t* sel_idx,
                          const int32_t* sel_count, float sm_scale, void* out,
                          int32_t out_dt, void* ws, size_t ws_bytes, void* stream);
size_t hq_prefill_ws_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t D,
                           const hq_policy* policy);

/* Description of the last error on the calling thread ("" if none). Valid
 * until the next hq_* call on this thread. */
const char* hq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* HQ_H_ */
