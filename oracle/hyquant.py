"""HyQuant-style hybrid-precision attention: the plain CPU definitions.

TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU
baseline may call it; the product path never does).

Sources (the pages are cited by title and section):
  [HQ-wiki]  "HyQuant: Hybrid-Precision Quantization for LLM Attention"
             (wiki summary): TL;DR, flowchart, "What problem it solves",
             "Key results", "Gaps".
  [HQ-news]  "How HyQuant uses hybrid-precision attention to cut decode
             compute": "What hybrid-precision attention changes", "Why
             preserve selected positions?", "What the authors tested",
             "Memory and runtime costs".
  [HQ-abs]   The HyQuant abstract on the ACL Anthology author page.

What the method computes, in the pages' terms: a lightweight probe of the
attention pattern finds "vertical-line" key columns that almost every query
attends to; those columns plus a recent local window stay in high precision
and everything else is quantized to low bit width (K4/V4 in the reported
implementation). Prefill runs a hybrid-precision attention operator with the
same split; decode keeps a hybrid KV cache and fuses dequantization into
attention. The pages leave the probe statistic, the quantizer format, the
window shape, tie-breaks and rounding unspecified; the reading used for each
is stated at the function that depends on it.

Conventions: arrays are float64 copies of exact 16-bit inputs; per-(batch,
KV head) functions take one sequence at a time; GQA maps query head h to KV
head h // G.

Parity status: every function below is pinned by the CPU tests in
``tests/test_oracle_*.py`` (closed forms, invariants, special cases that
reduce to textbook/library attention, brute force on tiny inputs), except the
diagnostics at the end (kept-mass coverage, the uniform INT8 reference line's
attention), which are "parity unpinned" as measurements: they measure, they
do not define the method. The INT8 quantizer itself is pinned.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# ---------------------------------------------------------------------------
# 16-bit decoding
# ---------------------------------------------------------------------------


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE fp16 bit patterns (uint16) -> exact float64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "f16":
        return f16_to_f64(bits)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# O1: vertical-line probe (column scores)
# ---------------------------------------------------------------------------


def probe_column_scores(q_probe: np.ndarray, k: np.ndarray, T: int, sm_scale: float) -> np.ndarray:
    """Column scores of the vertical-line probe for one batch element.

    [HQ-wiki] TL;DR and "What problem it solves": vertical-line tokens are key
    columns that almost every query row attends to, found from a cheap pattern
    signal; [HQ-news] "Why preserve selected positions?": the retained set is
    the high-score positions; [HQ-abs]: "vertical-line-aware attention-pattern
    signals". Reading: the signal is the column sum of the row-normalised
    causal softmax over the last R query rows, summed over the query heads of
    a KV head (GQA):

        c[g, j] = sum_{h in group g} sum_{rows r} softmax_{j' <= pos_r}(q_{h,r} . k_{g,j'} * sm_scale)[j]

    q_probe: [Hq][R][D]; row r sits at position T - R + r (rows at negative
    positions, when T < R, are ignored). k: [Hkv][>=T][D]. Returns [Hkv][T].
    """
    Hq, R, D = q_probe.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    r_eff = min(R, T)
    rows = q_probe[:, R - r_eff:, :]
    pos = np.arange(T - r_eff, T)
    causal_out = np.arange(T)[None, :] > pos[:, None]          # [r_eff][T]
    c = np.zeros((Hkv, T), dtype=np.float64)
    for g in range(Hkv):
        kg = k[g, :T, :]
        for h in range(g * G, (g + 1) * G):
            logits = (rows[h] @ kg.T) * sm_scale
            logits[causal_out] = -np.inf
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            p = e / e.sum(axis=1, keepdims=True)
            c[g] += p.sum(axis=0)
    return c


# ---------------------------------------------------------------------------
# O2: top-k selection of the retained columns
# ---------------------------------------------------------------------------


def keep_count(T: int, window: int, keep_num: int, keep_den: int) -> int:
    """Number of retained columns k = min(floor(keep_num*T/keep_den), T - W).

    [HQ-news] "Why preserve selected positions?" / "What the authors tested":
    the top 5% of key positions plus a local window stay in high precision.
    Reading: the percentage is taken over the full context T (integer floor);
    candidates exclude the window, so the kept total is k + min(W, T).
    """
    n_cand = max(0, T - window)
    return min((keep_num * T) // keep_den, n_cand)


@dataclasses.dataclass
class Selection:
    idx: np.ndarray      # ascending int64 positions
    k: int
    tau: float           # score of the k-th ranked candidate (+inf when k == 0)
    j_k: int             # its position (-1 when k == 0)


def select_topk(c_g: np.ndarray, T: int, window: int, keep_num: int, keep_den: int) -> Selection:
    """Top-k candidates by (score descending, position ascending).

    Candidates are [0, T - W). Ties go to the lower position. Returns the
    selected set in ascending order and the threshold pair (tau, j_k) of the
    k-th ranked element, used by the append rule.
    """
    n_cand = max(0, T - window)
    k = keep_count(T, window, keep_num, keep_den)
    cand = np.arange(n_cand)
    order = np.lexsort((cand, -c_g[:n_cand]))
    top = order[:k]
    if k == 0:
        return Selection(np.zeros(0, dtype=np.int64), 0, float("inf"), -1)
    return Selection(np.sort(top).astype(np.int64), k, float(c_g[top[-1]]), int(top[-1]))


def ranks_above(c_d: float, d: int, tau: float, j_k: int) -> bool:
    """(c_d, -d) ranks above (tau, -j_k) in the selection order."""
    return (c_d > tau) or (c_d == tau and d < j_k)


# ---------------------------------------------------------------------------
# O3: asymmetric per-token INT4 quantizer (group 32, fp16 scale and zero)
# ---------------------------------------------------------------------------

INT4_GROUP = 32


def int4_quantize(x: np.ndarray):
    """Asymmetric INT4 codes per 32-channel group of each token.

    [HQ-news] "What the authors tested": the non-retained K and V are stored
    as Key-4bit / Value-4bit. Format (reading of the unspecified details):
        mn, mx = min, max over the group; d = mx - mn (exact in fp32)
        s = fp16_rne(fp32_rne(d / 15));  z = fp16_rne(mn)
        code = clamp(rint_even(fp32(x - z) / fp32 s), 0, 15), or 0 when s == 0
    The code decision is taken in fp32 (x, z, s are exact fp32 values; one
    fp32 subtraction, one correctly rounded fp32 division, round half to
    even). Dequantization x_hat = code*s + z is exact in float64.

    x: [..., D] float64 holding exact 16-bit values. Returns
    (codes uint8 [..., D], s float16 [..., D/32], z float16 [..., D/32]).
    """
    D = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (D // INT4_GROUP, INT4_GROUP))
    mn = g.min(axis=-1)
    mx = g.max(axis=-1)
    d32 = (mx - mn).astype(np.float32)
    if not np.array_equal(d32.astype(np.float64), mx - mn):
        raise ArithmeticError("group range not exact in fp32")
    s16 = (d32 / np.float32(15.0)).astype(np.float16)
    z16 = mn.astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    z32 = z16.astype(np.float32)[..., None]
    diff = g.astype(np.float32) - z32
    with np.errstate(divide="ignore", invalid="ignore"):
        qq = diff / s32
    codes = np.where(s32 > 0, np.clip(np.rint(qq), 0, 15), 0).astype(np.uint8)
    return codes.reshape(x.shape), s16, z16


def int4_dequantize(codes: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """x_hat = code * s + z per group (exact in float64)."""
    D = codes.shape[-1]
    c = codes.reshape(codes.shape[:-1] + (D // INT4_GROUP, INT4_GROUP)).astype(np.float64)
    xh = c * s16.astype(np.float64)[..., None] + z16.astype(np.float64)[..., None]
    return xh.reshape(codes.shape)


def int4_pack(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte: byte i = code[2i] | code[2i+1] << 4 (canonical order)."""
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def int4_unpack(packed: np.ndarray) -> np.ndarray:
    p = packed.astype(np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


# ---------------------------------------------------------------------------
# O4 / O6: the hybrid KV cache of one (batch, KV head)
# ---------------------------------------------------------------------------

MODE_INT4, MODE_KEPT, MODE_WINDOW = 0, 1, 2


@dataclasses.dataclass
class HybridCache:
    """Canonical (position-indexed) view of one (batch, KV head) cache.

    [HQ-wiki] flowchart / "Key results" and [HQ-news] "What hybrid-precision
    attention changes": most positions are held in low bit width, the
    vertical-line positions and the recent window in high precision.
    Reading: a retained token is stored only in 16-bit form (never also in
    INT4), which is what makes the pages' "about 15% over strict 4-bit"
    storage figure come out (see storage_ratio_vs_int4).
    """
    k: np.ndarray          # [T][D] exact 16-bit values (for kept/window rows)
    v: np.ndarray
    mode: np.ndarray       # [T] int8
    k_codes: np.ndarray    # [T][D] uint8 (valid where mode == INT4)
    v_codes: np.ndarray
    k_s: np.ndarray        # [T][D/32] float16
    k_z: np.ndarray
    v_s: np.ndarray
    v_z: np.ndarray
    window: int
    T0: int                # context length when the probe ran
    col_scores: np.ndarray  # [T0] probe scores (used by the append rule)
    tau: float
    j_k: int

    @property
    def T(self) -> int:
        return int(self.mode.shape[0])


def build_cache(k: np.ndarray, v: np.ndarray, T: int, sel: Selection, window: int,
                col_scores: np.ndarray) -> HybridCache:
    """Quantize one (b, g) sequence into the hybrid cache (O4).

    Kept set H = S u [T - W, T); every other position is INT4-quantized,
    K and V alike.
    """
    D = k.shape[-1]
    mode = np.full(T, MODE_INT4, dtype=np.int8)
    mode[sel.idx] = MODE_KEPT
    mode[max(0, T - window):T] = MODE_WINDOW
    kk = k[:T].copy()
    vv = v[:T].copy()
    kc, ks, kz = int4_quantize(kk)
    vc, vs, vz = int4_quantize(vv)
    return HybridCache(kk, vv, mode, kc, vc, ks, kz, vs, vz, window, T,
                       np.asarray(col_scores[:T], dtype=np.float64), sel.tau, sel.j_k)


def cache_kv_hat(cache: HybridCache):
    """Effective (K~, V~) seen by attention: exact on kept/window positions,
    dequantized INT4 elsewhere."""
    kq = int4_dequantize(cache.k_codes, cache.k_s, cache.k_z)
    vq = int4_dequantize(cache.v_codes, cache.v_s, cache.v_z)
    hi = (cache.mode != MODE_INT4)[:, None]
    return np.where(hi, cache.k, kq), np.where(hi, cache.v, vq)


def append_token(cache: HybridCache, k_new: np.ndarray, v_new: np.ndarray) -> HybridCache:
    """One decode-time append (O6).

    The new token p = T enters the window. The token that leaves the window,
    d = T - W (when T >= W), is kept in 16-bit form when it was probed
    (d < T0) and its probe score ranks above the k-th selected candidate (it
    would have been selected had it been a candidate), and is quantized to
    INT4 otherwise. Tokens generated after the probe always quantize when
    they leave the window. Reading of "tokens leaving the window are
    quantized unless selected".
    """
    T, W = cache.T, cache.window
    D = cache.k.shape[-1]
    k = np.vstack([cache.k, k_new.reshape(1, D)])
    v = np.vstack([cache.v, v_new.reshape(1, D)])
    mode = np.concatenate([cache.mode, [MODE_WINDOW]]).astype(np.int8)
    grow = lambda a, fill: np.concatenate([a, np.full((1,) + a.shape[1:], fill, dtype=a.dtype)])
    kc, vc = grow(cache.k_codes, 0), grow(cache.v_codes, 0)
    ks, kz, vs, vz = (grow(a, 0) for a in (cache.k_s, cache.k_z, cache.v_s, cache.v_z))
    T1 = T + 1
    for d in np.nonzero((mode == MODE_WINDOW) & (np.arange(T1) < T1 - W))[0]:
        probed = d < cache.T0
        if probed and ranks_above(float(cache.col_scores[d]), int(d), cache.tau, cache.j_k):
            mode[d] = MODE_KEPT
        else:
            mode[d] = MODE_INT4
            c1, s1, z1 = int4_quantize(k[d:d + 1])
            kc[d], ks[d], kz[d] = c1[0], s1[0], z1[0]
            c2, s2, z2 = int4_quantize(v[d:d + 1])
            vc[d], vs[d], vz[d] = c2[0], s2[0], z2[0]
    return HybridCache(k, v, mode, kc, vc, ks, kz, vs, vz, W, cache.T0, cache.col_scores,
                       cache.tau, cache.j_k)


def append_tokens(cache: HybridCache, k_rows: np.ndarray, v_rows: np.ndarray) -> HybridCache:
    """s consecutive appends (O6) in one pass: the same cache as s calls of
    append_token with the rows in order.

    Every position that has left the window after the s steps (d < T + s - W)
    and was still in it is decided by the same rule as in append_token; the
    rule depends only on d's probe score and the threshold, never on the
    order in which departures happen, so deciding them together is the same.
    k_rows, v_rows: [s][D].
    """
    T, W = cache.T, cache.window
    D = cache.k.shape[-1]
    s = k_rows.shape[0]
    k = np.vstack([cache.k, k_rows.reshape(s, D)])
    v = np.vstack([cache.v, v_rows.reshape(s, D)])
    mode = np.concatenate([cache.mode, np.full(s, MODE_WINDOW)]).astype(np.int8)
    grow = lambda a: np.concatenate([a, np.zeros((s,) + a.shape[1:], dtype=a.dtype)])
    kc, vc = grow(cache.k_codes), grow(cache.v_codes)
    ks, kz, vs, vz = (grow(a) for a in (cache.k_s, cache.k_z, cache.v_s, cache.v_z))
    T1 = T + s
    left = np.nonzero((mode == MODE_WINDOW) & (np.arange(T1) < T1 - W))[0]
    keep = np.array([d < cache.T0 and ranks_above(float(cache.col_scores[d]), int(d), cache.tau, cache.j_k)
                     for d in left], dtype=bool)
    mode[left[keep]] = MODE_KEPT
    q = left[~keep]
    mode[q] = MODE_INT4
    if len(q):
        kc[q], ks[q], kz[q] = int4_quantize(k[q])
        vc[q], vs[q], vz[q] = int4_quantize(v[q])
    return HybridCache(k, v, mode, kc, vc, ks, kz, vs, vz, W, cache.T0, cache.col_scores,
                       cache.tau, cache.j_k)


def storage_ratio_vs_int4(T: int, window: int, k: int) -> float:
    """Non-window bits per element relative to strict 4-bit storage.

    [HQ-news] "Memory and runtime costs": at 5% retention the non-window
    cache is about 15% larger than strict 4-bit. With retained tokens held
    only in 16 bits: (k*16 + (T - W - k)*4) / ((T - W)*4).
    """
    n = T - window
    return (k * 16 + (n - k) * 4) / (n * 4)


# ---------------------------------------------------------------------------
# O5: decode attention over the hybrid cache
# ---------------------------------------------------------------------------


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Plain softmax attention of G query vectors over T keys (no mask)."""
    logits = (q @ K.T) * sm_scale
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return (e @ V) / e.sum(axis=-1, keepdims=True)


def decode_attention(q_group: np.ndarray, cache: HybridCache, sm_scale: float) -> np.ndarray:
    """Decode attention of the G query heads of one KV head (O5).

    [HQ-wiki] TL;DR / "Key results" and [HQ-abs]: decode attends over the
    hybrid cache with dequantization fused into attention; numerically it is
    softmax(q K~^T * sm_scale) V~ over all T cached tokens (the current one
    included; no mask).
    """
    Kh, Vh = cache_kv_hat(cache)
    return softmax_attention(q_group, Kh, Vh, sm_scale)


# ---------------------------------------------------------------------------
# O7: prefill INT8 block quantization
# ---------------------------------------------------------------------------

INT8_BLOCK = 64


def int8_block_quantize(x: np.ndarray):
    """Symmetric INT8 per 64-token block over all channels (O7).

    [HQ-news] "What hybrid-precision attention changes" / [HQ-abs]: during
    prefill the rest of the context is processed in low precision. Format
    (reading): per block of 64 rows of one head, s = fp32_rne(max|x| / 127);
    code = clamp(rint_even(fp32 x / s), -127, 127), 0 when s == 0. Decisions
    in fp32 like the kernels.

    x: [T][D] float64 exact values. Returns (codes int8 [T][D], s float32 [ceil(T/64)]).
    """
    T, D = x.shape
    nb = (T + INT8_BLOCK - 1) // INT8_BLOCK
    codes = np.zeros((T, D), dtype=np.int8)
    scales = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        blk = x[b * INT8_BLOCK:(b + 1) * INT8_BLOCK].astype(np.float32)
        amax = np.float32(np.abs(blk).max()) if blk.size else np.float32(0)
        s = np.float32(amax / np.float32(127.0))
        scales[b] = s
        if s > 0:
            codes[b * INT8_BLOCK:(b + 1) * INT8_BLOCK] = np.clip(np.rint(blk / s), -127, 127).astype(np.int8)
    return codes, scales


# ---------------------------------------------------------------------------
# O11: OCP FP8 (E4M3) block quantization, the prefill's other low-bit format
# ---------------------------------------------------------------------------

FP8_MAX = 448.0  # largest finite E4M3 magnitude: 2^8 x 1.75


def fp8_e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 bit patterns -> float64 (O11).

    The OCP 8-bit floating point format E4M3: sign, 4 exponent bits (bias
    7), 3 mantissa bits; exponent field 0 holds the subnormals m/8 x 2^-6;
    exponent 15 with mantissa 7 is NaN (no infinities), so the largest
    finite value is 1.75 x 2^8 = 448. Written from that definition."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp8_e4m3_encode(x32: np.ndarray) -> np.ndarray:
    """float32 -> E4M3 bit patterns, round to nearest, ties to even (O11).

    The spacing of E4M3 values is 2^(e - 3) in the binade [2^e, 2^(e+1)) for
    e >= -6 and 2^-9 below 2^-6 (subnormals), so |x| rounds to an integer
    multiple of that spacing (ties to the even multiple, i.e. to the even
    mantissa). Magnitudes that round above 448 saturate to 448 (reading: the
    kernels never produce them, |x / s| <= 448 (1 + 2^-23) by construction).
    The sign of zero is kept. x32: finite float32 values."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)  # exact
    a = np.abs(x)
    _, ex = np.frexp(a)                        # a = f 2^ex, f in [1/2, 1)
    e = np.maximum(ex - 1, -6)                 # binade exponent, subnormals share e = -6
    q = np.ldexp(1.0, e - 3)                   # spacing
    r = np.rint(a / q) * q                     # a / q exact (power of two); rint: ties to even
    r = np.minimum(r, FP8_MAX)
    # bits of r: exponent field and mantissa
    _, er = np.frexp(r)
    normal = r >= 2.0 ** -6
    efield = np.where(normal, er - 1 + 7, 0)
    mant = np.where(normal, np.rint(np.ldexp(r, -(er - 1)) * 8.0) - 8.0, np.rint(np.ldexp(r, 9)))
    bits = (efield.astype(np.int64) << 3) | mant.astype(np.int64)
    bits = bits | np.where(np.signbit(x), 0x80, 0)
    return bits.astype(np.uint8)


def fp8_block_quantize(x: np.ndarray):
    """Symmetric OCP FP8 (E4M3) per 64-token block over all channels (O11).

    [HQ-wiki] "Gaps": FP8 as a third precision point is left open; the
    reading taken here mirrors O7 with the E4M3 grid: per block of 64 rows of
    one head, s = fp32_rne(max|x| / 448), code = E4M3_rne(fp32_rne(x / s)),
    all codes +0 when s == 0. The value of a code is decode(code) * s.

    x: [T][D] float64 exact values. Returns (codes uint8 [T][D], s float32 [ceil(T/64)])."""
    T, D = x.shape
    nb = (T + INT8_BLOCK - 1) // INT8_BLOCK
    codes = np.zeros((T, D), dtype=np.uint8)
    scales = np.zeros(nb, dtype=np.float32)
    for b in range(nb):
        blk = x[b * INT8_BLOCK:(b + 1) * INT8_BLOCK].astype(np.float32)
        amax = np.float32(np.abs(blk).max()) if blk.size else np.float32(0)
        s = np.float32(amax / np.float32(FP8_MAX))
        scales[b] = s
        if s > 0:
            codes[b * INT8_BLOCK:(b + 1) * INT8_BLOCK] = fp8_e4m3_encode((blk / s).astype(np.float32))
    return codes, scales


# ---------------------------------------------------------------------------
# O8: prefill hybrid-precision attention
# ---------------------------------------------------------------------------


def prefill_attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel_idx: np.ndarray,
                           window: int, sm_scale: float, q8: np.ndarray, sq: np.ndarray,
                           k8: np.ndarray, sk: np.ndarray, rows: np.ndarray,
                           route: np.ndarray | None = None) -> np.ndarray:
    """Causal hybrid-precision attention for one query head, selected rows (O8).

    [HQ-abs] (Prefill stage) and [HQ-news] "What hybrid-precision attention
    changes": selected positions and the local window are computed in full
    precision, the remaining context in low precision; [HQ-wiki] "How this
    relates to prior wiki pages": both precision paths update one softmax.

    Score of (i, j <= i):
      j in S or i - j < W : (q_i . k_j) * sm_scale              (exact)
      otherwise           : (Q8_i . K8_j) * sQ(i) * sK(j) * sm_scale
    o_i = sum_j softmax_j(score) v_j with exact V.

    q: [T][D], k, v: [T][D] (this head's KV head), q8/sq: this query head's
    INT8 codes/scales, k8/sk: the KV head's; rows: query positions to compute.
    With the FP8 low path (O11), q8 and k8 are the decoded E4M3 values
    (fp8_e4m3_decode of the codes) and sq, sk the FP8 block scales. route
    (O12, optional): bool [ceil(T/128)][ceil(T/64)]; a routed tile's
    scores are exact as well.
    Returns [len(rows)][D].
    """
    T, D = k.shape
    in_sel = np.zeros(T, dtype=bool)
    in_sel[sel_idx] = True
    k8f = k8.astype(np.float64)
    skf = sk.astype(np.float64)[np.arange(T) // INT8_BLOCK]
    out = np.empty((len(rows), D), dtype=np.float64)
    for n, i in enumerate(rows):
        i = int(i)
        j = np.arange(i + 1)
        exact = k[:i + 1] @ q[i]
        low = (k8f[:i + 1] @ q8[i].astype(np.float64)) * float(sq[i // INT8_BLOCK]) * skf[:i + 1]
        use_exact = in_sel[:i + 1] | (i - j < window)
        if route is not None:
            use_exact = use_exact | route[i // TILE_ROWS][j // INT8_BLOCK]
        logits = np.where(use_exact, exact, low) * sm_scale
        m = logits.max()
        e = np.exp(logits - m)
        out[n] = (e @ v[:i + 1]) / e.sum()
    return out


def prefill_attention_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, sel_idx: np.ndarray,
                            window: int, sm_scale: float, q8: np.ndarray, sq: np.ndarray,
                            k8: np.ndarray, sk: np.ndarray, r0: int, r1: int,
                            route: np.ndarray | None = None) -> np.ndarray:
    """Same definition as prefill_attention_rows for the contiguous rows
    [r0, r1), written with matrix products (one fp64 GEMM per precision)."""
    T, D = k.shape
    rows = np.arange(r0, r1)
    cols = np.arange(r1)
    in_sel = np.zeros(r1, dtype=bool)
    in_sel[sel_idx[sel_idx < r1]] = True
    exact = q[r0:r1] @ k[:r1].T
    low = (q8[r0:r1].astype(np.float64) @ k8[:r1].astype(np.float64).T)
    low *= sq.astype(np.float64)[rows // INT8_BLOCK][:, None]
    low *= sk.astype(np.float64)[cols // INT8_BLOCK][None, :]
    diff = rows[:, None] - cols[None, :]
    use_exact = in_sel[None, :] | (diff < window)
    if route is not None:
        use_exact = use_exact | route[rows // TILE_ROWS][:, cols // INT8_BLOCK]
    logits = np.where(use_exact, exact, low) * sm_scale
    logits[diff < 0] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    return (e @ v[:r1]) / e.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# O12: tile-level precision routing composed with the token routing
# ---------------------------------------------------------------------------

TILE_ROWS = 128  # query rows of a routed tile (the key side is one 64-token INT8 block)


def tile_route(q8: np.ndarray, k8: np.ndarray, sk: np.ndarray, T: int, window: int,
               num: int, den: int) -> np.ndarray:
    """Which (128-row query block, 64-key block) tiles take the 16-bit path (O12).

    [HQ-wiki] "How this relates to prior wiki pages" and "Gaps": TileMix
    routes tiles of the score matrix between an FP16 and an INT8 path, and
    whether that composes with HyQuant's token routing is the open
    experiment. The tile criterion is not given; reading: rank a query
    block's candidate key blocks by the INT8 score error bound of O8 (whose
    pinned form gives |q.k - Q8.K8 sQ sK| <= sQ sK ((|Q8|_1 + |K8|_1) / 2 +
    5 D / 4)), i.e. by E(kb) = fp32(sK(kb) * (A + B(kb) + 5 D / 2)) with
    A = max over the block's rows (< T) of sum|Q8_i|, B(kb) = max over the
    key block of sum|K8_j| (integers; one fp32 rounding), and route the
    floor(num * n / den) largest (ties: lower kb) of the n = kb_band
    candidate blocks, the blocks every row of the query block sees only
    below its window band: kb_band = min(nkb, max(0, (i0 - W + 1) // 64)),
    i0 = 128 qb, nkb = the blocks holding keys <= the block's last row.

    q8: [T][D] int8 codes of one query head; k8: [T][D] of its KV head; sk:
    [ceil(T/64)] fp32. Returns bool [ceil(T/128)][ceil(T/64)]."""
    D = k8.shape[1]
    nblk = (T + INT8_BLOCK - 1) // INT8_BLOCK
    nqb = (T + TILE_ROWS - 1) // TILE_ROWS
    l1q = np.abs(q8[:T].astype(np.int64)).sum(1)
    l1k = np.abs(k8[:T].astype(np.int64)).sum(1)
    Bk = np.array([l1k[j * INT8_BLOCK:(j + 1) * INT8_BLOCK].max() for j in range(nblk)])
    route = np.zeros((nqb, nblk), dtype=bool)
    for qb in range(nqb):
        i0 = qb * TILE_ROWS
        A = int(l1q[i0:min(T, i0 + TILE_ROWS)].max())
        nkb = min(nblk, (i0 + TILE_ROWS + INT8_BLOCK - 1) // INT8_BLOCK)
        kb_band = min(nkb, max(0, (i0 - window + 1) // INT8_BLOCK))
        n = num * kb_band // den
        if n == 0:
            continue
        E = (sk[:kb_band].astype(np.float32) * (A + Bk[:kb_band] + 5 * D // 2).astype(np.float32)).astype(np.float32)
        order = sorted(range(kb_band), key=lambda kb: (-float(E[kb]), kb))
        route[qb, order[:n]] = True
    return route


# ---------------------------------------------------------------------------
# Whole-batch drivers (numpy in, numpy out)
# ---------------------------------------------------------------------------


def probe_select_batch(q_probe: np.ndarray, k: np.ndarray, seq_lens, sm_scale: float,
                       window: int, keep_num: int, keep_den: int):
    """O1 + O2 for every (b, g). Returns (scores list[b] -> [Hkv][T_b],
    selections list[b][g])."""
    B = q_probe.shape[0]
    Hkv = k.shape[1]
    scores, sels = [], []
    for b in range(B):
        T = int(seq_lens[b])
        c = probe_column_scores(q_probe[b], k[b], T, sm_scale)
        scores.append(c)
        sels.append([select_topk(c[g], T, window, keep_num, keep_den) for g in range(Hkv)])
    return scores, sels


def decode_batch(q: np.ndarray, caches, sm_scale: float) -> np.ndarray:
    """O5 over the batch: q [B][Hq][D], caches[b][g] -> out [B][Hq][D]."""
    B, Hq, D = q.shape
    Hkv = len(caches[0])
    G = Hq // Hkv
    out = np.empty((B, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            out[b, g * G:(g + 1) * G] = decode_attention(q[b, g * G:(g + 1) * G], caches[b][g], sm_scale)
    return out


# ---------------------------------------------------------------------------
# Diagnostics (parity unpinned: measurements, not definitions)
# ---------------------------------------------------------------------------


def kept_mass_coverage(q_group: np.ndarray, K: np.ndarray, mode: np.ndarray, sm_scale: float) -> float:
    """Fraction of the exact attention mass that falls on kept/window tokens
    ([HQ-news] "Why preserve selected positions?" reports this for real
    models; here it is only a synthetic analogue). parity unpinned."""
    logits = (q_group @ K.T) * sm_scale
    p = np.exp(logits - logits.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return float(p[:, mode != MODE_INT4].sum(axis=-1).mean())


def int8_token_quantize(x: np.ndarray):
    """Uniform per-token INT8 of a [T][D] block (O9 reference line).

    [HQ-news] "Why preserve selected positions?": the authors compare the
    hybrid cache's operator-level error with a uniform 8-bit cache. The pages
    do not give that cache's format; reading (the plainest symmetric one):
    per token, s = fp32_rne(max_c |x[t][c]| / 127); code = clamp(rint_even(
    fp32 x / s), -127, 127); 0 when s == 0. Decisions in fp32, like the other
    quantizers here.

    x: [T][D] float64 exact values. Returns (codes int8 [T][D], s float32 [T]).
    """
    xf = x.astype(np.float32)
    s = (np.abs(xf).max(axis=1) / np.float32(127.0)).astype(np.float32)
    codes = np.zeros(x.shape, dtype=np.int8)
    nz = s > 0
    codes[nz] = np.clip(np.rint(xf[nz] / s[nz, None]), -127, 127).astype(np.int8)
    return codes, s


def uniform_int8_attention(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float) -> np.ndarray:
    """Decode attention over a cache that holds every token of K and V in
    uniform per-token INT8 (the dequantized values code * s), fp64 softmax.
    A diagnostic reference line (O9), not a path of the method."""
    kc, ks = int8_token_quantize(K)
    vc, vs = int8_token_quantize(V)
    Kh = kc.astype(np.float64) * ks.astype(np.float64)[:, None]
    Vh = vc.astype(np.float64) * vs.astype(np.float64)[:, None]
    return softmax_attention(q_group, Kh, Vh, sm_scale)


# ---------------------------------------------------------------------------
# O10: re-probing the hybrid cache from decode-time queries (a "next" step)
# ---------------------------------------------------------------------------


def bf16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 with round-half-to-even, returned as float64 (finite inputs)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def reprobe_keys(cache: HybridCache, dtype: str) -> np.ndarray:
    """The keys as a re-probe over the hybrid cache sees them (O10).

    [HQ-wiki] "Gaps": whether the vertical lines found on the prompt persist
    through decoding is left open; re-probing from decode-time attention
    tracks it. The probe takes 16-bit keys; reading: kept and window rows are
    the stored 16-bit values, INT4 rows are dequantized in fp32,
    x = code * s + z with one rounding (code * s is exact: 4 bits times an
    fp16), then rounded to the cache's 16-bit type with round half to even.

    Returns [T][D] float64 (exact 16-bit values)."""
    D = cache.k.shape[-1]
    s32 = np.repeat(cache.k_s.astype(np.float32), INT4_GROUP, axis=-1).reshape(cache.k_codes.shape)
    z32 = np.repeat(cache.k_z.astype(np.float32), INT4_GROUP, axis=-1).reshape(cache.k_codes.shape)
    x32 = (cache.k_codes.astype(np.float32) * s32 + z32).astype(np.float32)
    kq = bf16_rne(x32) if dtype == "bf16" else x32.astype(np.float16).astype(np.float64)
    hi = (cache.mode != MODE_INT4)[:, None]
    return np.where(hi, cache.k[:, :D], kq)


def reprobe(cache: HybridCache, q_recent: np.ndarray, sm_scale: float, keep_num: int, keep_den: int,
            dtype: str = "bf16"):
    """Re-probe one (batch, KV head) from its last R decode queries (O10).

    q_recent: [G][R][D] float64, row r the query issued when the cache held
    T - R + r + 1 tokens, i.e. at position T - R + r with the causal structure
    of the prompt probe's rows (O1). Scores the cached keys as reprobe_keys
    gives them, selects as O2 over the candidates [0, T - W), and counts how
    many of the new selection are already in the kept store (persistence).
    Returns (col_scores [T], Selection, n_persist)."""
    T = len(cache.mode)
    K = reprobe_keys(cache, dtype)
    c = probe_column_scores(q_recent, K[None], T, sm_scale)[0]
    sel = select_topk(c, T, cache.window, keep_num, keep_den)
    n_persist = int((cache.mode[sel.idx] == MODE_KEPT).sum())
    return c, sel, n_persist
