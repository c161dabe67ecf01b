"""Pins for the oracle's cache build, decode attention, append rule and
prefill hybrid attention: special cases that reduce to textbook or library
softmax attention, brute-force loops, invariants, and the pages' storage
figure."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from synth import bf16_bits_from_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16(x):
    return O.bf16_to_f64(bf16_bits_from_f32(np.asarray(x, dtype=np.float32)))


def _kv(seed, T, D=128, outliers=True):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, D), dtype=np.float32)
    if outliers:
        k[:, [1, D // 2, (3 * D) // 4, D - 1]] *= 20
    v = rng.standard_normal((T, D), dtype=np.float32)
    return _bf16(k), _bf16(v)


def _sdpa(q, K, V, sm, causal=False):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sm, is_causal=causal)
    return o[0, 0].numpy()


def _cache(k, v, T, W, num, den, seed=0):
    c = np.random.default_rng(seed).random(T)
    sel = O.select_topk(c, T, W, num, den)
    return O.build_cache(k, v, T, sel, W, c), sel, c


# ---------------------------------------------------------------- decode


def test_decode_ratio_100_equals_exact_attention():
    T, D = 700, 128
    k, v = _kv(1, T)
    q = _bf16(np.random.default_rng(2).standard_normal((4, D)))
    cache, sel, _ = _cache(k, v, T, 128, 100, 100)
    assert np.all(cache.mode != O.MODE_INT4)
    sm = 1 / math.sqrt(D)
    out = O.decode_attention(q, cache, sm)
    assert np.allclose(out, _sdpa(q, k, v, sm), rtol=1e-12, atol=1e-13)


def test_decode_window_covering_context_equals_exact_attention():
    T, D = 300, 128
    k, v = _kv(3, T)
    q = _bf16(np.random.default_rng(4).standard_normal((2, D)))
    cache, _, _ = _cache(k, v, T, 512, 5, 100)
    sm = 1 / math.sqrt(D)
    assert np.allclose(O.decode_attention(q, cache, sm), _sdpa(q, k, v, sm), rtol=1e-12, atol=1e-13)


def test_decode_all_quantized_brute_force():
    """ratio 0, W = 0: attention over the fully dequantized cache, written as
    scalar loops (per-element dequant, explicit softmax)."""
    T, D = 40, 64
    k, v = _kv(5, T, D)
    q = _bf16(np.random.default_rng(6).standard_normal((1, D)))
    cache, sel, _ = _cache(k, v, T, 0, 0, 100)
    assert len(sel.idx) == 0 and np.all(cache.mode == O.MODE_INT4)
    sm = 0.125
    kh = np.zeros((T, D))
    vh = np.zeros((T, D))
    for t in range(T):
        for d in range(D):
            g = d // 32
            kh[t, d] = int(cache.k_codes[t, d]) * float(cache.k_s[t, g]) + float(cache.k_z[t, g])
            vh[t, d] = int(cache.v_codes[t, d]) * float(cache.v_s[t, g]) + float(cache.v_z[t, g])
    logit = [sum(q[0, d] * kh[t, d] for d in range(D)) * sm for t in range(T)]
    mx = max(logit)
    w = [math.exp(x - mx) for x in logit]
    ref = [sum(w[t] * vh[t, d] for t in range(T)) / sum(w) for d in range(D)]
    out = O.decode_attention(q, cache, sm)
    assert np.allclose(out[0], ref, rtol=1e-12, atol=1e-13)


def test_decode_invariant_to_key_order():
    T, D = 400, 128
    k, v = _kv(7, T)
    q = _bf16(np.random.default_rng(8).standard_normal((4, D)))
    cache, _, _ = _cache(k, v, T, 128, 5, 100)
    kh, vh = O.cache_kv_hat(cache)
    perm = np.random.default_rng(9).permutation(T)
    sm = 1 / math.sqrt(D)
    a = O.softmax_attention(q, kh, vh, sm)
    b = O.softmax_attention(q, kh[perm], vh[perm], sm)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
    assert np.allclose(a, O.decode_attention(q, cache, sm), rtol=0, atol=0)


def test_cache_modes_and_kept_count():
    T = 4096
    k, v = _kv(10, T)
    cache, sel, _ = _cache(k, v, T, 128, 5, 100)
    assert (cache.mode == O.MODE_KEPT).sum() == 204
    assert (cache.mode == O.MODE_WINDOW).sum() == 128
    assert (cache.mode == O.MODE_INT4).sum() == T - 204 - 128
    assert np.all(cache.mode[T - 128:] == O.MODE_WINDOW)


# ---------------------------------------------------------------- append


def test_append_equals_rebuild_from_scratch():
    """After s appends the cache equals a fresh build over [0, T0 + s) whose
    kept set is S plus the flagged departures, with the last W as window."""
    T0, W, D, steps = 600, 128, 128, 200
    k, v = _kv(11, T0 + steps)
    c = np.random.default_rng(12).random(T0)
    c[T0 - W:] *= 0.01         # window tokens rank low ...
    c[T0 - W + 5] = 10.0       # window tokens that outrank the k-th candidate
    c[T0 - W + 17] = 9.0
    sel = O.select_topk(c, T0, W, 5, 100)
    cache = O.build_cache(k, v, T0, sel, W, c)
    for s in range(steps):
        cache = O.append_token(cache, k[T0 + s], v[T0 + s])
    T = T0 + steps
    flagged = [d for d in range(T0 - W, T0) if O.ranks_above(c[d], d, sel.tau, sel.j_k)]
    assert flagged == [T0 - W + 5, T0 - W + 17]
    kept = np.sort(np.concatenate([sel.idx, flagged])).astype(np.int64)
    fresh = O.build_cache(k, v, T, O.Selection(kept, len(kept), sel.tau, sel.j_k), W, c)
    assert np.array_equal(cache.mode, fresh.mode)
    q4 = cache.mode == O.MODE_INT4
    for a in ("k_codes", "v_codes"):
        assert np.array_equal(getattr(cache, a)[q4], getattr(fresh, a)[q4])
    for a in ("k_s", "k_z", "v_s", "v_z"):
        assert np.array_equal(getattr(cache, a)[q4].view(np.uint16), getattr(fresh, a)[q4].view(np.uint16))
    q = _bf16(np.random.default_rng(13).standard_normal((4, D)))
    assert np.allclose(O.decode_attention(q, cache, 0.088), O.decode_attention(q, fresh, 0.088),
                       rtol=0, atol=1e-15)


def test_append_before_window_fills():
    """While T < W nothing departs; with W = 0 a new token quantizes at once."""
    T0, D = 50, 128
    k, v = _kv(14, T0 + 3)
    c = np.ones(T0)
    cache = O.build_cache(k, v, T0, O.select_topk(c, T0, 128, 5, 100), 128, c)
    cache = O.append_token(cache, k[T0], v[T0])
    assert np.all(cache.mode == O.MODE_WINDOW) and cache.T == T0 + 1
    cache0 = O.build_cache(k, v, T0, O.select_topk(c, T0, 0, 0, 100), 0, c)
    cache0 = O.append_token(cache0, k[T0], v[T0])
    assert np.all(cache0.mode == O.MODE_INT4)


# ---------------------------------------------------------------- storage


def test_storage_overhead_matches_pages():
    """The pages: ~15% more non-window cache than strict 4-bit at 5%."""
    with open(os.path.join(GOLDEN, "storage_overhead.json")) as f:
        g = json.load(f)
    T, W = g["T"], g["window"]
    k = O.keep_count(T, W, 5, 100)
    r = O.storage_ratio_vs_int4(T, W, k)
    assert abs(r - 1.0 - g["pages_overhead"]) < g["pages_tolerance"]
    assert round(r, 4) == g["closed_form_ratio"]


# ---------------------------------------------------------------- prefill


def _prefill_inputs(T, D, Hq=1, seed=20):
    rng = np.random.default_rng(seed)
    q = _bf16(rng.standard_normal((T, D)))
    k, v = _kv(seed + 1, T, D)
    q8, sq = O.int8_block_quantize(q)
    k8, sk = O.int8_block_quantize(k)
    return q, k, v, q8, sq, k8, sk


def test_prefill_ratio_100_equals_exact_causal_attention():
    """Every j <= i is selected or inside the row window => exact attention."""
    T, D, W = 500, 128, 128
    q, k, v, q8, sq, k8, sk = _prefill_inputs(T, D)
    sel = np.arange(T - W)                   # ratio 100%: all candidates
    sm = 1 / math.sqrt(D)
    out = O.prefill_attention_block(q, k, v, sel, W, sm, q8, sq, k8, sk, 0, T)
    assert np.allclose(out, _sdpa(q, k, v, sm, causal=True), rtol=1e-11, atol=1e-12)


def test_prefill_window_covering_context_is_exact():
    T, D = 200, 128
    q, k, v, q8, sq, k8, sk = _prefill_inputs(T, D, seed=30)
    sm = 1 / math.sqrt(D)
    out = O.prefill_attention_block(q, k, v, np.zeros(0, dtype=np.int64), 256, sm, q8, sq, k8, sk, 0, T)
    assert np.allclose(out, _sdpa(q, k, v, sm, causal=True), rtol=1e-11, atol=1e-12)


def test_prefill_brute_force_loops():
    """Explicit per-element loops at T = 150 with a random selected set."""
    T, D, W = 150, 32, 40
    q, k, v, q8, sq, k8, sk = _prefill_inputs(T, D, seed=40)
    sel = np.sort(np.random.default_rng(41).choice(T - W, 7, replace=False))
    sm = 0.2
    rows = np.array([0, 1, 39, 40, 41, 63, 64, 65, 100, 149])
    out = O.prefill_attention_rows(q, k, v, sel, W, sm, q8, sq, k8, sk, rows)
    blk = O.prefill_attention_block(q, k, v, sel, W, sm, q8, sq, k8, sk, 0, T)
    for n, i in enumerate(rows):
        logit = []
        for j in range(i + 1):
            if j in set(sel.tolist()) or i - j < W:
                s = sum(q[i, d] * k[j, d] for d in range(D))
            else:
                s = sum(int(q8[i, d]) * int(k8[j, d]) for d in range(D)) * float(sq[i // 64]) * float(sk[j // 64])
            logit.append(s * sm)
        mx = max(logit)
        w = [math.exp(x - mx) for x in logit]
        ref = [sum(w[j] * v[j, d] for j in range(i + 1)) / sum(w) for d in range(D)]
        assert np.allclose(out[n], ref, rtol=1e-11, atol=1e-12)
        assert np.allclose(blk[i], ref, rtol=1e-11, atol=1e-12)


def test_prefill_int8_score_error_bound():
    """One 64-row block: |q.k - Q8.K8 sQ sK| <= sK/2 sum|q| + sQ/2 sum|k| + 3 D sQ sK / 4."""
    T, D = 64, 128
    q, k, v, q8, sq, k8, sk = _prefill_inputs(T, D, seed=50)
    exact = q @ k.T
    low = (q8.astype(np.float64) @ k8.astype(np.float64).T) * float(sq[0]) * float(sk[0])
    s_q, s_k = float(sq[0]), float(sk[0])
    bound = (s_k / 2) * np.abs(q).sum(1)[:, None] + (s_q / 2) * np.abs(k).sum(1)[None, :] + 3 * D * s_q * s_k / 4
    assert np.all(np.abs(exact - low) <= bound + 1e-12)
