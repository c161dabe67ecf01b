"""CPU pins of O10, re-probing the hybrid cache from decode-time queries.

Pinned against the prompt probe (O1/O2, itself pinned elsewhere) in the two
cases where the re-probe's keys must equal the prompt's keys exactly, and
against a brute-force loop for the dequantize-and-round step."""
import numpy as np

import oracle as O
from synth import bf16_bits_from_f32


def _bf16(rng, shape, scale=1.0):
    return O.to_f64(bf16_bits_from_f32((rng.standard_normal(shape) * scale).astype(np.float32)), "bf16")


def test_reprobe_all_kept_equals_prompt_probe():
    """Every candidate selected (ratio 100%): the cache holds K exactly, so the
    re-probe from the same rows is the prompt probe, scores and selection."""
    rng = np.random.default_rng(101)
    T, G, R, D, W = 700, 4, 64, 128, 128
    k, v = _bf16(rng, (T, D)), _bf16(rng, (T, D))
    q = _bf16(rng, (G, R, D))
    sm = float(np.float32(1 / np.sqrt(D)))
    c = O.probe_column_scores(q, k[None], T, sm)[0]
    sel = O.select_topk(c, T, W, 100, 100)
    assert sel.k == T - W
    cache = O.build_cache(k, v, T, sel, W, c)
    assert not (cache.mode == O.MODE_INT4).any()
    assert np.array_equal(O.reprobe_keys(cache, "bf16"), k)
    c2, sel2, n = O.reprobe(cache, q, sm, 5, 100)
    ref = O.select_topk(c, T, W, 5, 100)
    assert np.array_equal(c2, c)
    assert np.array_equal(sel2.idx, ref.idx) and n == ref.k


def _grid_keys(rng, T, D):
    """Rows whose 32-channel groups lie on an INT4 grid z + code * s with codes
    0 and 15 present, s a power of two, every value exact in bf16: the INT4
    quantizer reproduces them and the dequantized keys equal them."""
    codes = rng.integers(0, 16, size=(T, D // 32, 32))
    codes[..., 0], codes[..., 1] = 0, 15
    s = np.ldexp(1.0, rng.integers(-5, -2, size=(T, D // 32, 1)))
    z = rng.integers(-40, 20, size=(T, D // 32, 1)) / 16.0
    return (z + codes * s).reshape(T, D)


def test_reprobe_on_int4_grid_keys_equals_prompt_probe_and_persists():
    rng = np.random.default_rng(102)
    T, G, R, D, W = 900, 4, 64, 128, 128
    k = _grid_keys(rng, T, D)
    assert np.array_equal(O.to_f64(bf16_bits_from_f32(k.astype(np.float32)), "bf16"), k)
    v = _bf16(rng, (T, D))
    q = _bf16(rng, (G, R, D), 0.5)
    sm = float(np.float32(1 / np.sqrt(D)))
    c = O.probe_column_scores(q, k[None], T, sm)[0]
    sel = O.select_topk(c, T, W, 5, 100)
    cache = O.build_cache(k, v, T, sel, W, c)
    assert (cache.mode == O.MODE_INT4).sum() == T - W - sel.k
    assert np.array_equal(O.reprobe_keys(cache, "bf16"), k)
    c2, sel2, n = O.reprobe(cache, q, sm, 5, 100)
    assert np.array_equal(c2, c)
    assert np.array_equal(sel2.idx, sel.idx)
    assert n == sel.k  # the same rows re-select the kept columns


def test_reprobe_keys_brute_force():
    """Element by element: fp32 code * s + z (one rounding), then RNE to bf16
    (or fp16), on a tiny cache; kept and window rows are the stored values."""
    rng = np.random.default_rng(103)
    T, D, W = 70, 128, 16
    k, v = _bf16(rng, (T, D), 3.0), _bf16(rng, (T, D))
    c = rng.random(T)
    sel = O.select_topk(c, T, W, 10, 100)
    cache = O.build_cache(k, v, T, sel, W, c)
    for dtype in ("bf16", "f16"):
        got = O.reprobe_keys(cache, dtype)
        for t in range(T):
            for ch in range(0, D, 7):
                if cache.mode[t] != O.MODE_INT4:
                    assert got[t, ch] == k[t, ch]
                    continue
                g = ch // 32
                x = np.float32(np.float32(int(cache.k_codes[t, ch])) * np.float32(cache.k_s[t, g]) +
                               np.float32(cache.k_z[t, g]))
                if dtype == "f16":
                    want = float(np.float16(x))
                else:
                    bits = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
                    lsb = (bits >> 16) & 1
                    want = float(np.array([((bits + 0x7FFF + lsb) >> 16) << 16], dtype=np.uint32).view(np.float32)[0])
                assert got[t, ch] == want, (dtype, t, ch)


def test_reprobe_persistence_counts_the_overlap():
    """Fresh queries: the persistence count is the size of the intersection of
    the new selection with the kept set, counted here with Python sets."""
    rng = np.random.default_rng(104)
    T, G, R, D, W = 600, 2, 32, 128, 64
    k, v = _bf16(rng, (T, D)), _bf16(rng, (T, D))
    sm = float(np.float32(1 / np.sqrt(D)))
    q0 = _bf16(rng, (G, R, D))
    c = O.probe_column_scores(q0, k[None], T, sm)[0]
    sel = O.select_topk(c, T, W, 10, 100)
    cache = O.build_cache(k, v, T, sel, W, c)
    q1 = 0.5 * q0 + _bf16(rng, (G, R, D), 0.5)
    c2, sel2, n = O.reprobe(cache, q1, sm, 10, 100)
    assert sel2.k == sel.k
    kept = {t for t in range(T) if cache.mode[t] == O.MODE_KEPT}
    assert kept == set(sel.idx.tolist())
    assert n == len(kept & set(sel2.idx.tolist()))
    assert 0 < n < sel.k  # the overlap is partial for these queries
