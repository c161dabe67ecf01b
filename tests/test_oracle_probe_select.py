"""Pins for the oracle's vertical-line probe and top-k selection."""
import math

import numpy as np
import pytest

import oracle as O
from synth import CONFIGS


def _rand(seed, shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_column_scores_sum_to_rows_times_heads():
    """Each probe row's softmax sums to 1, so sum_j c[g, j] = G * R."""
    Hq, Hkv, R, T, D = 8, 2, 16, 300, 32
    q = _rand(1, (Hq, R, D))
    k = _rand(2, (Hkv, T, D))
    c = O.probe_column_scores(q, k, T, 1 / math.sqrt(D))
    G = Hq // Hkv
    assert np.allclose(c.sum(axis=1), G * R, rtol=0, atol=1e-9)
    assert np.all(c >= 0)


def test_column_scores_identical_keys_closed_form():
    """All keys equal => every row is uniform over its causal prefix:
    c[g, j] = G * sum_{rows r at position p >= j} 1 / (p + 1)."""
    Hq, Hkv, R, T, D = 4, 1, 8, 20, 16
    q = _rand(3, (Hq, R, D))
    k = np.tile(_rand(4, (1, 1, D)), (Hkv, T, 1))
    c = O.probe_column_scores(q, k, T, 0.3)
    pos = np.arange(T - R, T)
    expect = np.array([Hq * sum(1.0 / (p + 1) for p in pos if p >= j) for j in range(T)])
    assert np.allclose(c[0], expect, rtol=1e-12, atol=1e-14)


def test_column_scores_brute_force_loops():
    """Explicit scalar loops (math.exp) at tiny size, including T < R."""
    for (Hq, Hkv, R, T, D) in [(4, 2, 6, 11, 8), (2, 1, 8, 5, 4)]:
        q = _rand(5 + T, (Hq, R, D))
        k = _rand(6 + T, (Hkv, T, D), 2.0)
        sm = 1 / math.sqrt(D)
        c = O.probe_column_scores(q, k, T, sm)
        G = Hq // Hkv
        ref = np.zeros((Hkv, T))
        for h in range(Hq):
            g = h // G
            for r in range(R):
                p = T - R + r
                if p < 0:
                    continue
                logit = [sum(q[h, r, d] * k[g, j, d] for d in range(D)) * sm for j in range(p + 1)]
                mx = max(logit)
                ex = [math.exp(x - mx) for x in logit]
                tot = sum(ex)
                for j in range(p + 1):
                    ref[g, j] += ex[j] / tot
        assert np.allclose(c, ref, rtol=1e-12, atol=1e-15)


def test_column_scores_invariant_to_head_order_within_group():
    Hq, Hkv, R, T, D = 8, 2, 8, 64, 16
    q = _rand(7, (Hq, R, D))
    k = _rand(8, (Hkv, T, D))
    c1 = O.probe_column_scores(q, k, T, 0.25)
    perm = np.array([2, 0, 3, 1, 7, 5, 4, 6])       # permutes inside each group of 4
    c2 = O.probe_column_scores(q[perm], k, T, 0.25)
    assert np.allclose(c1, c2, rtol=1e-13, atol=1e-15)


def test_planted_column_is_found():
    """A key aligned with every probe query is the top column."""
    Hq, Hkv, R, T, D = 4, 1, 16, 400, 32
    q = _rand(9, (Hq, R, D)) + 1.0
    k = _rand(10, (Hkv, T, D))
    k[0, 57] = 3.0 * np.ones(D)
    c = O.probe_column_scores(q, k, T, 1 / math.sqrt(D))
    sel = O.select_topk(c[0], T, 128, 5, 100)
    assert 57 in sel.idx and int(np.argmax(c[0][: T - 128])) == 57


# ---------------------------------------------------------------- selection


def _brute_topk(c, T, W, num, den):
    n = max(0, T - W)
    k = min(num * T // den, n)
    ranked = sorted(range(n), key=lambda j: (-c[j], j))
    return sorted(ranked[:k]), (ranked[k - 1] if k else -1)


@pytest.mark.parametrize("T,W,num,den", [(500, 128, 5, 100), (512, 64, 1, 100), (300, 128, 37, 100),
                                         (100, 128, 5, 100), (129, 128, 5, 100), (400, 0, 5, 100)])
def test_select_matches_full_stable_sort(T, W, num, den):
    rng = np.random.default_rng(T + W + num)
    c = rng.random(T)
    c[rng.integers(0, T, 40)] = 0.5                     # exact ties
    c[:10] = c[10]                                      # a run of ties
    sel = O.select_topk(c, T, W, num, den)
    ref, jk = _brute_topk(c, T, W, num, den)
    assert list(sel.idx) == ref
    assert sel.j_k == jk
    if ref:
        assert sel.tau == c[jk]


def test_select_ratio_100_percent_keeps_every_candidate():
    c = np.random.default_rng(0).random(1000)
    sel = O.select_topk(c, 1000, 128, 100, 100)
    assert list(sel.idx) == list(range(872))


def test_select_lower_index_wins_ties():
    c = np.zeros(400)
    c[[10, 20, 30, 40]] = 1.0
    sel = O.select_topk(c, 400, 128, 1, 100)            # k = 4
    assert list(sel.idx) == [10, 20, 30, 40]
    sel = O.select_topk(c, 400, 128, 1, 200)            # k = 2
    assert list(sel.idx) == [10, 20] and sel.j_k == 20 and sel.tau == 1.0
    assert O.ranks_above(1.0, 15, sel.tau, sel.j_k)
    assert not O.ranks_above(1.0, 25, sel.tau, sel.j_k)


@pytest.mark.parametrize("T,k_expect", [(4096, 204), (32768, 1638), (131072, 6553), (16384, 819)])
def test_kept_count_is_top5_percent_plus_window(T, k_expect):
    """Kept total = floor(5T/100) + 128 at every workload length."""
    k = O.keep_count(T, 128, 5, 100)
    assert k == k_expect
    assert k + min(128, T) == T * 5 // 100 + 128


def test_kept_count_ragged_lengths():
    for T in [16384, 20000, 40001, 65536]:
        assert O.keep_count(T, 128, 5, 100) == T // 20
    assert O.keep_count(100, 128, 5, 100) == 0          # whole context is the window
    assert O.keep_count(130, 128, 5, 100) == 2          # capped by the 2 candidates


def test_workload_lengths_match_kept_counts():
    for name, spec in CONFIGS.items():
        if spec.T and hasattr(spec, "append_steps"):
            assert O.keep_count(spec.T, spec.window, 5, 100) == spec.T // 20
