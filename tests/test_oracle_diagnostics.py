"""O9 diagnostics on the seeded synthetic decode inputs (CPU, oracle only).

These are measurements, not parity items ("parity unpinned"): the pages'
claims they echo are directional and made on model activations
([HQ-news] "Why preserve selected positions?": the top-5% + window kept set
covers most of the attention mass; retaining 1% or 5% in 16 bits brings the
4-bit cache's operator-level error toward a uniform 8-bit cache). The checks
assert only what the method must show on these inputs: keeping columns
lowers the error of the all-INT4 cache, keeping more lowers it further, a
uniform INT8 cache is more accurate than a uniform INT4 one, and coverage
grows with the ratio."""
import numpy as np

import oracle as O
from synth import small_decode_inputs


def _rel_l2(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_error_ordering_and_kept_mass_coverage():
    inp = small_decode_inputs(B=1, Hq=8, Hkv=2, T=2048, n_outlier=4, outlier_scale=20.0, seed=95)
    sp = inp.spec
    G = sp.Hq // sp.Hkv
    sm = 1 / np.sqrt(sp.D)
    qp, k, v = (O.to_f64(x, sp.dtype) for x in (inp.q_probe, inp.k, inp.v))
    q = O.to_f64(inp.q, sp.dtype)
    T = int(inp.seq_lens[0])
    rows = {}
    for g in range(sp.Hkv):
        qg = q[0, g * G:(g + 1) * G]
        K, V = k[0, g, :T], v[0, g, :T]
        exact = O.softmax_attention(qg, K, V, sm)
        c = O.probe_column_scores(qp[0, g * G:(g + 1) * G], k[0, g:g + 1, :T], T, sm)[0]
        err, cov = {}, {}
        for name, (num, W) in {"int4_all": (0, 0), "hybrid_1pct": (1, 128), "hybrid_5pct": (5, 128),
                               "hybrid_20pct": (20, 128)}.items():
            sel = O.select_topk(c, T, W, num, 100)
            cache = O.build_cache(K, V, T, sel, W, c)
            err[name] = _rel_l2(O.decode_attention(qg, cache, sm), exact)
            cov[name] = O.kept_mass_coverage(qg, K, cache.mode, sm)
        err["uniform_int8"] = _rel_l2(O.uniform_int8_attention(qg, K, V, sm), exact)
        rows[g] = (err, cov)
        print(f"g={g}: rel-L2 vs exact {err}; kept-mass coverage {cov}", flush=True)
        assert err["int4_all"] > err["hybrid_1pct"] > err["hybrid_5pct"] > err["hybrid_20pct"]
        assert err["uniform_int8"] < err["int4_all"]
        assert cov["int4_all"] == 0.0
        assert 0.0 < cov["hybrid_1pct"] < cov["hybrid_5pct"] < cov["hybrid_20pct"] <= 1.0
