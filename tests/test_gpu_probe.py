"""GPU parity of hq_probe_select: column scores against the fp64 oracle,
the selected index sets (bit-exact, lower-index tie-break; flips allowed
only between near-ties whose oracle scores differ by < 1e-6 relative, each
counted and reported), and the top-k applied to the GPU's own fp32 scores
(bit-exact)."""
import math

import numpy as np
import pytest

import oracle as O
from synth import small_decode_inputs
from synth.inputs import bf16_bits_from_f32

from gpu_common import SCORE_RTOL, compare_selection, fp32_scale, ints_to_dev, to_dev

pytestmark = pytest.mark.gpu


def run_probe(inp, window, keep):
    import kv_cache_amd as hq
    sp = inp.spec
    pol = hq.Policy(keep[0], keep[1], window, sp.probe_rows)
    col, sel, cnt, thr = hq.probe_select(to_dev(inp.q_probe, sp.dtype), to_dev(inp.k, sp.dtype),
                                         ints_to_dev(inp.seq_lens), pol)
    return tuple(t.cpu().numpy() for t in (col, sel, cnt, thr))


def check_probe(inp, window=128, keep=(5, 100), rel_tol=SCORE_RTOL, sample=None, floor=0.0):
    """floor > 0: oracle scores below it (under the fp32 range the scores are
    returned in) are checked to be at most the floor instead of relatively."""
    sp = inp.spec
    col, sel, cnt, thr = run_probe(inp, window, keep)
    sm = fp32_scale(sp.D)
    qp = O.to_f64(inp.q_probe, sp.dtype)
    flips, worst = 0, 0.0
    pairs = sample or [(b, g) for b in range(sp.B) for g in range(sp.Hkv)]
    for (b, g) in pairs:
        T = int(inp.seq_lens[b])
        c_or = O.probe_column_scores(qp[b, g * (sp.Hq // sp.Hkv):(g + 1) * (sp.Hq // sp.Hkv)],
                                     O.to_f64(inp.k[b, g:g + 1], sp.dtype), T, sm)[0]
        big = c_or >= floor
        rel = np.abs(col[b, g, :T].astype(np.float64) - c_or)[big] / np.maximum(c_or[big], 1e-300)
        worst = max(worst, float(rel.max()))
        assert rel.max() <= rel_tol, (b, g, float(rel.max()))
        assert np.all(col[b, g, :T][~big] <= floor), (b, g)
        assert np.all(col[b, g, T:] == 0)
        flips += compare_selection(sel[b, g, : cnt[b, g]], int(cnt[b, g]), c_or, T, window, keep)
        # the top-k stage alone: the oracle's selection on the GPU's own fp32 scores
        s32 = O.select_topk(col[b, g, :T].astype(np.float64), T, window, keep[0], keep[1])
        assert np.array_equal(sel[b, g, : cnt[b, g]], s32.idx), (b, g)
        assert np.all(sel[b, g, cnt[b, g]:] == -1)
        assert int(thr[b, g, 1]) == s32.j_k
        tau = float(thr[b, g, 0:1].view(np.float32)[0])
        assert (tau == s32.tau) or (s32.k == 0 and math.isinf(tau))
    print(f"probe: max rel err {worst:.3e}, near-tie flips {flips}", flush=True)
    return flips


@pytest.mark.parametrize("kw,window,keep", [
    (dict(B=2, Hq=8, Hkv=2, T=700, ragged_min=389, seed=41), 128, (5, 100)),
    (dict(B=1, Hq=1, Hkv=1, T=1000, dtype="f16", seed=42), 128, (5, 100)),
    (dict(B=2, Hq=16, Hkv=2, T=2500, ragged_min=1100, n_outlier=8, outlier_scale=30.0, plant_frac=0.01,
          seed=43), 128, (5, 100)),
    (dict(B=2, Hq=4, Hkv=2, T=1500, seed=44), 128, (1, 100)),
    (dict(B=1, Hq=4, Hkv=1, T=600, seed=45), 128, (100, 100)),
    (dict(B=2, Hq=2, Hkv=1, T=40, seed=46), 128, (5, 100)),        # T < probe rows, T < window
    (dict(B=1, Hq=8, Hkv=1, T=300, probe_rows=16, seed=47), 64, (5, 100)),
])
def test_probe_matches_oracle(kw, window, keep):
    inp = small_decode_inputs(window=window, **kw)
    check_probe(inp, window, keep)


def test_probe_exact_ties_take_lower_index():
    """Copies of a key row placed before every probe row give exactly equal
    column scores; among the tied columns the selection must be a prefix in
    position order."""
    inp = small_decode_inputs(B=1, Hq=4, Hkv=1, T=800, seed=48)
    inp.k[0, 0, 100:400] = inp.k[0, 0, 0]   # token 0 is a planted vertical line
    flips = check_probe(inp, 128, (5, 100))
    assert flips == 0
    col, sel, cnt, thr = run_probe(inp, 128, (5, 100))
    tied = np.array([0] + list(range(100, 400)))
    assert np.all(col[0, 0, tied] == col[0, 0, 0])
    chosen = sorted(set(sel[0, 0, : cnt[0, 0]].tolist()) & set(tied.tolist()))
    assert chosen == sorted(tied.tolist())[: len(chosen)]
    print(f"tied columns selected: {len(chosen)} of {len(tied)}")


def test_probe_logit_range_beyond_reference():
    """Logits spanning far more than 2^9 in log2 units inside one key chunk:
    the probe's per-row reference has to move (the rare rescale path). All
    probe rows share a direction u; keys 300..450 lie along u, giving logits
    ~600 (log2 units) above the other keys, so nearly all of the softmax
    mass, and every selected column, is on that plateau, while the other
    columns' scores fall below the fp32 range."""
    inp = small_decode_inputs(B=1, Hq=4, Hkv=1, T=1500, seed=49)
    rng = np.random.default_rng(4949)
    u = np.ones(128, dtype=np.float32)
    qp = u + 0.3 * rng.standard_normal(inp.q_probe.shape, dtype=np.float32)
    kp = 37.0 * u + rng.standard_normal((151, 128), dtype=np.float32)
    inp.q_probe[...] = bf16_bits_from_f32(qp)
    inp.k[0, 0, 300:451] = bf16_bits_from_f32(kp)
    sm = fp32_scale(128)
    logits = O.to_f64(inp.q_probe, "bf16")[0, 0] @ O.to_f64(inp.k, "bf16")[0, 0].T * sm / math.log(2)
    assert logits[:, 300:451].min() - logits[:, :300].max() > 512
    check_probe(inp, 128, (5, 100), floor=1e-30)


def test_probe_logits_far_below_zero():
    """Every logit near -1.5e6 in log2 units: channel 0 carries 29,952 in
    every probe query and -392 in every key (a constant -1.498e6 added to
    each logit; the other channels are the seeded N(0, 1) values, so the
    softmax is that of an ordinary probe). Far below any fixed starting
    reference, each row's reference has to be taken from its first valid
    logit however negative (a row that kept a placeholder reference would
    see all its terms underflow and drop out of the scores)."""
    inp = small_decode_inputs(B=1, Hq=4, Hkv=1, T=900, seed=53)
    q = O.to_f64(inp.q_probe, "bf16").astype(np.float32)
    k = O.to_f64(inp.k, "bf16").astype(np.float32)
    q[..., 0] = 29952.0
    k[..., 0] = -392.0
    inp.q_probe[...] = bf16_bits_from_f32(q)
    inp.k[...] = bf16_bits_from_f32(k)
    sm = fp32_scale(128)
    z = O.to_f64(inp.q_probe, "bf16")[0].reshape(-1, 128) @ O.to_f64(inp.k, "bf16")[0, 0].T * sm / math.log(2)
    assert z.max() < -2.0 ** 20 - 1000 and z.max() - z.min() < 200
    check_probe(inp, 128, (5, 100), floor=1e-30)


def _reference_move_inputs():
    """All probe rows along one direction u; every key near zero except 8
    keys (300..307) along u whose logits sit ~103 log2 units higher. The
    probe's key chunks are 256 keys here, so in the chunk of keys 256..511
    every row's reference is set by the tile of keys 256..287 and then has to
    move (by more than 100) at the tile holding the 8 keys; the terms already
    stored for keys 256..287 are rescaled by that power of two and stay
    normal fp32 numbers, so every score keeps the relative bound (the scores
    of the near-zero keys are 1e-32 .. 1e-30: a key is seen by fewer probe
    rows the later it is)."""
    inp = small_decode_inputs(B=1, Hq=4, Hkv=1, T=1500, seed=51)
    rng = np.random.default_rng(5151)
    u = np.ones(128, dtype=np.float32)
    inp.q_probe[...] = bf16_bits_from_f32(u + 0.05 * rng.standard_normal(inp.q_probe.shape, dtype=np.float32))
    k = 0.05 * rng.standard_normal((1500, 128), dtype=np.float32)
    k[300:308] += 6.35 * u
    inp.k[0, 0] = bf16_bits_from_f32(k)
    return inp


def test_probe_reference_move_rescales_stored_terms():
    inp = _reference_move_inputs()
    sm = fp32_scale(128)
    z = O.to_f64(inp.q_probe, "bf16")[0].reshape(-1, 128) @ O.to_f64(inp.k, "bf16")[0, 0].T * sm / math.log(2)
    ref0 = np.ceil(z[:, 256:288].max(axis=1))                     # each row's reference after keys 256..287
    assert np.all(z[:, 300:308].max(axis=1) - ref0 > 100)         # every row's reference moves
    assert np.all(z[:, 256:288].min(axis=1) - np.ceil(z[:, 300:308].max(axis=1)) > -126)  # rescaled terms stay normal
    assert np.all(z.max(axis=1) - z.min(axis=1) < 120)           # no term below fp32's normal range anywhere
    c_or = O.probe_column_scores(O.to_f64(inp.q_probe, "bf16")[0], O.to_f64(inp.k[0, 0:1], "bf16"), 1500, sm)[0]
    assert c_or.min() > 1e-36                                     # normal fp32 scores, all checked relatively
    check_probe(inp, 128, (5, 100))


def test_probe_at_the_16k_prefill_shape():
    """The 16K prefill's probe (B=1, 32 query / 8 KV heads, its last 64 rows):
    the only workload whose pass 1 runs on 512-key chunks (two per pass-2
    block). Every (b, g) against the oracle."""
    import types
    from synth.inputs import CONFIGS, make_prefill_inputs
    pin = make_prefill_inputs(CONFIGS["prefill_8b_16k"])
    sp = pin.spec
    inp = types.SimpleNamespace(
        spec=types.SimpleNamespace(B=sp.B, Hq=sp.Hq, Hkv=sp.Hkv, D=sp.D, dtype=sp.dtype, probe_rows=sp.probe_rows),
        q_probe=np.ascontiguousarray(pin.q[:, :, sp.T - sp.probe_rows:]), k=pin.k,
        seq_lens=np.full(sp.B, sp.T, dtype=np.int32))
    flips = check_probe(inp, 128, (5, 100))
    print(f"16K prefill probe: near-tie flips {flips}", flush=True)
