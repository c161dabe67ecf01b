"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: the whole decode path (probe -> select -> quantize ->
[appends] -> decode) on the 8B 32K, 8B 128K (+64 appends) and ragged
70B-like workloads, checked against the oracle on sampled (batch, KV head)
pairs (the oracle recomputes each sampled pair completely)."""
import math

import numpy as np
import pytest

import oracle as O
from synth.inputs import CONFIGS, make_append_tokens, make_decode_inputs

from gpu_common import assert_attn_close, ints_to_dev, to_dev
from hq_layout import read_cache
from test_gpu_probe import compare_selection

pytestmark = pytest.mark.gpu


def _pipeline(spec, inp, cap_extra=0):
    import torch
    import kv_cache_amd as hq
    pol = hq.Policy()
    Tmax = inp.k.shape[2]
    k, v = to_dev(inp.k, spec.dtype), to_dev(inp.v, spec.dtype)
    lens = ints_to_dev(inp.seq_lens)
    col, sel, cnt, thr = hq.probe_select(to_dev(inp.q_probe, spec.dtype), k, lens, pol)
    cache = hq.HybridCache(spec.B, spec.Hkv, Tmax + cap_extra, Tmax,
                           torch.bfloat16 if spec.dtype == "bf16" else torch.float16, "cuda", pol)
    hq.quantize_kv(cache, k, v, lens, sel, cnt, col, thr)
    torch.cuda.synchronize()
    del k, v
    return cache, tuple(t.cpu().numpy() for t in (col, sel, cnt, thr))


def _oracle_pair(spec, inp, b, g, gsel, check_sel=True):
    """Oracle probe/selection check and cache for one (b, g), using the GPU's
    selection (near-tie flips are legitimate and counted)."""
    col, sel, cnt, thr = gsel
    T = int(inp.seq_lens[b])
    G = spec.Hq // spec.Hkv
    sm = 1 / math.sqrt(spec.D)
    flips = 0
    if check_sel:
        qp = O.to_f64(inp.q_probe[b, g * G:(g + 1) * G], spec.dtype)
        c_or = O.probe_column_scores(qp, O.to_f64(inp.k[b, g:g + 1, :T], spec.dtype), T, sm)[0]
        rel = np.abs(col[b, g, :T].astype(np.float64) - c_or) / c_or
        assert rel.max() < 1e-6, float(rel.max())
        flips = compare_selection(sel[b, g, : cnt[b, g]], int(cnt[b, g]), c_or, T, spec.window, (5, 100))
    idx = sel[b, g, : cnt[b, g]].astype(np.int64)
    assert len(idx) == T * 5 // 100                      # kept = top-5% (+ the 128 window)
    tau = float(thr[b, g, 0:1].view(np.float32)[0])
    c = O.build_cache(O.to_f64(inp.k[b, g, :T], spec.dtype), O.to_f64(inp.v[b, g, :T], spec.dtype), T,
                      O.Selection(idx, len(idx), tau, int(thr[b, g, 1])), spec.window,
                      col[b, g, :T].astype(np.float64))
    return c, flips


def _check_codes(gcache, oc, bg):
    qpos = np.nonzero(oc.mode == O.MODE_INT4)[0]
    nq = len(qpos)
    assert np.array_equal(gcache["q_pos"][bg, :nq], qpos)
    assert np.array_equal(gcache["k_codes"][bg, :nq], oc.k_codes[qpos])
    assert np.array_equal(gcache["v_codes"][bg, :nq], oc.v_codes[qpos])
    for n in ("k_s", "k_z", "v_s", "v_z"):
        assert np.array_equal(gcache[n][bg, :nq].view(np.uint16), getattr(oc, n)[qpos].view(np.uint16))


SAMPLES = {
    "c2_decode_8b_32k": [(0, 0), (3, 5), (7, 2), (11, 7), (15, 3)],
    "c5_decode_70b_ragged_64k": [(0, 0), (2, 4), (5, 7), (7, 1)],
}


@pytest.mark.parametrize("name", ["c2_decode_8b_32k", "c5_decode_70b_ragged_64k"])
def test_decode_path_full_size(name):
    import torch
    import kv_cache_amd as hq
    spec = CONFIGS[name]
    print(f"generating {name}", flush=True)
    inp = make_decode_inputs(spec)
    cache, gsel = _pipeline(spec, inp)
    assert cache.err_flag() == 0
    out = hq.decode_attn(cache, to_dev(inp.q, spec.dtype)).cpu().numpy()
    torch.cuda.synchronize()
    gc = read_cache(cache)
    G = spec.Hq // spec.Hkv
    flips = 0
    for (b, g) in SAMPLES[name]:
        oc, f = _oracle_pair(spec, inp, b, g, gsel)
        flips += f
        _check_codes(gc, oc, b * spec.Hkv + g)
        ref = O.decode_attention(O.to_f64(inp.q[b, g * G:(g + 1) * G], spec.dtype), oc, 1 / math.sqrt(spec.D))
        assert_attn_close(out[b, g * G:(g + 1) * G], ref, f"{name} decode (b={b}, g={g})")
        planted = set(inp.planted[b][g].tolist())
        recall = len(planted & set(gsel[1][b, g, : gsel[2][b, g]].tolist())) / len(planted)
        print(f"  (b={b}, g={g}) planted-line recall {recall:.3f}", flush=True)
    print(f"{name}: near-tie selection flips {flips}", flush=True)


def test_decode_with_appends_128k():
    """8B shape at 128K, batch 4, 64 consecutive appends, each followed by a
    decode with its own query; checked at steps 1, 2, 32 and 64."""
    import torch
    import kv_cache_amd as hq
    spec = CONFIGS["c3_decode_8b_128k_append"]
    print("generating c3", flush=True)
    inp = make_decode_inputs(spec)
    cache, gsel = _pipeline(spec, inp, cap_extra=64)
    kn, vn, qn = make_append_tokens(spec, inp.outlier_channels, 64)
    G = spec.Hq // spec.Hkv
    pairs = [(0, 1), (1, 6), (3, 3)]
    ocs = {}
    for (b, g) in pairs:
        ocs[(b, g)], _ = _oracle_pair(spec, inp, b, g, gsel, check_sel=(b, g) == (0, 1))
    kd, vd, qd = to_dev(kn, "bf16"), to_dev(vn, "bf16"), to_dev(qn, "bf16")
    for s in range(64):
        hq.append_kv(cache, kd[s], vd[s])
        out = hq.decode_attn(cache, qd[s])
        for (b, g) in pairs:
            ocs[(b, g)] = O.append_token(ocs[(b, g)], O.to_f64(kn[s, b, g], "bf16"), O.to_f64(vn[s, b, g], "bf16"))
        if s + 1 in (1, 2, 32, 64):
            o = out.cpu().numpy()
            for (b, g) in pairs:
                ref = O.decode_attention(O.to_f64(qn[s, b, g * G:(g + 1) * G], "bf16"), ocs[(b, g)],
                                         1 / math.sqrt(spec.D))
                assert_attn_close(o[b, g * G:(g + 1) * G], ref, f"c3 step {s + 1} (b={b}, g={g})")
    torch.cuda.synchronize()
    assert cache.err_flag() == 0
    gc = read_cache(cache)
    for (b, g) in pairs:
        oc = ocs[(b, g)]
        _check_codes(gc, oc, b * spec.Hkv + g)
        cnts = gc["counts"][b, g]
        assert cnts[0] == oc.T and cnts[2] == int((oc.mode == O.MODE_KEPT).sum())
