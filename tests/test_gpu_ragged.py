"""GPU checks of the ragged INT4 cache layout (hq_cache_layout_ragged).

The same batch is cached twice, in the uniform layout sized for the longest
sequence and in the ragged layout sized per sequence (the longest one given
the same capacity, so both layouts split the decode alike). Quantize, 40
appends with a decode after each, and a re-probe must give bit-identical
results in both layouts, the cache contents must be equal slot for slot, and
the decode must match the oracle. A sequence given no room beyond its prompt
must overflow on its own: err_flag bit 2, nothing stored, the other
sequences unaffected."""
import numpy as np
import pytest

import oracle as O
from synth import small_decode_inputs
from synth.inputs import make_append_tokens

from gpu_common import (assert_attn_close, fp32_scale, ints_to_dev, oracle_caches, oracle_selection, selection_tensors,
                        to_dev, torch_dtype)
from hq_layout import read_cache

pytestmark = pytest.mark.gpu


def _build(inp, caps, steps, pol):
    import torch
    import kv_cache_amd as hq
    sp = inp.spec
    W = pol.window
    scores, sels = oracle_selection(inp, W, (pol.keep_num, pol.keep_den))
    Tmax = inp.k.shape[2]
    sel, cnt, col, thr = selection_tensors(scores, sels, sp.B, sp.Hkv, Tmax, hq.sel_stride(Tmax, pol))
    cache = hq.HybridCache(sp.B, sp.Hkv, caps, Tmax, torch_dtype(sp.dtype), "cuda", pol)
    hq.quantize_kv(cache, to_dev(inp.k, sp.dtype), to_dev(inp.v, sp.dtype), ints_to_dev(inp.seq_lens), sel, cnt,
                   col, thr)
    kn, vn, qn = make_append_tokens(sp, inp.outlier_channels, steps)
    kd, vd, qd = to_dev(kn, sp.dtype), to_dev(vn, sp.dtype), to_dev(qn, sp.dtype)
    outs = []
    for s in range(steps):
        hq.append_kv(cache, kd[s], vd[s])
        outs.append(hq.decode_attn(cache, qd[s]).cpu().numpy())
    torch.cuda.synchronize()
    return cache, outs, (scores, sels, kn, vn, qn)


def test_ragged_layout_matches_uniform_and_oracle():
    import kv_cache_amd as hq
    inp = small_decode_inputs(B=3, Hq=8, Hkv=2, T=1500, ragged_min=500, seed=81)
    sp = inp.spec
    steps = 40
    pol = hq.Policy()
    Tmax = inp.k.shape[2]
    lens = [int(x) for x in inp.seq_lens]
    caps = [Tmax + steps] + [n + steps for n in lens[1:]]
    print(f"ragged: seq_lens {lens}, capacities {caps}", flush=True)
    uni, outs_u, _ = _build(inp, Tmax + steps, steps, pol)
    rag, outs_r, (scores, sels, kn, vn, qn) = _build(inp, caps, steps, pol)
    assert uni.err_flag() == 0 and rag.err_flag() == 0
    assert rag.c.cap_q == uni.c.cap_q
    print(f"INT4 pool bytes: ragged {rag.sizes.k_codes} vs uniform {uni.sizes.k_codes}", flush=True)
    assert rag.sizes.k_codes < uni.sizes.k_codes
    for s in range(steps):
        assert np.array_equal(outs_r[s].view(np.uint32), outs_u[s].view(np.uint32)), s
    gu, gr = read_cache(uni), read_cache(rag)
    for name in gu:
        assert np.array_equal(np.asarray(gu[name]), np.asarray(gr[name])), name
    # re-probe over both layouts from the last 64 decode queries
    q_recent = np.ascontiguousarray(np.concatenate([inp.q_probe[:, :, steps:], qn.transpose(1, 2, 0, 3)], axis=2))
    qr = to_dev(q_recent, sp.dtype)
    ru = [t.cpu().numpy() for t in hq.reprobe(uni, qr)[:5]]
    rr = [t.cpu().numpy() for t in hq.reprobe(rag, qr)[:5]]
    for a, b in zip(ru, rr):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)
    # the oracle after all appends
    oc = oracle_caches(inp, sels, scores, pol.window)
    for b in range(sp.B):
        for g in range(sp.Hkv):
            oc[b][g] = O.append_tokens(oc[b][g], O.to_f64(kn[:, b, g], sp.dtype), O.to_f64(vn[:, b, g], sp.dtype))
    ref = O.decode_batch(O.to_f64(qn[-1], sp.dtype), oc, fp32_scale(sp.D))
    assert_attn_close(outs_r[-1], ref, "ragged layout, decode after 40 appends")


def test_ragged_overflow_is_contained():
    """Sequence 1 gets exactly its prompt's capacity: once its INT4 store is
    full an append sets err_flag bit 2 and stores nothing for it, while
    sequences 0 and 2 decode exactly as in a uniform cache."""
    import kv_cache_amd as hq
    inp = small_decode_inputs(B=3, Hq=8, Hkv=2, T=900, ragged_min=500, seed=82)
    steps = 160   # more INT4 departures than the k + 63 free slots of a tight store
    pol = hq.Policy()
    Tmax = inp.k.shape[2]
    lens = [int(x) for x in inp.seq_lens]
    caps = [Tmax + steps, lens[1], lens[2] + steps]
    uni, outs_u, _ = _build(inp, Tmax + steps, steps, pol)
    rag, outs_r, _ = _build(inp, caps, steps, pol)
    assert uni.err_flag() == 0
    assert rag.err_flag() & 2
    cu, cr = uni.counts().cpu().numpy(), rag.counts().cpu().numpy()
    qt1 = (rag.q_tile_off[3] - rag.q_tile_off[2])
    print(f"sequence 1: INT4 capacity {qt1 * 64} slots, n_q {cr[1, :, 1].tolist()} (uniform {cu[1, :, 1].tolist()})",
          flush=True)
    assert np.all(cr[1, :, 1] <= qt1 * 64) and np.all(cr[1, :, 1] < cu[1, :, 1])
    for b in (0, 2):
        assert np.array_equal(cr[b], cu[b])
        for s in range(steps):
            assert np.array_equal(outs_r[s][b].view(np.uint32), outs_u[s][b].view(np.uint32)), (b, s)
