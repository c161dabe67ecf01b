"""hq_decode_attn_noalloc through the C ABI: the same output as
hq_decode_attn with a caller workspace (bit for bit: same kernels, same
split count) and within the attention bars of the oracle, on two calls in a
row, the second on a smaller cache (the static scratch keeps the first
call's partials; nothing of them may leak into the second)."""

import numpy as np
import pytest

import oracle as O
from synth import small_decode_inputs

from gpu_common import assert_attn_close, fp32_scale, ints_to_dev, oracle_caches, oracle_selection, selection_tensors, to_dev

pytestmark = pytest.mark.gpu


def _built(kw):
    import torch
    import kv_cache_amd as hq
    inp = small_decode_inputs(**kw)
    sp = inp.spec
    pol = hq.Policy(5, 100, 128, sp.probe_rows)
    scores, sels = oracle_selection(inp, 128, (5, 100))
    Tmax = inp.k.shape[2]
    sel, cnt, col, thr = selection_tensors(scores, sels, sp.B, sp.Hkv, Tmax, hq.sel_stride(Tmax, pol))
    dt = torch.bfloat16 if sp.dtype == "bf16" else torch.float16
    cache = hq.HybridCache(sp.B, sp.Hkv, Tmax, Tmax, dt, "cuda", pol)
    hq.quantize_kv(cache, to_dev(inp.k, sp.dtype), to_dev(inp.v, sp.dtype), ints_to_dev(inp.seq_lens), sel, cnt,
                   col, thr)
    return inp, cache, oracle_caches(inp, sels, scores, 128)


def test_noalloc_matches_workspace_entry_point():
    import torch
    import kv_cache_amd as hq
    big = dict(B=3, Hq=16, Hkv=2, T=5000, ragged_min=3000, n_outlier=8, outlier_scale=30.0, seed=61)
    small = dict(B=1, Hq=4, Hkv=1, T=900, seed=62)
    for n, kw in enumerate((big, small)):
        inp, cache, ocaches = _built(kw)
        sp = inp.spec
        q = to_dev(inp.q, sp.dtype)
        need = hq.lib.hq_decode_ws_bytes(cache.ptr(), sp.Hq)
        assert 0 < need <= (16 << 20)
        ref_ws = hq.decode_attn(cache, q)
        out = hq.decode_attn_noalloc(cache, q)
        torch.cuda.synchronize()
        print(f"call {n + 1}: B={sp.B} Hq={sp.Hq} Hkv={sp.Hkv} T={sp.T}, partials {need} bytes", flush=True)
        assert torch.equal(out, ref_ws), "noalloc output differs from the workspace entry point"
        ref = O.decode_batch(O.to_f64(inp.q, sp.dtype), ocaches, fp32_scale(sp.D))
        assert_attn_close(out.cpu().numpy(), ref, f"noalloc call {n + 1}")
        # 16-bit output from the same entry point equals the fp32 one rounded once
        o16 = hq.decode_attn_noalloc(cache, q, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o16, out.to(torch.bfloat16))
