"""Guard bands around every device buffer handed to the library.

Each buffer of a pipeline (inputs, the cache's stores, metadata, counts and
error flag, the ragged layout's tile offsets, every workspace and every
output) is cut out of a larger allocation with GUARD bytes of 0xFF on each
side, and its payload is sized exactly as the size queries say. 0xFF bytes
are a NaN in every float format used here and -1 as an integer, so a value
read from a guard into a result poisons it. The pipeline runs twice on the
same seeded inputs, once on guarded allocations and once on plain ones whose
payloads start the same way. Afterwards every guard byte must still be 0xFF
(nothing was written outside its buffer) and every result must be
bit-identical between the two runs (nothing read from outside its buffer
reached a result)."""
import ctypes

import numpy as np
import pytest

from synth import small_decode_inputs
from synth.inputs import PrefillSpec, make_append_tokens, make_prefill_inputs

from gpu_common import fp32_scale, ints_to_dev, to_dev, torch_dtype

pytestmark = pytest.mark.gpu

GUARD = 4096
PAT = 0xFF
D = 128


class Plain:
    """Plain allocations: payloads start zeroed or 0xFF, as in Guarded."""

    def bytes(self, name, n, zero):
        import torch
        t = torch.full((n + 256,), PAT, dtype=torch.uint8, device="cuda")[:n]
        if zero:
            t.zero_()
        return t

    def empty(self, name, shape, dtype):
        import torch
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        return self.bytes(name, n, zero=False).view(dtype).view(shape)

    def copy(self, name, t):
        out = self.empty(name, tuple(t.shape), t.dtype)
        out.copy_(t)
        return out

    def check(self):
        pass


class Guarded(Plain):
    """Payloads of exactly the requested size between two guard bands."""

    def __init__(self):
        self.blocks = []

    def bytes(self, name, n, zero):
        import torch
        base = torch.full((n + 2 * GUARD,), PAT, dtype=torch.uint8, device="cuda")
        body = base[GUARD:GUARD + n]
        if zero:
            body.zero_()
        self.blocks.append((name, base, n))
        return body

    def check(self):
        import torch
        torch.cuda.synchronize()
        bad = [name for name, base, n in self.blocks
               if not (bool((base[:GUARD] == PAT).all()) and bool((base[GUARD + n:] == PAT).all()))]
        assert not bad, f"guard bytes overwritten around: {bad}"
        print(f"{len(self.blocks)} guarded buffers intact", flush=True)


def _abi():
    import kv_cache_amd as hq
    return hq, hq.lib, hq._ptr, hq._stream


def _probe(A, tag, q_probe, k, lens, pol, sm):
    import torch
    hq, lib, P, S = _abi()
    B, Hq, _, _ = q_probe.shape
    _, Hkv, Tmax, _ = k.shape
    pc = pol.c()
    stride = hq.sel_stride(Tmax, pol)
    col = A.empty(f"{tag} col_scores", (B, Hkv, Tmax), torch.float32)
    sel = A.empty(f"{tag} sel_idx", (B, Hkv, stride), torch.int32)
    cnt = A.empty(f"{tag} sel_count", (B, Hkv), torch.int32)
    thr = A.empty(f"{tag} thresh", (B, Hkv, 2), torch.int32)
    ws = A.bytes(f"{tag} ws", lib.hq_probe_ws_bytes(B, Hq, Hkv, Tmax, D, ctypes.byref(pc)), zero=False)
    hq._check(lib.hq_probe_select(P(q_probe), P(k), P(lens), B, Hq, Hkv, Tmax, D, hq._dt(k), ctypes.byref(pc), sm,
                                  P(col), P(sel), P(cnt), P(thr), P(ws), ws.numel(), S()))
    return col, sel, cnt, thr


def decode_pipeline(A, inp, ragged, steps):
    """Probe and selection, quantize, appends with a decode after each, the
    last decode also into a 16-bit output and through the entry point with
    no workspace, the INT4 read helper and the re-probe."""
    import torch
    hq, lib, P, S = _abi()
    sp = inp.spec
    B, Hq, Hkv = sp.B, sp.Hq, sp.Hkv
    Tmax = inp.k.shape[2]
    pol = hq.Policy()
    pc = pol.c()
    sm = fp32_scale(D)
    res = {}
    print(f"guard decode pipeline: B={B} Hq={Hq} Hkv={Hkv} Tmax={Tmax} {sp.dtype} ragged={ragged} "
          f"guarded={isinstance(A, Guarded)}", flush=True)
    q_probe = A.copy("q_probe", to_dev(inp.q_probe, sp.dtype))
    k = A.copy("k", to_dev(inp.k, sp.dtype))
    v = A.copy("v", to_dev(inp.v, sp.dtype))
    lens = A.copy("seq_lens", ints_to_dev(inp.seq_lens))
    col, sel, cnt, thr = _probe(A, "probe", q_probe, k, lens, pol, sm)
    res.update({"probe col": col, "probe sel": sel, "probe cnt": cnt, "probe thr": thr})

    caps = [Tmax + steps] + [int(n) + steps for n in inp.seq_lens[1:]] if ragged else Tmax + steps
    cache = hq.HybridCache(B, Hkv, caps, Tmax, torch_dtype(sp.dtype), "cuda", pol)
    for name in hq._CACHE_PTRS:
        t = A.bytes(f"cache {name}", int(getattr(cache.sizes, name)), zero=True)
        cache.bufs[name] = t
        setattr(cache.c, name, t.data_ptr())
    if ragged:
        t = A.copy("cache q_tile_off", cache.bufs["q_tile_off"])
        cache.bufs["q_tile_off"] = t
        cache.c.q_tile_off = t.data_ptr()
    hq._check(lib.hq_quantize_kv(P(k), P(v), P(lens), Tmax, P(sel), P(cnt), P(col), P(thr), ctypes.byref(pc),
                                 cache.ptr(), S()))

    kn, vn, qn = make_append_tokens(sp, inp.outlier_channels, steps)
    for s in range(steps):
        kd = A.copy(f"k_new {s}", to_dev(kn[s], sp.dtype))
        vd = A.copy(f"v_new {s}", to_dev(vn[s], sp.dtype))
        qd = A.copy(f"q {s}", to_dev(qn[s], sp.dtype))
        hq._check(lib.hq_append_kv(cache.ptr(), P(kd), P(vd), S()))
        ws = A.bytes(f"decode ws {s}", lib.hq_decode_ws_bytes(cache.ptr(), Hq), zero=False)
        out = A.empty(f"decode out {s}", (B, Hq, D), torch.float32)
        hq._check(lib.hq_decode_attn(cache.ptr(), P(qd), Hq, sm, P(out), hq.HQ_F32, P(ws), ws.numel(), S()))
        res[f"decode {s}"] = out
    out16 = A.empty("decode out 16-bit", (B, Hq, D), torch_dtype(sp.dtype))
    ws = A.bytes("decode ws 16-bit", lib.hq_decode_ws_bytes(cache.ptr(), Hq), zero=False)
    hq._check(lib.hq_decode_attn(cache.ptr(), P(qd), Hq, sm, P(out16), hq._dt(out16), P(ws), ws.numel(), S()))
    res["decode 16-bit"] = out16
    outn = A.empty("decode out no workspace", (B, Hq, D), torch.float32)
    hq._check(lib.hq_decode_attn_noalloc(cache.ptr(), P(qd), Hq, sm, P(outn), hq.HQ_F32, S()))
    res["decode no workspace"] = outn
    sink = A.bytes("diag sink", lib.hq_diag_read_int4_sink_bytes(cache.ptr()), zero=False)
    hq._check(lib.hq_diag_read_int4(cache.ptr(), P(sink), sink.numel(), S()))
    res["diag sink"] = sink

    tcap = hq.reprobe_tcap(cache)
    stride = hq.sel_stride(tcap, pol)
    qr = A.copy("q_recent", to_dev(inp.q_probe, sp.dtype))
    rcol = A.empty("reprobe col_scores", (B, Hkv, tcap), torch.float32)
    rsel = A.empty("reprobe sel_idx", (B, Hkv, stride), torch.int32)
    rcnt = A.empty("reprobe sel_count", (B, Hkv), torch.int32)
    rthr = A.empty("reprobe thresh", (B, Hkv, 2), torch.int32)
    rper = A.empty("reprobe n_persist", (B, Hkv), torch.int32)
    ws = A.bytes("reprobe ws", lib.hq_reprobe_ws_bytes(cache.ptr(), Hq, ctypes.byref(pc)), zero=False)
    hq._check(lib.hq_reprobe(cache.ptr(), P(qr), Hq, ctypes.byref(pc), sm, P(rcol), P(rsel), P(rcnt), P(rthr),
                             P(rper), P(ws), ws.numel(), S()))
    res.update({"reprobe col": rcol, "reprobe sel": rsel, "reprobe cnt": rcnt, "reprobe thr": rthr,
                "reprobe persist": rper, "reprobe expanded keys": ws[: B * Hkv * tcap * D * 2]})
    for name in hq._CACHE_PTRS:
        res[f"cache {name}"] = cache.bufs[name]
    torch.cuda.synchronize()
    assert cache.err_flag() == 0
    return res


def prefill_pipeline(A, inp, pol):
    """Probe and selection on the prompt's last rows, then the prefill."""
    import torch
    hq, lib, P, S = _abi()
    sp = inp.spec
    B, Hq, Hkv, T = sp.B, sp.Hq, sp.Hkv, sp.T
    pc = pol.c()
    sm = fp32_scale(D)
    print(f"guard prefill pipeline: B={B} Hq={Hq} Hkv={Hkv} T={T} {sp.dtype} low_fmt={pol.low_fmt} "
          f"tile={pol.tile_num}/{pol.tile_den} guarded={isinstance(A, Guarded)}", flush=True)
    q = A.copy("q", to_dev(inp.q, sp.dtype))
    k = A.copy("k", to_dev(inp.k, sp.dtype))
    v = A.copy("v", to_dev(inp.v, sp.dtype))
    R = min(pol.probe_rows, T)
    q_probe = A.copy("q_probe", q[:, :, T - R:].contiguous())
    lens = A.copy("seq_lens", ints_to_dev(np.full(B, T)))
    col, sel, cnt, thr = _probe(A, "probe", q_probe, k, lens, pol, sm)
    ws = A.bytes("prefill ws", lib.hq_prefill_ws_bytes(B, Hq, Hkv, T, D, ctypes.byref(pc)), zero=False)
    out = A.empty("prefill out", (B, Hq, T, D), torch.float32)
    hq._check(lib.hq_prefill_attn(P(q), P(k), P(v), B, Hq, Hkv, T, D, hq._dt(q), ctypes.byref(pc), P(sel), P(cnt),
                                  sm, P(out), hq.HQ_F32, P(ws), ws.numel(), S()))
    out16 = A.empty("prefill out 16-bit", (B, Hq, T, D), torch_dtype(sp.dtype))
    hq._check(lib.hq_prefill_attn(P(q), P(k), P(v), B, Hq, Hkv, T, D, hq._dt(q), ctypes.byref(pc), P(sel), P(cnt),
                                  sm, P(out16), hq._dt(out16), P(ws), ws.numel(), S()))
    torch.cuda.synchronize()
    return {"probe col": col, "probe sel": sel, "probe cnt": cnt, "prefill out": out, "prefill out 16-bit": out16}


def _raw(t):
    import torch
    return t.contiguous().view(-1).view(torch.uint8)


def _same(a, b):
    import torch
    diff = [name for name in a if not torch.equal(_raw(a[name]), _raw(b[name]))]
    assert not diff, f"guarded and plain runs differ in: {diff}"


@pytest.mark.parametrize("ragged,dtype", [(False, "f16"), (True, "bf16")], ids=["uniform-f16", "ragged-bf16"])
def test_decode_path_stays_inside_its_buffers(ragged, dtype):
    inp = small_decode_inputs(B=3, Hq=8, Hkv=2, T=1500, dtype=dtype, ragged_min=500, seed=97)
    A = Guarded()
    got = decode_pipeline(A, inp, ragged, steps=12)
    A.check()
    _same(got, decode_pipeline(Plain(), inp, ragged, steps=12))


@pytest.mark.parametrize("mode", ["int8", "fp8", "int8-tile"])
def test_prefill_path_stays_inside_its_buffers(mode):
    import kv_cache_amd as hq
    spec = PrefillSpec(name="guard", B=2, Hq=4, Hkv=2, T=700, dtype="bf16", window=128, plant_frac=0.01, seed=98)
    inp = make_prefill_inputs(spec)
    pol = {"int8": hq.Policy(),
           "fp8": hq.Policy(low_fmt=hq.HQ_LOW_FP8),
           "int8-tile": hq.Policy(tile_num=20, tile_den=100)}[mode]
    A = Guarded()
    got = prefill_pipeline(A, inp, pol)
    A.check()
    _same(got, prefill_pipeline(Plain(), inp, pol))
