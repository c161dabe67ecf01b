"""GPU parity of hq_prefill_attn against the oracle's hybrid prefill.

INT8 stage: the Q8/K8 codes and the per-64-block fp32 scales read back from
the documented workspace prefix are compared bit-exactly with
oracle.int8_block_quantize. Attention: the fp32 output is compared with
oracle.prefill_attention_block (all rows, small sizes) or
oracle.prefill_attention_rows (sampled rows, the 16K prefill workload) within
max-abs 2e-3 and relative L2 1e-3.

The selected set S is an input of the operator: small cases take the oracle's
probe selection, edge cases take seeded sets, and the full-size case takes
what hq_probe_select returned on the device (the same S is fed to both)."""
import math

import numpy as np
import pytest

import oracle as O
from synth.inputs import CONFIGS, PrefillSpec, make_prefill_inputs

from gpu_common import assert_attn_close, to_dev

pytestmark = pytest.mark.gpu

D = 128


def _al(x):
    return (x + 255) // 256 * 256


def ws_int8_stage(ws, B, Hq, Hkv, T):
    """Q8, sQ, K8, sK from the workspace prefix documented in include/hq.h."""
    nb = (T + 63) // 64
    Tp = 64 * nb
    h = ws.cpu().numpy()
    o1 = _al(B * Hq * Tp * D)
    o2 = o1 + _al(4 * B * Hq * nb)
    o3 = o2 + _al(B * Hkv * Tp * D)
    q8 = h[: B * Hq * Tp * D].view(np.int8).reshape(B, Hq, Tp, D)
    sq = h[o1: o1 + 4 * B * Hq * nb].view(np.float32).reshape(B, Hq, nb)
    k8 = h[o2: o2 + B * Hkv * Tp * D].view(np.int8).reshape(B, Hkv, Tp, D)
    sk = h[o3: o3 + 4 * B * Hkv * nb].view(np.float32).reshape(B, Hkv, nb)
    return q8, sq, k8, sk


def oracle_sel(inp, window, keep):
    sp = inp.spec
    R = min(sp.probe_rows, sp.T)
    qp = O.to_f64(inp.q[:, :, sp.T - R:], sp.dtype)
    k = O.to_f64(inp.k, sp.dtype)
    _, sels = O.probe_select_batch(qp, k, np.full(sp.B, sp.T), 1 / math.sqrt(D), window, keep[0], keep[1])
    return [[s.idx.astype(np.int64) for s in row] for row in sels]


def seeded_sel(B, Hkv, T, frac, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(B):
        row = []
        for _ in range(Hkv):
            n = int(frac * T)
            row.append(np.sort(rng.choice(T, size=n, replace=False)).astype(np.int64))
        out.append(row)
    return out


def sel_device(sels, B, Hkv, stride):
    import torch
    idx = np.full((B, Hkv, stride), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            s = sels[b][g]
            assert len(s) <= stride
            idx[b, g, : len(s)] = s
            cnt[b, g] = len(s)
    return torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()


def run_prefill(inp, sels, pol, out_dtype=None):
    import torch
    import kv_cache_amd as hq
    sp = inp.spec
    stride = hq.sel_stride(sp.T, pol)
    idx, cnt = sel_device(sels, sp.B, sp.Hkv, stride)
    q, k, v = (to_dev(x, sp.dtype) for x in (inp.q, inp.k, inp.v))
    n = hq.lib.hq_prefill_ws_bytes(sp.B, sp.Hq, sp.Hkv, sp.T, D, __import__("ctypes").byref(pol.c()))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = hq.prefill_attn(q, k, v, idx, cnt, pol, out_dtype=out_dtype, ws=ws)
    torch.cuda.synchronize()
    return out, ws


def check_int8_stage(inp, ws, heads=None):
    sp = inp.spec
    q8, sq, k8, sk = ws_int8_stage(ws, sp.B, sp.Hq, sp.Hkv, sp.T)
    T = sp.T
    qf = O.to_f64(inp.q, sp.dtype)
    kf = O.to_f64(inp.k, sp.dtype)
    for b in range(sp.B):
        for g in range(sp.Hkv):
            c, s = O.int8_block_quantize(kf[b, g])
            assert np.array_equal(k8[b, g, :T], c), (b, g)
            assert np.all(k8[b, g, T:] == 0)
            assert np.array_equal(sk[b, g].view(np.uint32), s.view(np.uint32)), (b, g)
        for h in (heads if heads is not None else range(sp.Hq)):
            c, s = O.int8_block_quantize(qf[b, h])
            assert np.array_equal(q8[b, h, :T], c), (b, h)
            assert np.all(q8[b, h, T:] == 0)
            assert np.array_equal(sq[b, h].view(np.uint32), s.view(np.uint32)), (b, h)


def oracle_prefill_all(inp, sels, window):
    sp = inp.spec
    G = sp.Hq // sp.Hkv
    sm = 1 / math.sqrt(D)
    qf, kf, vf = (O.to_f64(x, sp.dtype) for x in (inp.q, inp.k, inp.v))
    ref = np.empty((sp.B, sp.Hq, sp.T, D))
    for b in range(sp.B):
        for g in range(sp.Hkv):
            k8, sk = O.int8_block_quantize(kf[b, g])
            for h in range(g * G, (g + 1) * G):
                q8, sq = O.int8_block_quantize(qf[b, h])
                ref[b, h] = O.prefill_attention_block(qf[b, h], kf[b, g], vf[b, g], sels[b][g], window, sm,
                                                      q8, sq, k8, sk, 0, sp.T)
    return ref


# name, B, Hq, Hkv, T, dtype, window, keep, selection source
CASES = [
    ("bf16_ragged", 1, 4, 2, 333, "bf16", 128, (5, 100), "oracle"),
    ("f16_g2", 2, 4, 2, 520, "f16", 128, (5, 100), "oracle"),
    ("g8", 1, 8, 1, 300, "bf16", 128, (5, 100), "oracle"),
    ("no_window", 1, 2, 1, 300, "bf16", 0, (5, 100), "oracle"),
    ("window192", 1, 2, 1, 450, "bf16", 192, (5, 100), "oracle"),
    ("many_selected", 1, 2, 1, 700, "bf16", 128, (50, 100), "seeded"),
    ("none_selected", 1, 2, 1, 400, "bf16", 128, (0, 100), "oracle"),
    ("T1", 1, 2, 1, 1, "bf16", 128, (5, 100), "seeded"),
    ("T64", 1, 2, 1, 64, "f16", 128, (5, 100), "seeded"),
    ("T129", 1, 2, 2, 129, "bf16", 64, (5, 100), "seeded"),
    ("T1000_w64", 1, 4, 1, 1000, "bf16", 64, (10, 100), "oracle"),
    # every candidate selected: all scores 16-bit, i.e. exact causal attention
    ("all_selected", 1, 4, 2, 900, "bf16", 128, (100, 100), "oracle"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_prefill_parity(case):
    import kv_cache_amd as hq
    name, B, Hq, Hkv, T, dtype, W, keep, src = case
    spec = PrefillSpec(name=name, B=B, Hq=Hq, Hkv=Hkv, T=T, dtype=dtype, window=W, plant_frac=0.01, seed=77 + T)
    inp = make_prefill_inputs(spec)
    pol = hq.Policy(keep[0], keep[1], W, 64)
    if src == "oracle":
        sels = oracle_sel(inp, W, keep)
    else:
        frac = keep[0] / keep[1]
        sels = seeded_sel(B, Hkv, T, frac, seed=T)
    print(f"prefill case {name}: B={B} Hq={Hq} Hkv={Hkv} T={T} {dtype} W={W} |S|={[len(s) for s in sels[0]]}",
          flush=True)
    out, ws = run_prefill(inp, sels, pol)
    check_int8_stage(inp, ws)
    ref = oracle_prefill_all(inp, sels, W)
    assert_attn_close(out.cpu().numpy(), ref, name)
    if keep == (100, 100):
        # every candidate selected: exact causal softmax attention
        o = out.cpu().numpy()
        G, sm = Hq // Hkv, 1 / math.sqrt(spec.D)
        qf, kf, vf = (O.to_f64(x, dtype) for x in (inp.q, inp.k, inp.v))
        ex = np.zeros_like(o, dtype=np.float64)
        for h in range(Hq):
            for i in range(T):
                ex[0, h, i] = O.softmax_attention(qf[0, h, i:i + 1], kf[0, h // G, :i + 1], vf[0, h // G, :i + 1], sm)[0]
        assert_attn_close(o, ex, f"{name} exact causal attention")


def test_prefill_zero_block_and_out_dtypes():
    """An all-zero K block and Q block (scale 0, codes 0), and 16-bit outputs
    equal to the fp32 output rounded once."""
    import torch
    import kv_cache_amd as hq
    spec = PrefillSpec(name="zero", B=1, Hq=2, Hkv=1, T=260, seed=5)
    inp = make_prefill_inputs(spec)
    inp.k[0, 0, 64:128] = 0
    inp.q[0, 1, 128:192] = 0
    pol = hq.Policy()
    sels = oracle_sel(inp, 128, (5, 100))
    out, ws = run_prefill(inp, sels, pol)
    check_int8_stage(inp, ws)
    _, sq, _, sk = ws_int8_stage(ws, 1, 2, 1, spec.T)
    assert sk[0, 0, 1] == 0 and sq[0, 1, 2] == 0
    ref = oracle_prefill_all(inp, sels, 128)
    assert_attn_close(out.cpu().numpy(), ref, "zero blocks")
    for dt in (torch.bfloat16, torch.float16):
        o16, _ = run_prefill(inp, sels, pol, out_dtype=dt)
        assert torch.equal(o16.cpu(), out.cpu().to(dt)), dt


def test_prefill_deterministic():
    spec = PrefillSpec(name="det", B=1, Hq=4, Hkv=1, T=700, seed=11)
    inp = make_prefill_inputs(spec)
    import kv_cache_amd as hq
    pol = hq.Policy()
    sels = oracle_sel(inp, 128, (5, 100))
    a, _ = run_prefill(inp, sels, pol)
    b, _ = run_prefill(inp, sels, pol)
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


@pytest.mark.slow
def test_prefill_16k_sampled():
    """The 16K causal prefill workload (B=1, 32 query / 8 KV heads), launched
    as the benchmark launches it: the INT8 stage bit-exact for the sampled
    heads and every K head, sampled output rows against the oracle."""
    import torch
    import kv_cache_amd as hq
    spec = CONFIGS["c4_prefill_8b_16k"]
    inp = make_prefill_inputs(spec)
    T, G = spec.T, spec.Hq // spec.Hkv
    pol = hq.Policy()
    print("prefill 16k: probe", flush=True)
    q, k = to_dev(inp.q, spec.dtype), to_dev(inp.k, spec.dtype)
    lens = torch.full((1,), T, dtype=torch.int32, device="cuda")
    col, sel, cnt, thr = hq.probe_select(q[:, :, T - 64:].contiguous(), k, lens, pol)
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    sels = [[sel_h[0, g, : cnt_h[0, g]].astype(np.int64) for g in range(spec.Hkv)]]
    del q, k, col, sel, cnt, thr
    print("prefill 16k: attention", flush=True)
    out, ws = run_prefill(inp, sels, pol)
    heads = [0, 5, 13, 31]
    check_int8_stage(inp, ws, heads=heads)
    out = out.cpu().numpy()
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, 129, 255, 4095, 8191, T - 129, T - 128, T - 1],
                                     rng.integers(0, T, size=12)]))
    qf, kf, vf = (O.to_f64(x, spec.dtype) for x in (inp.q, inp.k, inp.v))
    sm = 1 / math.sqrt(D)
    for h in heads:
        g = h // G
        k8, sk = O.int8_block_quantize(kf[0, g])
        q8, sq = O.int8_block_quantize(qf[0, h])
        ref = O.prefill_attention_rows(qf[0, h], kf[0, g], vf[0, g], sels[0][g], 128, sm, q8, sq, k8, sk, rows)
        assert_attn_close(out[0, h, rows], ref, f"16k head {h}")
