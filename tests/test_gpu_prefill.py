"""GPU parity of hq_prefill_attn against the oracle's hybrid prefill.

Low-precision stage (INT8, or FP8 E4M3 with policy.low_fmt): the Q8/K8 code
bytes and the per-64-block fp32 scales read back from the documented
workspace prefix are compared bit-exactly with oracle.int8_block_quantize or
oracle.fp8_block_quantize. Attention: the fp32 output is compared with
oracle.prefill_attention_block (all rows, small sizes) or
oracle.prefill_attention_rows (sampled rows, the 16K prefill workload) within
max-abs 2e-3 and relative L2 1e-3.

The selected set S is an input of the operator: small cases take the oracle's
probe selection, edge cases take seeded sets, and the full-size case takes
what hq_probe_select returned on the device (the same S is fed to both)."""

import numpy as np
import pytest

import oracle as O
from synth.inputs import CONFIGS, PrefillSpec, make_prefill_inputs

from gpu_common import assert_attn_close, fp32_scale, to_dev

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
    _, sels = O.probe_select_batch(qp, k, np.full(sp.B, sp.T), fp32_scale(D), window, keep[0], keep[1])
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


def low_quant(x, fp8):
    """Oracle codes (as stored bytes), block scales and the code values the
    attention uses (INT8 integers, or decoded E4M3)."""
    if fp8:
        c, s = O.fp8_block_quantize(x)
        return c.view(np.int8), s, O.fp8_e4m3_decode(c)
    c, s = O.int8_block_quantize(x)
    return c, s, c


def check_int8_stage(inp, ws, heads=None, fp8=False):
    sp = inp.spec
    q8, sq, k8, sk = ws_int8_stage(ws, sp.B, sp.Hq, sp.Hkv, sp.T)
    T = sp.T
    qf = O.to_f64(inp.q, sp.dtype)
    kf = O.to_f64(inp.k, sp.dtype)
    for b in range(sp.B):
        for g in range(sp.Hkv):
            c, s, _ = low_quant(kf[b, g], fp8)
            assert np.array_equal(k8[b, g, :T], c), (b, g)
            assert np.all(k8[b, g, T:] == 0)
            assert np.array_equal(sk[b, g].view(np.uint32), s.view(np.uint32)), (b, g)
        for h in (heads if heads is not None else range(sp.Hq)):
            c, s, _ = low_quant(qf[b, h], fp8)
            assert np.array_equal(q8[b, h, :T], c), (b, h)
            assert np.all(q8[b, h, T:] == 0)
            assert np.array_equal(sq[b, h].view(np.uint32), s.view(np.uint32)), (b, h)


# The E4M3 matrix instruction (v_mfma_f32_32x32x64_f8f6f4) sums its 64 exact
# products in a block-aligned format: its error, measured against exact sums
# on random E4M3 operands spanning the whole format, reaches 2^-12.5 of the
# sum of |products| (the 16-bit instructions stay within 3 fp32 ulps of it).
# The FP8 path's bar adds what score errors |delta_j| <= d_j can do to a row,
# d_j = 2^-11 (a factor 2 of margin) sum_c |Q8_c K8_jc| sQ sK sm_scale on the
# low-precision keys and 0 on the exact ones. With w the exact softmax
# weights, the perturbed weights are w'_j = w_j e^delta_j / Z' where
# e^(-sum w d) <= Z' <= sum w e^d (Jensen), so |w'_j - w_j| <= w_j (e^(d_j + L) - 1),
# L = ln sum_k w_k e^(d_k), and since sum (w' - w) = 0,
#   |o'_c - o_c| <= sum_j w_j (e^(d_j + L) - 1) (|v_jc| + |o_c|).
FP8_SUM_EPS = 2.0 ** -11


def fp8_bars(qf, kf, qd, sq, kd, sk, vf, ref, rows, sel, W, sm):
    """Per-element max-abs bars [len(rows)][D] of the FP8 path: the 2e-3 of
    the INT8 path plus the bound above (qf, kf: exact 16-bit values of the
    query head and its KV head; qd, kd: decoded E4M3 codes; ref: the
    oracle's output rows)."""
    T = kd.shape[0]
    cols = np.arange(T)
    in_sel = np.zeros(T, dtype=bool)
    in_sel[sel] = True
    causal = cols[None, :] <= rows[:, None]
    exact = in_sel[None, :] | (rows[:, None] - cols[None, :] < W)
    scl = sq.astype(np.float64)[rows // 64][:, None] * sk.astype(np.float64)[cols // 64][None, :]
    logits = np.where(exact, qf[rows] @ kf.T, (qd[rows] @ kd.T) * scl) * sm
    logits[~causal] = -np.inf
    w = np.exp(logits - logits.max(1, keepdims=True))
    w /= w.sum(1, keepdims=True)
    d = FP8_SUM_EPS * (np.abs(qd[rows]) @ np.abs(kd).T) * scl * sm
    d[exact | ~causal] = 0.0
    L = np.log((w * np.exp(d)).sum(1, keepdims=True))
    a = w * np.expm1(d + L)
    return 2e-3 + a @ np.abs(vf) + np.abs(ref) * a.sum(1, keepdims=True)


def assert_fp8_rows(out, ref, bars, what):
    err = np.abs(out - ref)
    worst = float((err / bars).max())
    rl2 = float(np.linalg.norm(out - ref) / np.linalg.norm(ref))
    print(f"{what}: FP8 max-abs {err.max():.3e}, worst error / its bar {worst:.3f} (bars "
          f"{bars.min():.2e}..{bars.max():.2e}), rel-L2 {rl2:.3e}", flush=True)
    assert worst <= 1.0, (what, worst)
    assert rl2 <= 1e-3, (what, rl2)


def oracle_prefill_all(inp, sels, window, fp8=False):
    sp = inp.spec
    G = sp.Hq // sp.Hkv
    sm = fp32_scale(D)
    qf, kf, vf = (O.to_f64(x, sp.dtype) for x in (inp.q, inp.k, inp.v))
    ref = np.empty((sp.B, sp.Hq, sp.T, D))
    for b in range(sp.B):
        for g in range(sp.Hkv):
            _, sk, k8 = low_quant(kf[b, g], fp8)
            for h in range(g * G, (g + 1) * G):
                _, sq, q8 = low_quant(qf[b, h], fp8)
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


FP8_CASES = ["bf16_ragged", "f16_g2", "g8", "no_window", "many_selected", "T1", "T129", "T1000_w64",
             "all_selected"]


@pytest.mark.parametrize("case,fp8", [(c, False) for c in CASES] + [(c, True) for c in CASES if c[0] in FP8_CASES],
                         ids=[c[0] for c in CASES] + [c[0] + "-fp8" for c in CASES if c[0] in FP8_CASES])
def test_prefill_parity(case, fp8):
    import kv_cache_amd as hq
    name, B, Hq, Hkv, T, dtype, W, keep, src = case
    spec = PrefillSpec(name=name, B=B, Hq=Hq, Hkv=Hkv, T=T, dtype=dtype, window=W, plant_frac=0.01, seed=77 + T)
    inp = make_prefill_inputs(spec)
    pol = hq.Policy(keep[0], keep[1], W, 64, hq.HQ_LOW_FP8 if fp8 else hq.HQ_LOW_INT8)
    if src == "oracle":
        sels = oracle_sel(inp, W, keep)
    else:
        frac = keep[0] / keep[1]
        sels = seeded_sel(B, Hkv, T, frac, seed=T)
    print(f"prefill case {name}: B={B} Hq={Hq} Hkv={Hkv} T={T} {dtype} W={W} |S|={[len(s) for s in sels[0]]} "
          f"low={'fp8' if fp8 else 'int8'}", flush=True)
    out, ws = run_prefill(inp, sels, pol)
    check_int8_stage(inp, ws, fp8=fp8)
    ref = oracle_prefill_all(inp, sels, W, fp8)
    if fp8:
        o = out.cpu().numpy()
        G = Hq // Hkv
        qf, kf, vf = (O.to_f64(x, dtype) for x in (inp.q, inp.k, inp.v))
        for b in range(B):
            for h in range(Hq):
                _, sq, qd = low_quant(qf[b, h], True)
                _, sk, kd = low_quant(kf[b, h // G], True)
                rows = np.arange(T)
                bars = fp8_bars(qf[b, h], kf[b, h // G], qd, sq, kd, sk, vf[b, h // G], ref[b, h], rows,
                                sels[b][h // G], W, fp32_scale(D))
                assert_fp8_rows(o[b, h], ref[b, h], bars, f"{name} b={b} h={h}")
    else:
        assert_attn_close(out.cpu().numpy(), ref, name)
    if keep == (100, 100):
        # every candidate selected: exact causal softmax attention
        o = out.cpu().numpy()
        G, sm = Hq // Hkv, fp32_scale(spec.D)
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


@pytest.mark.parametrize("fp8,tile", [(False, 0), (True, 0), (False, 5)], ids=["int8", "fp8", "int8_tile5"])
def test_prefill_16k_full_size(fp8, tile):
    """The 16K causal prefill workload (B=1, 32 query / 8 KV heads), launched
    as the benchmark launches it (INT8, and the FP8 low path): the
    low-precision stage bit-exact for every Q and K
    head, and 1,024 rows of every head against the oracle: the last 64 rows,
    runs of 64 rows across the first window / block boundaries and the
    middle block boundary, and 13 runs at seeded random offsets (not aligned
    to the 64-row blocks)."""
    import time
    import torch
    import kv_cache_amd as hq
    spec = CONFIGS["prefill_8b_16k"]
    inp = make_prefill_inputs(spec)
    T, G = spec.T, spec.Hq // spec.Hkv
    pol = hq.Policy(low_fmt=hq.HQ_LOW_FP8 if fp8 else hq.HQ_LOW_INT8, tile_num=tile)
    print(f"prefill 16k ({'fp8' if fp8 else 'int8'}, tile routing {tile}%): probe", flush=True)
    q, k = to_dev(inp.q, spec.dtype), to_dev(inp.k, spec.dtype)
    lens = torch.full((1,), T, dtype=torch.int32, device="cuda")
    col, sel, cnt, thr = hq.probe_select(q[:, :, T - 64:].contiguous(), k, lens, pol)
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    sels = [[sel_h[0, g, : cnt_h[0, g]].astype(np.int64) for g in range(spec.Hkv)]]
    del q, k, col, sel, cnt, thr
    print("prefill 16k: attention", flush=True)
    out, ws = run_prefill(inp, sels, pol)
    check_int8_stage(inp, ws, fp8=fp8)
    print("prefill 16k: low-precision stage bit-exact on all heads", flush=True)
    bits = ws_route_bits(ws, 1, spec.Hq, T) if tile else None
    out = out.cpu().numpy()
    rng = np.random.default_rng(4)
    starts = [T - 64, 96, 8160] + sorted(int(x) for x in rng.integers(0, T - 64, size=13))
    qf, kf, vf = (O.to_f64(x, spec.dtype) for x in (inp.q, inp.k, inp.v))
    sm = fp32_scale(D)
    t0 = time.time()
    k8s = [low_quant(kf[0, g], fp8) for g in range(spec.Hkv)]
    refs = np.zeros((spec.Hq, len(starts) * 64, D))
    rows = np.concatenate([np.arange(r0, r0 + 64) for r0 in starts])
    for h in range(spec.Hq):
        g = h // G
        _, sk, k8 = k8s[g]
        _, sq, q8 = low_quant(qf[0, h], fp8)
        route = None
        if tile:
            route = O.tile_route(q8, k8, sk, T, 128, tile, 100)
            assert np.array_equal(bits[0, h], route), h
        for n, r0 in enumerate(starts):
            refs[h, 64 * n:64 * (n + 1)] = O.prefill_attention_block(qf[0, h], kf[0, g], vf[0, g], sels[0][g], 128,
                                                                     sm, q8, sq, k8, sk, r0, r0 + 64, route)
        if fp8:
            bars = fp8_bars(qf[0, h], kf[0, g], q8, sq, k8, sk, vf[0, g], refs[h], rows, sels[0][g], 128, sm)
            assert_fp8_rows(out[0][h, rows], refs[h], bars, f"16k prefill head {h}")
        if h % 8 == 7:
            print(f"  heads 0..{h} computed ({time.time() - t0:.0f} s)", flush=True)
    if not fp8:
        assert_attn_close(out[0][:, rows], refs, f"16k prefill, {len(rows)} rows x {spec.Hq} heads")


def _q_tie_blocks(inp):
    """Q blocks whose INT8 quotients x / s land exactly on half-integers or
    one bf16 step beside them, with block scales on both sides of the bounds
    [2^-100, 2^100) at which the Q quantizer switches from the reciprocal and
    FMA residual quotient to the IEEE divide. A block's maximum is 127 * u
    (s = u exactly) and its other values (k + 1/2) * u, k in 0..126."""
    from synth import bf16_bits_from_f32
    rng = np.random.default_rng(2024)
    q = inp.q
    B, Hq, T, _ = q.shape
    us = [2.0 ** -100, 2.0 ** -101, 2.0 ** 99, 2.0 ** 100, 1.1 * 2.0 ** -100, 1.1 * 2.0 ** 99, 2.0 ** -3, 1.0]
    for h in range(Hq):
        for blk in range(T // 64):
            u = us[(blk + h) % len(us)]
            k = rng.integers(0, 127, size=(64, D)).astype(np.float64)
            x = (k + 0.5) * u * np.where(rng.random((64, D)) < 0.5, -1.0, 1.0)
            x[rng.integers(0, 64), rng.integers(0, D)] = 127.0 * u
            bits = bf16_bits_from_f32(x.astype(np.float32))
            step = rng.integers(-1, 2, size=bits.shape) * (rng.random(bits.shape) < 0.25)
            bits = np.where(np.abs(x) == 127.0 * u, bits, (bits.astype(np.int32) + step).astype(np.uint16))
            q[0, h, 64 * blk:64 * (blk + 1)] = bits


def test_prefill_int8_q_half_integer_quotients():
    """The INT8 Q stage where x / s sits on or next to k + 1/2, with scales
    just inside and just outside [2^-100, 2^100): Q8 and sQ bit-exact with
    the oracle (the codes round half to even on the correctly rounded fp32
    quotient). The softmax scale 2^-120 keeps the attention finite for the
    2^100-scale rows; only the INT8 stage is compared."""
    import kv_cache_amd as hq
    spec = PrefillSpec(name="qties", B=1, Hq=4, Hkv=1, T=512, seed=321)
    inp = make_prefill_inputs(spec)
    _q_tie_blocks(inp)
    qf = O.to_f64(inp.q, "bf16")
    q8, sq = O.int8_block_quantize(qf[0, 0])
    with np.errstate(divide="ignore", invalid="ignore"):
        quo = qf[0, 0].astype(np.float32) / np.repeat(sq, 64)[:, None]
    assert np.count_nonzero(np.abs(quo - np.trunc(quo)) == 0.5) > 10000
    pol = hq.Policy()
    sels = oracle_sel(inp, 128, (5, 100))
    import torch
    stride = hq.sel_stride(spec.T, pol)
    idx, cnt = sel_device(sels, 1, 1, stride)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    n = hq.lib.hq_prefill_ws_bytes(1, 4, 1, spec.T, D, __import__("ctypes").byref(pol.c()))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = hq.prefill_attn(q, k, v, idx, cnt, pol, sm_scale=2.0 ** -120, ws=ws)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    check_int8_stage(inp, ws)


def test_prefill_fp8_q_ties_subnormals_and_signed_zero():
    """The FP8 Q stage on quotients x / s that sit exactly on the midpoints
    between E4M3 values (ties to the even mantissa), one bf16 step beside
    them, in the E4M3 subnormal range, and on signed zeros: Q8 bytes and sQ
    bit-exact with the oracle's encoder (itself pinned against the format and
    torch's cast). Block maximum 448 u with u a power of two, so s = u."""
    import torch
    import kv_cache_amd as hq
    from synth import bf16_bits_from_f32
    spec = PrefillSpec(name="fp8ties", B=1, Hq=2, Hkv=1, T=384, seed=322)
    inp = make_prefill_inputs(spec)
    table = O.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (table[:-1] + table[1:]) / 2                    # exact, and exact in bf16 (<= 5 significant bits)
    rng = np.random.default_rng(77)
    for h in range(2):
        for blk in range(spec.T // 64):
            u = 2.0 ** int(rng.integers(-12, 4))
            x = rng.choice(mids, size=(64, D)) * np.where(rng.random((64, D)) < 0.5, -1.0, 1.0)
            x[:8] = rng.choice(table[:8], size=(8, D)) / 3.0     # subnormal quotients (rounded in bf16 first)
            x[8, :] = 0.0
            x[9, :] = -0.0
            x[rng.integers(10, 64), rng.integers(0, D)] = 448.0
            bits = bf16_bits_from_f32((x * u).astype(np.float32))
            step = rng.integers(-1, 2, size=bits.shape) * (rng.random(bits.shape) < 0.2)
            keep = (np.abs(x) == 448.0) | (np.abs(x) == 0.0)
            bits = np.where(keep, bits, (bits.astype(np.int32) + step).astype(np.uint16))
            inp.q[0, h, 64 * blk:64 * (blk + 1)] = bits
    qf = O.to_f64(inp.q, "bf16")
    c, s = O.fp8_block_quantize(qf[0, 0])
    quo = qf[0, 0].astype(np.float32) / np.repeat(s, 64)[:, None]
    on_mid = np.isin(np.abs(quo.astype(np.float64)), mids)
    assert np.count_nonzero(on_mid) > 3000 and np.any((c & 0x78) == 0) and np.any(c == 0x80)
    pol = hq.Policy(low_fmt=hq.HQ_LOW_FP8)
    sels = oracle_sel(inp, 128, (5, 100))
    stride = hq.sel_stride(spec.T, pol)
    idx, cnt = sel_device(sels, 1, 1, stride)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    n = hq.lib.hq_prefill_ws_bytes(1, 2, 1, spec.T, D, __import__("ctypes").byref(pol.c()))
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = hq.prefill_attn(q, k, v, idx, cnt, pol, sm_scale=2.0 ** -8, ws=ws)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    check_int8_stage(inp, ws, fp8=True)


def ws_route_bits(ws, B, Hq, T):
    """The routed tiles' masks from the end of the workspace (include/hq.h)."""
    nb, nqb = (T + 63) // 64, (T + 127) // 128
    nw = (nb + 63) // 64
    n = B * Hq * nqb * nw * 8
    h = ws.cpu().numpy()
    words = h[len(h) - _al(n): len(h) - _al(n) + n].view(np.uint64).reshape(B, Hq, nqb, nw)
    bits = np.zeros((B, Hq, nqb, nb), dtype=bool)
    for kb in range(nb):
        bits[..., kb] = (words[..., kb // 64] >> np.uint64(kb % 64)) & np.uint64(1)
    return bits


TILE_CASES = [
    # name, B, Hq, Hkv, T, dtype, window, keep, tile fraction
    ("token5_tile10", 1, 4, 2, 1000, "bf16", 128, (5, 100), (10, 100)),
    ("tile30_only_f16", 2, 4, 2, 700, "f16", 64, (0, 100), (30, 100)),
    ("token5_tile100", 1, 2, 1, 2000, "bf16", 128, (5, 100), (100, 100)),
    ("g8_tile20", 1, 8, 1, 900, "bf16", 128, (5, 100), (20, 100)),
    ("T129_tile50", 1, 2, 1, 129, "bf16", 64, (5, 100), (50, 100)),
]


@pytest.mark.parametrize("case", TILE_CASES, ids=[c[0] for c in TILE_CASES])
def test_prefill_tile_routing_parity(case):
    """Tile routing composed with the token routing: the routed key blocks
    of every (head, 128-row query block) bit-exact with oracle.tile_route on
    the oracle's INT8 codes, and the attention against the oracle's prefill
    with that routing."""
    import torch
    import kv_cache_amd as hq
    name, B, Hq, Hkv, T, dtype, W, keep, tile = case
    spec = PrefillSpec(name=name, B=B, Hq=Hq, Hkv=Hkv, T=T, dtype=dtype, window=W, plant_frac=0.01, seed=91 + T)
    inp = make_prefill_inputs(spec)
    pol = hq.Policy(keep[0], keep[1], W, 64, hq.HQ_LOW_INT8, tile[0], tile[1])
    sels = oracle_sel(inp, W, keep)
    out, ws = run_prefill(inp, sels, pol)
    check_int8_stage(inp, ws)
    bits = ws_route_bits(ws, B, Hq, T)
    G, sm = Hq // Hkv, fp32_scale(D)
    qf, kf, vf = (O.to_f64(x, dtype) for x in (inp.q, inp.k, inp.v))
    ref = np.empty((B, Hq, T, D))
    routed = 0
    for b in range(B):
        for g in range(Hkv):
            k8, sk = O.int8_block_quantize(kf[b, g])
            for h in range(g * G, (g + 1) * G):
                q8, sq = O.int8_block_quantize(qf[b, h])
                r = O.tile_route(q8, k8, sk, T, W, tile[0], tile[1])
                assert np.array_equal(bits[b, h], r), (b, h)
                routed += int(r.sum())
                ref[b, h] = O.prefill_attention_block(qf[b, h], kf[b, g], vf[b, g], sels[b][g], W, sm, q8, sq, k8, sk,
                                                      0, T, r)
    print(f"tile routing {name}: {routed} routed tiles", flush=True)
    assert_attn_close(out.cpu().numpy(), ref, name)
