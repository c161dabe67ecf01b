#!/usr/bin/env python3
"""Benchmark of the HyQuant-style hybrid-precision attention hot path on one
MI355X.

One step = one pass of every row of the hot path over one batch of seeded
synthetic input, in the order a server runs them:
  decode workload (8B GQA shape: B=16, 32 Q / 8 KV heads, D=128, T=32768):
    the prompt once (probe + top-k select -> quantize/pack), then 16 decode
    tokens on that cache, each one append + one decode (split-K + cross-split
    reduce) with its own query;
  prefill workload (32 Q / 8 KV heads, causal, T=16384):
    probe + select on the last 64 rows -> INT8 block quantization + hybrid
    attention.
Inputs are resident in HBM before timing starts. Every kernel call is
bracketed by HIP events on the stream it is launched on (torch's current
stream). `value` is the steady-state decode attention time (hq_decode_attn,
the 2nd..16th decode of each step) in microseconds; the first decode after
the cache build is reported as decode_us_full_step; the once-per-prompt rows
(probe, quantize, prefill) are reported beside it, and so is a re-probe of
the step's cache from its last 64 query rows ("reprobe": time and the share
of the new selection already kept). After the timed steps the
other decode workloads (1-head 4K warm and cold, 128K with 64 appends, the
ragged 70B-like shape) and the 1K..32K context sweep are timed the same way
and reported under "workloads" and "sweep"; each of them also reports
decode_us_graph, the device time of one decode with no host work between
calls (20 calls captured in a HIP graph and replayed), which at short contexts
is well below the per-call time (the host's enqueue of a call takes ~12 us).

Prints ONE JSON line: the decode time and bandwidth, the prefill time and
TFLOP/s, a roofline object for each, the other decode workloads and the
context-length sweep, and the oracle's CPU timings.
"""
from __future__ import annotations

import os

# The oracle's CPU baseline: BLAS / OpenMP threads are fixed before numpy is
# first imported (a value already set in the environment is kept).
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(os.cpu_count() or 1))

import argparse  # noqa: E402
import json  # noqa: E402
import math  # noqa: E402
import platform  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
N_DECODE = 16  # decode tokens per step on the cache the step's prompt built
MFMA_BF16_TFLOPS = 2500.0
MFMA_I8_TOPS = 5000.0
MFMA_F64_TFLOPS = 78.6


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other decode workloads and the context sweep after the timed steps")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the decode tokens (append + decode) on one built cache (profiling aid)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill probe + attention per step and print its fields (profiling aid)")
    ap.add_argument("--probe-only", action="store_true",
                    help="time only hq_probe_select at the 32K decode shape per step and print its time (profiling aid)")
    ap.add_argument("--sweep", action="store_true",
                    help="decode on the 8B GQA shape (B=16, 32/8 heads) at T = 1K..32K; prints one JSON line")
    ap.add_argument("--ablation", action="store_true",
                    help="decode output error of the cache policies (uniform INT4, hybrid 1%%/5%%) against the "
                         "all-bf16 cache on the 8B GQA shape at T = 1K..32K; prints one JSON line")
    ap.add_argument("--configs", action="store_true",
                    help="append + decode timed on every decode workload (4K 1 head, 32K 8B, 128K 8B, ragged 64K "
                         "70B-like); prints one JSON line")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain device copy of this size (HBM counter calibration) and exit")
    return ap.parse_args()


def _dev16(a, dtype, dev):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(dev)


class Timer:
    """HIP-event timing of one labelled call on the current stream."""

    def __init__(self):
        self.ev = {}

    def __call__(self, name, fn, *a, **kw):
        import torch
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        r = fn(*a, **kw)
        e.record()
        self.ev.setdefault(name, []).append((s, e))
        return r

    def ms(self, name):
        v = [s.elapsed_time(e) for s, e in self.ev.get(name, [])]
        return sum(v) / len(v) if v else float("nan")

    def pct(self, name, scale=1.0):
        """p10, median, p90 of the call times (ms x scale)."""
        v = sorted(s.elapsed_time(e) * scale for s, e in self.ev.get(name, []))
        if not v:
            return None
        q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]
        return [round(q(0.1), 2), round(q(0.5), 2), round(q(0.9), 2)]

    def reset(self):
        self.ev = {}


def decode_bytes_per_step(counts):
    """Algorithmic HBM bytes of one decode over the cache: 160 B per INT4
    token-head (64+64 code bytes, 2x16 meta bytes), 512 B per 16-bit token-head."""
    T, nq, nk = counts[..., 0], counts[..., 1], counts[..., 2]
    nring = T.clip(max=128)
    return int((nq * 160 + (nk + nring) * 512).sum())


def prefill_flops(T, Hq, B=1):
    pairs = T * (T + 1) // 2
    return 4.0 * 128 * pairs * Hq * B


def prefill_pair_split(T, W, sel_idx, sel_cnt, G):
    """Causal (query, key) pairs whose score is exact (window band or selected
    column) and INT8 (the rest), summed over query heads. A selected column j
    adds the rows i >= j + W that the band does not already cover."""
    import numpy as np
    total = T * (T + 1) // 2
    band = sum(min(i + 1, W) for i in range(T)) if W > 0 else 0
    exact = 0
    B, Hkv = sel_cnt.shape
    for b in range(B):
        for g in range(Hkv):
            j = sel_idx[b, g, : sel_cnt[b, g]].astype(np.int64)
            exact += G * (band + int(np.clip(T - (j + W), 0, None).sum()))
    heads = B * Hkv * G
    return exact, heads * total - exact


def prefill_roofline(T, W, sel_idx, sel_cnt, G, ms):
    """Mixed MFMA floor: INT8 QK pairs at the int8 peak, exact QK pairs and
    every PV pair at the 16-bit peak (2 * 128 flops per pair each)."""
    exact, low = prefill_pair_split(T, W, sel_idx, sel_cnt, G)
    per = 2.0 * 128
    f16_flops = per * exact + per * (exact + low)
    i8_ops = per * low
    floor_s = f16_flops / (MFMA_BF16_TFLOPS * 1e12) + i8_ops / (MFMA_I8_TOPS * 1e12)
    total = f16_flops + i8_ops
    achieved = total / (ms * 1e-3) / 1e12
    peak = total / floor_s / 1e12
    return {"bound": "mfma", "kernel": "hq_prefill_attn (INT8 stage + hybrid attention)",
            "achieved": round(achieved, 1), "peak": round(peak, 1), "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": prefill_traffic(),
            "floor_us": round(floor_s * 1e6, 1), "int8_qk_pair_frac": round(low / (exact + low), 4)}


def prefill_low_error(hq, pf, psel, pol, polf, heads=4, nrows=512):
    """Output error of the INT8 and the FP8 low-precision paths against exact
    causal attention (fp64, plain torch on the device) on the last `nrows`
    rows of the first `heads` query heads: the pages' open question of FP8 as
    another precision point, measured on the seeded inputs."""
    import torch
    T = pf["spec"].T
    outs = {}
    for name, p in (("int8", pol), ("fp8", polf)):
        o = hq.prefill_attn(pf["q"], pf["k"], pf["v"], psel[1], psel[2], p)
        outs[name] = o[0, :heads, T - nrows:].double()
    G = pf["spec"].Hq // pf["spec"].Hkv
    q = pf["q"][0, :heads, T - nrows:].double()
    k = pf["k"][0, [h // G for h in range(heads)]].double()
    v = pf["v"][0, [h // G for h in range(heads)]].double()
    s = torch.matmul(q, k.transpose(1, 2).contiguous()) / math.sqrt(q.shape[-1])
    i = torch.arange(T - nrows, T, device=s.device)[:, None]
    s = s.masked_fill(torch.arange(T, device=s.device)[None, :] > i, float("-inf"))
    ref = torch.matmul(torch.softmax(s, -1), v)
    err = {}
    for name, o in outs.items():
        d = o - ref
        err[f"{name}_rel_l2_vs_exact"] = float(d.norm() / ref.norm())
        err[f"{name}_max_abs_vs_exact"] = float(d.abs().max())
    err["error_sample"] = f"last {nrows} rows of query heads 0..{heads - 1}"
    return {k2: (round(v2, 7) if isinstance(v2, float) else v2) for k2, v2 in err.items()}


def prefill_routing_study(hq, pf, psel, heads=4, nrows=512, fracs=(5, 20)):
    """The pages' additivity experiment at the 16K prefill shape: output
    error against exact causal attention (fp64, plain torch on the device;
    last `nrows` rows of the first `heads` query heads) and time of the INT8
    prefill with no routing (window only), token routing (the probe's top 5%),
    tile routing (a fraction of each query block's key blocks by the INT8
    error bound) and both. recovered = error(none) - error(config); the
    ratio recovered(both) / (recovered(token) + recovered(tile)) is 1 when
    the two are additive and near max/sum when they cash the same slack."""
    import torch
    T = pf["spec"].T
    G = pf["spec"].Hq // pf["spec"].Hkv
    q = pf["q"][0, :heads, T - nrows:].double()
    k = pf["k"][0, [h // G for h in range(heads)]].double()
    v = pf["v"][0, [h // G for h in range(heads)]].double()
    s = torch.matmul(q, k.transpose(1, 2).contiguous()) / math.sqrt(q.shape[-1])
    i = torch.arange(T - nrows, T, device=s.device)[:, None]
    s = s.masked_fill(torch.arange(T, device=s.device)[None, :] > i, float("-inf"))
    ref = torch.matmul(torch.softmax(s, -1), v)
    empty_cnt = torch.zeros_like(psel[2])

    def run(keep, tile):
        pol = hq.Policy(tile_num=tile)
        cnt = psel[2] if keep else empty_cnt
        for _ in range(2):
            o = hq.prefill_attn(pf["q"], pf["k"], pf["v"], psel[1], cnt, pol, None, pf["out"])
        torch.cuda.synchronize()
        ev = []
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            o = hq.prefill_attn(pf["q"], pf["k"], pf["v"], psel[1], cnt, pol, None, pf["out"])
            b.record()
            ev.append((a, b))
        torch.cuda.synchronize()
        d = o[0, :heads, T - nrows:].double() - ref
        return {"rel_l2": round(float(d.norm() / ref.norm()), 6), "max_abs": round(float(d.abs().max()), 5),
                "ms": round(sorted(x.elapsed_time(y) for x, y in ev)[1], 3)}

    res = {"none": run(False, 0), "token_5pct": run(True, 0)}
    base = res["none"]["rel_l2"]
    for f in fracs:
        res[f"tile_{f}pct"] = run(False, f)
        res[f"token_5pct+tile_{f}pct"] = both = run(True, f)
        rt = base - res["token_5pct"]["rel_l2"]
        rl = base - res[f"tile_{f}pct"]["rel_l2"]
        rb = base - both["rel_l2"]
        res[f"additivity_tile_{f}pct"] = {"recovered_token": round(rt, 6), "recovered_tile": round(rl, 6),
                                          "recovered_both": round(rb, 6),
                                          "both_over_sum": round(rb / (rt + rl), 4) if rt + rl > 0 else None,
                                          "max_over_sum": round(max(rt, rl) / (rt + rl), 4) if rt + rl > 0 else None}
    res["error_sample"] = f"last {nrows} rows of query heads 0..{heads - 1} against exact fp64 attention"
    return res


def committed_traffic(profile, source, key):
    """HBM bytes per call from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary (each counter scaled by the factor a plain copy of known size
    gives for it); None when the kernel source changed after the counters
    were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile)
    src = os.path.join(ROOT, "kv_cache_amd", "csrc", source)
    try:
        text = open(path).read()
        m = re.search(r"```json\n(.*?)\n```", text, re.S)
        rec = json.loads(m.group(1))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, AttributeError, ValueError):
        return None
    if rec.get(key) != sha:
        return None
    return int(rec["hbm_bytes_per_launch"])


def decode_traffic(launch_bytes_alg):
    return committed_traffic("decode_8b_32k_split_traffic.md", "decode.hip", "decode_hip_sha256")


def prefill_traffic():
    return committed_traffic("prefill_8b_16k_traffic.md", "prefill.hip", "prefill_hip_sha256")


def _host_info():
    """CPU model and memory of this host (for the CPU baseline's record)."""
    model, mem = platform.processor() or platform.machine(), None
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
        for ln in open("/proc/meminfo"):
            if ln.startswith("MemTotal"):
                mem = f"{int(ln.split()[1]) / 2**20:.0f} GiB"
                break
    except OSError:
        pass
    return {"cpu": model, "logical_cpus": os.cpu_count(), "memory": mem}


def _parity(gpu, ref, n, what):
    """Parity summary of the units the oracle computed: max-abs and
    relative L2 of the GPU's output against it, beside the bars."""
    import numpy as np
    d = gpu.astype(np.float64) - ref
    return {"what": what, "units": n, "max_abs": float(f"{np.abs(d).max():.3e}"),
            "rel_l2": float(f"{np.linalg.norm(d) / np.linalg.norm(ref):.3e}"), "bar_max_abs": 2e-3, "bar_rel_l2": 1e-3}


def cpu_baseline(inp, sels_gpu, q, budget_s=15.0, gpu_out=None):
    """The oracle (numpy fp64) timed on this host for the unit the GPU's
    `value` times: one decode step's attention over an already built hybrid
    cache (all (b, g) of the 32K decode workload). Caches are built for
    whole (b, g) units until the time budget is spent (the build is timed as
    its own field, the once-per-prompt cost); the decode of those units is
    timed and scaled to all units. gpu_out: the library's decode of q over
    the same caches, compared with the oracle's on those units."""
    import numpy as np
    import oracle as O
    sp = inp.spec
    sm = float(np.float32(1 / math.sqrt(sp.D)))  # the fp32 scale the library receives
    G = sp.Hq // sp.Hkv
    col, sel, cnt, thr = sels_gpu
    t_build, t_dec, refs, gots = [], [], [], []
    start = time.perf_counter()
    for b in range(sp.B):
        for g in range(sp.Hkv):
            if time.perf_counter() - start > budget_s:
                break
            T = int(inp.seq_lens[b])
            t0 = time.perf_counter()
            k = O.to_f64(inp.k[b, g, :T], sp.dtype)
            v = O.to_f64(inp.v[b, g, :T], sp.dtype)
            idx = sel[b, g, : cnt[b, g]].astype(np.int64)
            c = O.build_cache(k, v, T, O.Selection(idx, len(idx), float(thr[b, g, 0:1].view(np.float32)[0]),
                                                   int(thr[b, g, 1])), 128, col[b, g, :T].astype(np.float64))
            t1 = time.perf_counter()
            qg = O.to_f64(q[b, g * G:(g + 1) * G], sp.dtype)
            o = O.decode_attention(qg, c, sm)
            t2 = time.perf_counter()
            t_build.append(t1 - t0)
            t_dec.append(t2 - t1)
            refs.append(o)
            gots.append(gpu_out[b, g * G:(g + 1) * G] if gpu_out is not None else o)
    n, units = len(t_dec), sp.B * sp.Hkv
    rec = {"value": round(sum(t_dec) / n * units * 1e6, 1), "unit": "us/step", "cores": _cpu_threads(),
           "kind": "oracle",
           "sample": f"decode attention (fp64) over the built hybrid cache of {n} of {units} (batch, KV head) "
                     f"units of one 32K decode step ({sum(t_dec):.1f} s), scaled x{units / n:.1f}",
           "cache_build_us_per_prompt": round(sum(t_build) / n * units * 1e6, 1)}
    rec.update(_host_info())
    if gpu_out is not None:
        rec["parity"] = _parity(np.stack(gots), np.stack(refs), n,
                                "hq_decode_attn over the prompt's hybrid cache vs the oracle, (batch, KV head) units")
    return rec

def _cpu_threads():
    """Threads the oracle's numpy BLAS actually runs with."""
    try:
        from threadpoolctl import threadpool_info
        n = [d["num_threads"] for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline_prefill(pin, sel_idx, sel_cnt, budget_s=8.0, gpu_head0=None):
    """The oracle's hybrid prefill timed on this host on sampled query rows of
    the 16K workload (INT8 stage of the head + per-row fp64 attention),
    scaled to all rows of all heads, in ms. gpu_head0: the library's output
    of head 0 [T][D], compared with the oracle's on the sampled rows."""
    import numpy as np
    import oracle as O
    sp = pin.spec
    G = sp.Hq // sp.Hkv
    sm = float(np.float32(1 / math.sqrt(sp.D)))  # the fp32 scale the library receives
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    q = O.to_f64(pin.q[0, 0], sp.dtype)
    k = O.to_f64(pin.k[0, 0], sp.dtype)
    v = O.to_f64(pin.v[0, 0], sp.dtype)
    q8, sq = O.int8_block_quantize(q)
    k8, sk = O.int8_block_quantize(k)
    t_quant = time.perf_counter() - t0
    S = sel_idx[0, 0, : sel_cnt[0, 0]].astype(np.int64)
    done, t_rows, refs, gots = 0, 0.0, [], []
    while t_rows < budget_s:
        rows = rng.integers(0, sp.T, size=16)
        t1 = time.perf_counter()
        o = O.prefill_attention_rows(q, k, v, S, 128, sm, q8, sq, k8, sk, rows)
        t_rows += time.perf_counter() - t1
        done += len(rows)
        if gpu_head0 is not None:
            refs.append(o)
            gots.append(gpu_head0[rows])
    # rows are uniform over [0, T), so the mean row cost scales to all rows
    full_s = t_rows / done * sp.T * sp.Hq + t_quant * (sp.Hq + sp.Hkv) / 2
    rec = {"value": round(full_s * 1e3, 1), "unit": "ms/prefill", "cores": _cpu_threads(), "kind": "oracle",
           "sample": f"{done} uniformly drawn query rows of head 0 of the 16K prefill "
                     f"({t_rows:.1f} s) plus one head's INT8 stage, scaled to {sp.T} rows x {sp.Hq} heads"}
    if gpu_head0 is not None:
        rec["parity"] = _parity(np.concatenate(gots), np.concatenate(refs), done,
                                "hq_prefill_attn head 0 vs the oracle, query rows")
    return rec


def _graph_decode_us(hq, cache, q, out, n=20, reps=10):
    """Device time of one decode with no host work between calls: n calls of
    hq_decode_attn_noalloc captured in a HIP graph, replayed `reps` times
    (microseconds per call). The first replay is checked bit for bit against
    the eager call's output."""
    import torch
    hq.decode_attn_noalloc(cache, q, None, out)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for _ in range(n):
                hq.decode_attn_noalloc(cache, q, None, out)
    torch.cuda.synchronize()
    out.zero_()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("graph-replayed decode differs from the eager call")
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    torch.cuda.synchronize()
    del g
    return s.elapsed_time(e) * 1e3 / (n * reps)


def _time_decode(hq, cache, knew, vnew, q, out, steps, warmup):
    """Append + decode per step on one built cache; the Timer of the calls."""
    import torch
    tm = Timer()
    for i in range(warmup + steps):
        if i == warmup:
            torch.cuda.synchronize()
            tm.reset()
        tm("append_kv", hq.append_kv, cache, knew, vnew)
        tm("decode_attn", hq.decode_attn, cache, q, None, out)
    torch.cuda.synchronize()
    return tm


def _decode_workload(hq, name, steps, warmup, cold_mib=0):
    """One decode workload at its full shape: probe, quantize, then `steps`
    timed append + decode calls (after `warmup`), each decode with its own
    query. cold_mib > 0: also time decodes that each follow a write of that
    many MiB (the caches no longer hold the cache's bytes)."""
    import numpy as np
    import torch
    from synth.inputs import CONFIGS, make_append_tokens, make_decode_inputs
    dev = "cuda:0"
    pol = hq.Policy()
    spec = CONFIGS[name]
    t0 = time.perf_counter()
    inp = make_decode_inputs(spec)
    n = steps + warmup
    kn, vn, qn = make_append_tokens(spec, inp.outlier_channels, n)
    k, v = _dev16(inp.k, spec.dtype, dev), _dev16(inp.v, spec.dtype, dev)
    qp = _dev16(inp.q_probe, spec.dtype, dev)
    knew, vnew, qd = _dev16(kn, spec.dtype, dev), _dev16(vn, spec.dtype, dev), _dev16(qn, spec.dtype, dev)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float16
    cache = hq.HybridCache(spec.B, spec.Hkv, spec.T + n, spec.T, dt, dev, pol)
    col, sel, cnt, thr = hq.probe_select(qp, k, lens, pol)
    hq.quantize_kv(cache, k, v, lens, sel, cnt, col, thr)
    keep0 = cache.counts()[..., 2].clone()
    out = torch.empty((spec.B, spec.Hq, spec.D), dtype=torch.float32, device=dev)
    tm = Timer()
    for i in range(n):
        if i == warmup:
            torch.cuda.synchronize()
            tm.reset()
        tm("append_kv", hq.append_kv, cache, knew[i], vnew[i])
        tm("decode_attn", hq.decode_attn, cache, qd[i], None, out)
    torch.cuda.synchronize()
    counts = cache.counts().cpu().numpy()
    by = decode_bytes_per_step(counts)
    p = tm.pct("decode_attn", 1e3)
    dus = p[1]  # the median call: robust to a rare slow call in a long loop of short ones
    rec = {"B": spec.B, "Hq": spec.Hq, "Hkv": spec.Hkv, "T": spec.T, "dtype": spec.dtype,
           "decode_us": round(dus, 2), "decode_us_p10_p50_p90": p, "decode_us_mean": round(tm.ms("decode_attn") * 1e3, 2),
           "append_us": round(tm.pct("append_kv", 1e3)[1], 2),
           "steps": steps, "bytes": by, "TBps": round(by / (dus * 1e-6) / 1e12, 3),
           "frac_of_peak": round(by / (dus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
           "kept_by_append_rule": int((cache.counts()[..., 2] - keep0).sum().item())}
    gus = _graph_decode_us(hq, cache, qd[n - 1], out)
    rec["decode_us_graph"] = round(gus, 2)
    rec["frac_of_peak_graph"] = round(by / (gus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    if spec.ragged_min is not None:
        rec["seq_lens"] = [int(x) for x in inp.seq_lens]
        # the same batch in the ragged INT4 layout (hq_cache_layout_ragged):
        # each sequence sized for its own prompt plus the decode tokens
        caps = [int(x) + n for x in inp.seq_lens]
        rcache = hq.HybridCache(spec.B, spec.Hkv, caps, spec.T, dt, dev, pol)
        hq.quantize_kv(rcache, k, v, lens, sel, cnt, col, thr)
        tr = Timer()
        for i in range(n):
            hq.append_kv(rcache, knew[i], vnew[i])
            tr("decode_attn", hq.decode_attn, rcache, qd[i], None, out)
        torch.cuda.synchronize()
        pool = lambda sz: int(sz.k_codes + sz.v_codes + sz.k_meta + sz.v_meta + sz.q_pos)
        rec["ragged_layout"] = {"int4_store_bytes": pool(rcache.sizes), "uniform_int4_store_bytes": pool(cache.sizes),
                                "decode_us": tr.pct("decode_attn", 1e3)[1],
                                "same_counts": bool(torch.equal(rcache.counts(), cache.counts()))}
        del rcache
    if cold_mib:
        scrub = torch.empty(cold_mib << 20, dtype=torch.uint8, device=dev)
        tc = Timer()
        for i in range(steps):
            scrub.fill_(i & 255)
            tc("decode_attn", hq.decode_attn, cache, qd[i % n], None, out)
        torch.cuda.synchronize()
        rec["cold_decode_us"] = tc.pct("decode_attn", 1e3)[1]
        rec["cold_decode_us_p10_p50_p90"] = tc.pct("decode_attn", 1e3)
        rec["cold"] = f"each decode after a {cold_mib} MiB device write"
        del scrub
    print(f"# workload {name}: {rec} ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
    del cache, k, v, inp, knew, vnew, qd
    torch.cuda.empty_cache()
    return rec


def decode_workloads(args):
    """The decode workloads other than the 32K headline, each at its full
    shape: 1-head 4K (warm, and cold after a 512 MiB write), 8B 128K with 64
    consecutive appends, the ragged 70B-like 64K."""
    import kv_cache_amd as hq
    return {
        "decode_4k_1head": _decode_workload(hq, "decode_4k_1head", 200, 20, cold_mib=512),
        "decode_8b_128k_append": _decode_workload(hq, "decode_8b_128k_append", 64, 0),
        "decode_70b_ragged_64k": _decode_workload(hq, "decode_70b_ragged_64k", max(20, args.steps), 5),
    }


def decode_configs(args):
    print(json.dumps({"workloads": decode_workloads(args), "steps": args.steps, "warmup": args.warmup}), flush=True)

def decode_ablation(args):
    """Decode output error of each cache policy on the seeded 8B GQA inputs
    (outlier K channels, planted vertical lines) at T = 1K..32K: all-INT4,
    INT4 + bf16 window, the retained-ratio sweep (1, 2, 5, 10, 20% + 128
    window), the window sweep (64, 128, 256, 512 at 5%), every position in
    bf16. Each policy's output comes from hq_decode_attn on its own cache
    (probe, select, quantize, decode: all kernels). The errors are taken
    against exact softmax attention over the bf16 K/V in fp64, and two
    measurements ride along, computed with a few lines of plain torch on the
    device (diagnostics, not paths of the method): a uniform per-token INT8
    cache's output (s = max|x| / 127 per token, round half to even, K and V)
    and each kept set's share of the decode query's exact attention mass."""
    import dataclasses
    import torch
    import kv_cache_amd as hq
    from synth.inputs import CONFIGS, make_append_tokens, make_decode_inputs
    dev = "cuda:0"
    policies = [("int4_all", hq.Policy(0, 100, 0, 64)), ("int4_window128", hq.Policy(0, 100, 128, 64))]
    policies += [(f"hybrid_{r}pct", hq.Policy(r, 100, 128, 64)) for r in (1, 2, 5, 10, 20)]
    policies += [(f"hybrid_5pct_w{w}", hq.Policy(5, 100, w, 64)) for w in (64, 256, 512)]
    policies += [("bf16_all", hq.Policy(100, 100, 128, 64))]

    def int8_token(x):  # [..., T, D] fp64 exact -> dequantized uniform per-token INT8 (fp32 decisions)
        xf = x.float()
        s = xf.abs().amax(dim=-1, keepdim=True) / 127.0
        c = torch.where(s > 0, torch.round(xf / torch.where(s > 0, s, torch.ones_like(s))).clamp(-127, 127),
                        torch.zeros_like(xf))
        return c.double() * s.double()

    rows = []
    for T in (1024, 4096, 16384, 32768):
        spec = dataclasses.replace(CONFIGS["decode_8b_32k"], name=f"decode_8b_gqa_b16_{T}", T=T)
        inp = make_decode_inputs(spec)
        _, _, qn = make_append_tokens(spec, inp.outlier_channels, 1)
        k, v = _dev16(inp.k, "bf16", dev), _dev16(inp.v, "bf16", dev)
        qp, q = _dev16(inp.q_probe, "bf16", dev), _dev16(qn[0], "bf16", dev)
        lens = torch.from_numpy(inp.seq_lens).to(dev)
        B, Hkv, G, D = spec.B, spec.Hkv, spec.Hq // spec.Hkv, spec.D
        sm = 1.0 / math.sqrt(D)
        # exact attention, the INT8 line and the attention probabilities, per batch row
        exact = torch.empty((B, spec.Hq, D), dtype=torch.float64, device=dev)
        int8 = torch.empty_like(exact)
        probs = []
        for b in range(B):
            qb = q[b].double().view(Hkv, G, D)
            Kb, Vb = k[b].double(), v[b].double()
            p = torch.softmax(qb @ Kb.transpose(1, 2) * sm, dim=-1)      # [Hkv][G][T]
            exact[b] = (p @ Vb).view(spec.Hq, D)
            p8 = torch.softmax(qb @ int8_token(Kb).transpose(1, 2) * sm, dim=-1)
            int8[b] = (p8 @ int8_token(Vb)).view(spec.Hq, D)
            probs.append(p.sum(dim=1) / G)                                # [Hkv][T] mean over the G heads
        row = {"T": T}

        def err(o):
            d = o - exact
            return {"mse": float((d * d).mean()), "rel_l2": float(d.norm() / exact.norm()),
                    "max_abs": float(d.abs().max())}

        for name, pol in policies:
            cache = hq.HybridCache(B, Hkv, T, T, torch.bfloat16, dev, pol)
            col, sel, cnt, thr = hq.probe_select(qp, k, lens, pol)
            hq.quantize_kv(cache, k, v, lens, sel, cnt, col, thr)
            out = hq.decode_attn(cache, q).double()
            e = err(out)
            # kept set = the selection + the last W positions
            cov = []
            for b in range(B):
                m = torch.zeros((Hkv, T), dtype=torch.bool, device=dev)
                for g in range(Hkv):
                    n = int(cnt[b, g])
                    m[g, sel[b, g, :n].long()] = True
                m[:, max(0, T - pol.window):] = True
                cov.append((probs[b] * m).sum(dim=-1))
            e["kept_mass"] = float(torch.stack(cov).mean())
            row[name] = e
            del cache
            torch.cuda.empty_cache()
        row["uniform_int8"] = err(int8)
        rows.append(row)
        print(f"# ablation T={T}: " + ", ".join(f"{n} {row[n]['rel_l2']:.3g}" for n in row if n != "T"),
              file=sys.stderr, flush=True)
        del k, v, inp, probs, exact, int8
        torch.cuda.empty_cache()
    print(json.dumps({"ablation": "decode_8b_gqa_b16 (B=16, 32/8 heads, bf16 inputs); error of each policy's fp32 "
                                  "decode output (hq_decode_attn on its own cache) and of a uniform per-token INT8 "
                                  "cache (plain torch) against exact fp64 attention over the bf16 K/V; kept_mass: "
                                  "share of the decode query's exact attention mass on the kept set (selection + "
                                  "window), mean over (b, KV head) of the G heads' mean", "rows": rows}), flush=True)


def sweep(args):
    """Decode (append + decode per step, on one built cache) on the 8B GQA
    shape at the context lengths of the pages' speed table: absolute time and
    bandwidth per length, the streaming-read rate of the same INT4 store, and
    the same decode kernel on a cache that keeps every position in bf16 (ratio
    100%: the full-precision decode), for the hybrid / bf16 speed ratio. Then
    the 16K prefill, hybrid against every column selected (bf16 scores
    everywhere)."""
    import dataclasses
    import torch
    import kv_cache_amd as hq
    from synth.inputs import CONFIGS, make_append_tokens, make_decode_inputs, make_prefill_inputs
    dev = "cuda:0"
    pol = hq.Policy()
    pol_bf16 = hq.Policy(100, 100, pol.window, pol.probe_rows)
    rows = []
    for T in (1024, 2048, 4096, 8192, 16384, 32768):
        spec = dataclasses.replace(CONFIGS["decode_8b_32k"], name=f"decode_8b_gqa_b16_{T}", T=T)
        inp = make_decode_inputs(spec)
        kn, vn, qn = make_append_tokens(spec, inp.outlier_channels, 1)
        k, v = _dev16(inp.k, "bf16", dev), _dev16(inp.v, "bf16", dev)
        qp, q = _dev16(inp.q_probe, "bf16", dev), _dev16(qn[0], "bf16", dev)
        knew, vnew = _dev16(kn[0], "bf16", dev), _dev16(vn[0], "bf16", dev)
        lens = torch.from_numpy(inp.seq_lens).to(dev)
        cache = hq.HybridCache(spec.B, spec.Hkv, T + 64 + args.steps + args.warmup, T, torch.bfloat16, dev, pol)
        col, sel, cnt, thr = hq.probe_select(qp, k, lens, pol)
        hq.quantize_kv(cache, k, v, lens, sel, cnt, col, thr)
        out = torch.empty((spec.B, spec.Hq, spec.D), dtype=torch.float32, device=dev)
        tm = _time_decode(hq, cache, knew, vnew, q, out, args.steps, args.warmup)
        gus = _graph_decode_us(hq, cache, q, out)
        sink = hq.diag_read_int4(cache)
        for _ in range(10):
            tm("diag", hq.diag_read_int4, cache, sink)
        torch.cuda.synchronize()
        counts = cache.counts().cpu().numpy()
        by = decode_bytes_per_step(counts)
        dms = tm.ms("decode_attn")
        i4 = int((counts[..., 1] * 160).sum())
        rows.append({"T": T, "decode_us": round(dms * 1e3, 2), "decode_us_p10_p50_p90": tm.pct("decode_attn", 1e3),
                     "decode_us_graph": round(gus, 2),
                     "frac_of_peak_graph": round(by / (gus * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "bytes": by, "TBps": round(by / (dms * 1e-3) / 1e12, 3),
                     "frac_of_peak": round(by / (dms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "int4_stream_TBps": round(i4 / (tm.ms("diag") * 1e-3) / 1e12, 3)})
        del cache
        torch.cuda.empty_cache()
        # the same kernel with every position kept in bf16
        cache = hq.HybridCache(spec.B, spec.Hkv, T + 64 + args.steps + args.warmup, T, torch.bfloat16, dev, pol_bf16)
        col, sel, cnt, thr = hq.probe_select(qp, k, lens, pol_bf16)
        hq.quantize_kv(cache, k, v, lens, sel, cnt, col, thr)
        tmb = _time_decode(hq, cache, knew, vnew, q, out, args.steps, args.warmup)
        cb = cache.counts().cpu().numpy()
        byb = decode_bytes_per_step(cb)
        bms = tmb.ms("decode_attn")
        rows[-1].update({"bf16_decode_us": round(bms * 1e3, 2), "bf16_decode_us_p10_p50_p90": tmb.pct("decode_attn", 1e3),
                         "bf16_bytes": byb, "bf16_TBps": round(byb / (bms * 1e-3) / 1e12, 3),
                         # ratio of the medians (robust to a slow call at short lengths)
                         "bf16_over_hybrid": round(tmb.pct("decode_attn", 1e3)[1] / tm.pct("decode_attn", 1e3)[1], 3),
                         # tokens that left the window during the timed appends
                         # and ranked below the selection threshold
                         "bf16_cache_int4_tokens": int(cb[..., 1].sum())})
        print(f"# sweep T={T}: {rows[-1]}", file=sys.stderr, flush=True)
        del cache, k, v, inp
        torch.cuda.empty_cache()
    # prefill at 16K: hybrid against every column selected
    pspec = CONFIGS["prefill_8b_16k"]
    pin = make_prefill_inputs(pspec)
    pq, pk, pv = _dev16(pin.q, "bf16", dev), _dev16(pin.k, "bf16", dev), _dev16(pin.v, "bf16", dev)
    plens = torch.full((1,), pspec.T, dtype=torch.int32, device=dev)
    pqp = pq[:, :, pspec.T - 64:].contiguous()
    pout = torch.empty((1, pspec.Hq, pspec.T, 128), dtype=torch.float32, device=dev)
    prefill = {"T": pspec.T}
    for name, pl in (("hybrid", pol), ("bf16", pol_bf16)):
        psel = hq.probe_select(pqp, pk, plens, pl)
        tmp = Timer()
        for i in range(3 + max(5, args.steps // 2)):
            if i == 3:
                torch.cuda.synchronize()
                tmp.reset()
            tmp("prefill_attn", hq.prefill_attn, pq, pk, pv, psel[1], psel[2], pl, None, pout)
        torch.cuda.synchronize()
        prefill[f"{name}_ms"] = round(tmp.ms("prefill_attn"), 3)
        prefill[f"{name}_ms_p10_p50_p90"] = tmp.pct("prefill_attn", 1.0)
    prefill["bf16_over_hybrid"] = round(prefill["bf16_ms_p10_p50_p90"][1] / prefill["hybrid_ms_p10_p50_p90"][1], 3)
    print(f"# sweep prefill: {prefill}", file=sys.stderr, flush=True)
    return {"workload": "decode_8b_gqa_b16 (B=16, 32/8 heads, bf16, top-5% + 128 window, INT4 g32)",
            "steps": args.steps, "warmup": args.warmup, "rows": rows, "prefill_16k": prefill}


def decode_sweep(args):
    print(json.dumps({"sweep": sweep(args)}), flush=True)




def prefill_only(args):
    """Probe + hybrid prefill attention on the 16K workload only."""
    import torch
    import kv_cache_amd as hq
    from synth.inputs import CONFIGS, make_prefill_inputs
    dev = "cuda:0"
    pspec = CONFIGS["prefill_8b_16k"]
    pin = make_prefill_inputs(pspec)
    q, k, v = (_dev16(x, "bf16", dev) for x in (pin.q, pin.k, pin.v))
    lens = torch.full((1,), pspec.T, dtype=torch.int32, device=dev)
    qprobe = q[:, :, pspec.T - 64:].contiguous()
    out = torch.empty((1, pspec.Hq, pspec.T, 128), dtype=torch.float32, device=dev)
    pol = hq.Policy()
    tm = Timer()
    col, sel, cnt, thr = hq.probe_select(qprobe, k, lens, pol)
    for _ in range(args.warmup):
        hq.prefill_attn(q, k, v, sel, cnt, pol, None, out)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        tm("prefill_attn", hq.prefill_attn, q, k, v, sel, cnt, pol, None, out)
    torch.cuda.synchronize()
    pms = tm.ms("prefill_attn")
    res = {"prefill_ms": round(pms, 3),
           "prefill_TFLOPs": round(prefill_flops(pspec.T, pspec.Hq) / (pms * 1e-3) / 1e12, 1),
           "prefill_roofline": prefill_roofline(pspec.T, pol.window, sel.cpu().numpy(), cnt.cpu().numpy(),
                                                pspec.Hq // pspec.Hkv, pms)}
    print(json.dumps(res), flush=True)


def probe_only(args):
    """hq_probe_select (probe + top-k) on the 32K decode workload only."""
    import torch
    import kv_cache_amd as hq
    from synth.inputs import CONFIGS, make_decode_inputs
    dev = "cuda:0"
    spec = CONFIGS["decode_8b_32k"]
    inp = make_decode_inputs(spec)
    qp, k = _dev16(inp.q_probe, spec.dtype, dev), _dev16(inp.k, spec.dtype, dev)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    pol = hq.Policy()
    tm = Timer()
    for _ in range(args.warmup):
        hq.probe_select(qp, k, lens, pol)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        tm("probe_select", hq.probe_select, qp, k, lens, pol)
    torch.cuda.synchronize()
    print(json.dumps({"probe_select_ms": round(tm.ms("probe_select"), 3), "workload": "decode_8b_32k",
                      "steps": args.steps}), flush=True)


def main():
    args = _args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import kv_cache_amd as hq
    from synth.inputs import CONFIGS, make_append_tokens, make_decode_inputs, make_prefill_inputs

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n}))
        return

    if args.prefill_only:
        return prefill_only(args)
    if args.probe_only:
        return probe_only(args)
    if args.sweep:
        return decode_sweep(args)
    if args.ablation:
        return decode_ablation(args)
    if args.configs:
        return decode_configs(args)
    t_gen = time.perf_counter()
    spec = CONFIGS["decode_8b_32k"]
    inp = make_decode_inputs(spec)
    kn, vn, qn = make_append_tokens(spec, inp.outlier_channels, N_DECODE)
    print(f"# generated decode inputs in {time.perf_counter() - t_gen:.1f}s", file=sys.stderr, flush=True)
    pol = hq.Policy()
    B, Hq, Hkv, T, D = spec.B, spec.Hq, spec.Hkv, spec.T, spec.D
    k = _dev16(inp.k, "bf16", dev)
    v = _dev16(inp.v, "bf16", dev)
    qp = _dev16(inp.q_probe, "bf16", dev)
    qd, knew, vnew = _dev16(qn, "bf16", dev), _dev16(kn, "bf16", dev), _dev16(vn, "bf16", dev)
    lens = torch.from_numpy(inp.seq_lens).to(dev)
    cache = hq.HybridCache(B, Hkv, T + N_DECODE, T, torch.bfloat16, dev, pol)

    pf = None
    if not args.no_prefill and not args.decode_only:
        pspec = CONFIGS["prefill_8b_16k"]
        pin = make_prefill_inputs(pspec)
        pf = dict(spec=pspec, q=_dev16(pin.q, "bf16", dev), k=_dev16(pin.k, "bf16", dev),
                  v=_dev16(pin.v, "bf16", dev), lens=torch.full((1,), pspec.T, dtype=torch.int32, device=dev))
        pf["qprobe"] = pf["q"][:, :, pspec.T - 64:].contiguous()
        pf["out"] = torch.empty((1, pspec.Hq, pspec.T, 128), dtype=torch.float32, device=dev)
        if args.no_cpu_baseline:
            del pin
        else:
            pf["pin"] = pin
        print("# generated prefill inputs", file=sys.stderr, flush=True)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    tm = Timer()

    def step():
        if not args.decode_only:
            col, sel, cnt, thr = tm("probe_select", hq.probe_select, qp, k, lens, pol)
            tm("quantize_kv", hq.quantize_kv, cache, k, v, lens, sel, cnt, col, thr)
        for i in range(N_DECODE):
            tm("append_kv", hq.append_kv, cache, knew[i], vnew[i])
            first = i == 0 and not args.decode_only
            tm("decode_first" if first else "decode_attn", hq.decode_attn, cache, qd[i], None, out)
        if pf is not None:
            psel = tm("prefill_probe_select", hq.probe_select, pf["qprobe"], pf["k"], pf["lens"], pol)
            tm("prefill_attn", hq.prefill_attn, pf["q"], pf["k"], pf["v"], psel[1], psel[2], pol, None, pf["out"])

    if args.decode_only:
        # one built cache; the step is append + decode only (the cache grows by
        # N_DECODE tokens per step)
        cache = hq.HybridCache(B, Hkv, T + N_DECODE * (args.steps + args.warmup), T, torch.bfloat16, dev, pol)
        col, sel, cnt, thr = hq.probe_select(qp, k, lens, pol)
        hq.quantize_kv(cache, k, v, lens, sel, cnt, col, thr)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    tm.reset()
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    s0.record()
    for _ in range(args.steps):
        step()
    s1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = s0.elapsed_time(s1) / args.steps
    print(f"# timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)

    counts = cache.counts().cpu().numpy()
    dec_ms = tm.ms("decode_attn")
    dbytes = decode_bytes_per_step(counts)
    res = {
        "metric": "hybrid decode attn us/step + achieved HBM TB/s @32K; prefill TFLOP/s",
        "value": round(dec_ms * 1e3, 2),
        "unit": "us/step",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4+bf16 cache, fp32 accumulate",
        "data": "synthetic (seeded; Llama-3.1-8B attention shapes, outlier K channels, planted vertical lines)",
        "config": {"workload": "decode_8b_gqa_b16_32k (+ prefill_8b_gqa_16k causal)", "B": B, "Hq": Hq,
                   "Hkv": Hkv, "T": T, "head_dim": D, "keep": "top-5% + 128 window", "int4_group": 32,
                   "decode_tokens_per_step": N_DECODE},
        "decode_us": round(dec_ms * 1e3, 2),
        "decode_TBps": round(dbytes / (dec_ms * 1e-3) / 1e12, 3),
        "decode_bytes": dbytes,
        "decode_us_p10_p50_p90": tm.pct("decode_attn", 1e3),
        "append_us": round(tm.ms("append_kv") * 1e3, 2),
        "wall_s": round(wall, 3),
    }
    if not args.decode_only:
        res["decode_us_full_step"] = round(tm.ms("decode_first") * 1e3, 2)
        res["probe_select_ms"] = round(tm.ms("probe_select"), 3)
        res["quantize_ms"] = round(tm.ms("quantize_kv"), 3)
    res["roofline"] = {"bound": "hbm", "kernel": "hq_decode_attn (split-K + reduce)",
                       "achieved": round(dbytes / (dec_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                       "unit": "GB/s", "frac": round(dbytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "traffic": decode_traffic(dbytes)}
    # The achievable rate of the decode's access pattern on this GPU: the INT4
    # store streamed by hq_diag_read_int4 (same splits, tiles and loads, no
    # compute), timed after the step loop.
    int4_bytes = int((counts[..., 1] * 160).sum())
    sink = hq.diag_read_int4(cache)
    for _ in range(3):
        hq.diag_read_int4(cache, sink)
    torch.cuda.synchronize()
    for _ in range(10):
        tm("diag_read_int4", hq.diag_read_int4, cache, sink)
    torch.cuda.synchronize()
    ach = int4_bytes / (tm.ms("diag_read_int4") * 1e-3) / 1e9
    res["roofline"]["achievable"] = round(ach, 1)
    res["roofline"]["frac_of_achievable"] = round(res["roofline"]["achieved"] / ach, 4)
    res["int4_stream_read"] = {"bytes": int4_bytes, "us": round(tm.ms("diag_read_int4") * 1e3, 2),
                               "GBps": round(ach, 1)}
    # Re-probe of the step's cache (prompt + N_DECODE decode tokens) from its
    # last 64 query rows (the prompt's last 64 - N_DECODE probe rows, then the
    # decode queries), timed after the step loop: a periodic call, not a step.
    qr = torch.cat([qp[:, :, N_DECODE:], qd.permute(1, 2, 0, 3)], dim=2).contiguous()
    rp = hq.reprobe(cache, qr)
    for _ in range(2):
        rp = hq.reprobe(cache, qr, None, None, rp[5])
    torch.cuda.synchronize()
    for _ in range(5):
        rp = tm("reprobe", hq.reprobe, cache, qr, None, None, rp[5])
    torch.cuda.synchronize()
    npers, rcnt = rp[4].cpu().numpy(), rp[2].cpu().numpy()
    frac = npers / np.maximum(rcnt, 1)
    res["reprobe"] = {"ms": round(tm.ms("reprobe"), 3), "T": int(counts[0, 0, 0]),
                      "persistence_mean": round(float(frac.mean()), 4),
                      "persistence_min": round(float(frac.min()), 4)}
    del rp
    if pf is not None:
        pms = tm.ms("prefill_attn")
        psp = pf["spec"]
        fl = prefill_flops(psp.T, psp.Hq)
        res["prefill_ms"] = round(pms, 3)
        res["prefill_ms_p10_p50_p90"] = tm.pct("prefill_attn")
        res["prefill_TFLOPs"] = round(fl / (pms * 1e-3) / 1e12, 1)
        res["prefill_probe_select_ms"] = round(tm.ms("prefill_probe_select"), 3)
        psel = hq.probe_select(pf["qprobe"], pf["k"], pf["lens"], pol)
        psel_idx, psel_cnt = psel[1].cpu().numpy(), psel[2].cpu().numpy()
        res["prefill_roofline"] = prefill_roofline(psp.T, pol.window, psel_idx, psel_cnt, psp.Hq // psp.Hkv, pms)
        # the same prefill with the OCP FP8 (E4M3) low-precision path, timed
        # after the step loop (an option of the operator, not a step)
        polf = hq.Policy(low_fmt=hq.HQ_LOW_FP8)
        for _ in range(2):
            hq.prefill_attn(pf["q"], pf["k"], pf["v"], psel[1], psel[2], polf, None, pf["out"])
        torch.cuda.synchronize()
        for _ in range(5):
            tm("prefill_attn_fp8", hq.prefill_attn, pf["q"], pf["k"], pf["v"], psel[1], psel[2], polf, None,
               pf["out"])
        torch.cuda.synchronize()
        fms = tm.ms("prefill_attn_fp8")
        fr = prefill_roofline(psp.T, pol.window, psel_idx, psel_cnt, psp.Hq // psp.Hkv, fms)
        res["prefill_fp8"] = {"ms": round(fms, 3), "TFLOPs": round(fl / (fms * 1e-3) / 1e12, 1),
                              "frac": fr["frac"], "low_fmt": "OCP FP8 E4M3, per-64-token block scale"}
        res["prefill_fp8"].update(prefill_low_error(hq, pf, psel, pol, polf))
        res["prefill_routing"] = prefill_routing_study(hq, pf, psel)
    sels = tuple(t.cpu().numpy() for t in (hq.probe_select(qp, k, lens, pol)))
    par_dec = par_pf = None
    if not args.no_cpu_baseline:
        # the library's outputs on the units the oracle legs compute: decode of
        # the second decode query over the prompt's cache (the oracle builds the
        # same cache from the same selection), and the plain INT8 prefill
        pc = hq.HybridCache(B, Hkv, T + N_DECODE, T, torch.bfloat16, dev, pol)
        pcol, psl, pcnt, pthr = hq.probe_select(qp, k, lens, pol)
        hq.quantize_kv(pc, k, v, lens, psl, pcnt, pcol, pthr)
        par_dec = hq.decode_attn(pc, qd[1]).cpu().numpy()
        del pc
        if pf is not None:
            par_pf = hq.prefill_attn(pf["q"], pf["k"], pf["v"], psel[1], psel[2], pol)[0, 0].cpu().numpy()
    del cache, k, v, knew, vnew
    if pf is not None:
        for key in ("q", "k", "v", "out", "qprobe"):
            pf.pop(key)
    torch.cuda.empty_cache()
    if not args.decode_only and not args.no_workloads:
        res["workloads"] = decode_workloads(args)
        res["sweep"] = sweep(args)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, sels, qn[1], gpu_out=par_dec)
        if pf is not None and "pin" in pf:
            res["cpu_baseline_prefill"] = cpu_baseline_prefill(pf["pin"], psel_idx, psel_cnt, gpu_head0=par_pf)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
