"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the oracle on the same inputs, compare within the stated bars."""
import math

import numpy as np

import oracle as O

ATOL = 2e-3      # max-abs bar for attention outputs
RTOL_L2 = 1e-3   # relative-L2 bar for attention outputs
# Column-score bar: the probe's stated bound. A stored term is off by at most
# d = ln2 (logit budget 0.5e-7 + 2^-26, the fp32 rounding of the exponent's
# fraction) + 1.5 2^-24 (the hardware exponential on [-1/2, 1/2], checked over
# every fp32 input by test_gpu_diag.py; it measures 1.395 2^-24), a row's
# normaliser (a sum of such terms) by at most d, so a score by at most
# 2 d + 2^-24 (the final fp32 rounding) ~ 3.28e-7 relative.
HW_EXP2_REL = 1.5 * 2.0 ** -24
SCORE_RTOL = 2 * (math.log(2) * (0.5e-7 + 2.0 ** -26) + HW_EXP2_REL) + 2.0 ** -24


# Selection flips are allowed only between near-ties: columns whose oracle
# scores differ by less than this, relative (twice the score bar, 6.6e-7, is
# below it).
NEAR_TIE = 1e-6


def compare_selection(gpu_idx, gpu_cnt, c_or, T, W, keep):
    """The GPU's selected set against the oracle's selection on its fp64
    scores c_or. Returns the number of near-tie flips (a column swapped with
    one whose oracle score is within NEAR_TIE); fails on any other
    difference."""
    s = O.select_topk(c_or, T, W, keep[0], keep[1])
    assert gpu_cnt == s.k
    a, b = set(gpu_idx.tolist()), set(s.idx.tolist())
    only_gpu, only_or = sorted(a - b), sorted(b - a)
    assert len(only_gpu) == len(only_or)
    for x, y in zip(sorted(only_gpu, key=lambda j: -c_or[j]), sorted(only_or, key=lambda j: c_or[j])):
        gap = abs(c_or[x] - c_or[y]) / max(c_or[x], c_or[y])
        assert gap < NEAR_TIE, f"selection flip with gap {gap:.3e} (positions {x}, {y})"
    return len(only_gpu)


def fp32_scale(D):
    """The softmax scale 1/sqrt(D) as the library receives it: an fp32 value
    (its `float sm_scale` argument). The oracle is given this same number, so
    both sides compute the same softmax; 1/sqrt(128) rounded to fp32 differs
    from the real number by ~3e-8 relative, which on logits of ~20 (log2
    units) would alone move column scores by ~3e-7."""
    return float(np.float32(1 / math.sqrt(D)))


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float16


def to_dev(bits: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch_dtype(dtype)).cuda()


def ints_to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def oracle_selection(inp, window=128, keep=(5, 100)):
    """Oracle probe + selection for every (b, g) of a DecodeInputs."""
    sp = inp.spec
    sm = fp32_scale(sp.D)
    qp = O.to_f64(inp.q_probe, sp.dtype)
    k = O.to_f64(inp.k, sp.dtype)
    return O.probe_select_batch(qp, k, inp.seq_lens, sm, window, keep[0], keep[1])


def selection_tensors(scores, sels, B, Hkv, Tmax, stride):
    """Pack oracle selections into the ABI's device tensors."""
    import torch
    sel = np.full((B, Hkv, stride), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    col = np.zeros((B, Hkv, Tmax), dtype=np.float32)
    thr = np.zeros((B, Hkv, 2), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            s = sels[b][g]
            sel[b, g, : s.k] = s.idx
            cnt[b, g] = s.k
            T = scores[b].shape[1]
            col[b, g, :T] = scores[b][g].astype(np.float32)
            thr[b, g, 0] = np.float32(s.tau).view(np.int32)
            thr[b, g, 1] = s.j_k
    return (torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(), torch.from_numpy(col).cuda(),
            torch.from_numpy(thr).cuda())


def oracle_caches(inp, sels, scores, window):
    """Oracle hybrid caches; the probe scores / threshold the GPU holds are fp32."""
    sp = inp.spec
    k = O.to_f64(inp.k, sp.dtype)
    v = O.to_f64(inp.v, sp.dtype)
    out = []
    for b in range(sp.B):
        T = int(inp.seq_lens[b])
        row = []
        for g in range(sp.Hkv):
            s = sels[b][g]
            c32 = scores[b][g].astype(np.float32).astype(np.float64)
            s32 = O.Selection(s.idx, s.k, float(np.float32(s.tau)), s.j_k)
            row.append(O.build_cache(k[b, g], v[b, g], T, s32, window, c32))
        out.append(row)
    return out


def attn_errors(gpu: np.ndarray, ref: np.ndarray):
    diff = gpu.astype(np.float64) - ref
    return float(np.abs(diff).max()), float(np.linalg.norm(diff) / np.linalg.norm(ref))


def v_scale(caches):
    """sigma_V = max(1, RMS of the dequantized V values seen by attention)
    over a list of oracle caches: the unit in which the max-abs bar is read
    (R20: the kernels' arithmetic errors are proportional to the magnitude of
    V, so the 2e-3 bar, stated for unit-scale values, scales with it)."""
    ss, n = 0.0, 0
    for c in caches:
        _, vh = O.cache_kv_hat(c)
        ss += float((vh * vh).sum())
        n += vh.size
    return max(1.0, math.sqrt(ss / max(n, 1)))


def assert_attn_close(gpu, ref, what="", vscale=1.0):
    """max-abs <= ATOL * vscale and rel-L2 <= RTOL_L2; vscale = 1 for
    unit-scale V (every workload), sigma_V of v_scale() otherwise. Prints the
    unscaled errors."""
    mx, rl2 = attn_errors(gpu, ref)
    print(f"{what}: max-abs {mx:.3e} (bar {ATOL * vscale:.3e}, sigma_V {vscale:.2f}, max|o| "
          f"{float(np.abs(ref).max()):.2f}) rel-L2 {rl2:.3e}", flush=True)
    assert mx <= ATOL * vscale and rl2 <= RTOL_L2, (what, mx, rl2, vscale)
    return mx, rl2
