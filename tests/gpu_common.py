"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the oracle on the same inputs, compare within the stated bars."""
import math

import numpy as np

import oracle as O

ATOL = 2e-3      # max-abs bar for attention outputs
RTOL_L2 = 1e-3   # relative-L2 bar for attention outputs


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
    sm = 1 / math.sqrt(sp.D)
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


def assert_attn_close(gpu, ref, what=""):
    mx, rl2 = attn_errors(gpu, ref)
    print(f"{what}: max-abs {mx:.3e} rel-L2 {rl2:.3e}", flush=True)
    assert mx <= ATOL and rl2 <= RTOL_L2, (what, mx, rl2)
    return mx, rl2
