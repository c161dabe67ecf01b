"""kv_cache_amd: HyQuant-style hybrid-precision attention for MI355X.

A thin ctypes binding over libhyquant.so (include/hq.h). It only marshals
arguments: torch supplies device memory and the current HIP stream, and every
step of the computation runs in the library's HIP kernels. There is no CPU
fallback: importing this package without the built library raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhyquant.so")

HQ_OK, HQ_ERR_INVALID_ARG, HQ_ERR_UNSUPPORTED, HQ_ERR_CAPACITY, HQ_ERR_HIP = 0, -1, -2, -3, -4
HQ_F16, HQ_BF16, HQ_F32 = 0, 1, 2
HQ_LOW_INT8, HQ_LOW_FP8 = 0, 1

EXPORTED = (
    "hq_probe_select", "hq_probe_ws_bytes", "hq_quantize_kv", "hq_append_kv", "hq_decode_attn",
    "hq_decode_ws_bytes", "hq_decode_attn_noalloc", "hq_prefill_attn", "hq_prefill_ws_bytes", "hq_cache_layout", "hq_sel_stride",
    "hq_last_error", "hq_diag_read_int4", "hq_diag_read_int4_sink_bytes", "hq_reprobe", "hq_reprobe_ws_bytes",
    "hq_cache_layout_ragged", "hq_diag_exp2_error",
)


class HQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class hq_policy(ctypes.Structure):
    _fields_ = [("keep_num", ctypes.c_int32), ("keep_den", ctypes.c_int32),
                ("window", ctypes.c_int32), ("probe_rows", ctypes.c_int32), ("low_fmt", ctypes.c_int32),
                ("tile_num", ctypes.c_int32), ("tile_den", ctypes.c_int32)]


class hq_thresh(ctypes.Structure):
    _fields_ = [("tau", ctypes.c_float), ("j_k", ctypes.c_int32)]


_CACHE_PTRS = ("k_codes", "v_codes", "k_meta", "v_meta", "k_keep", "v_keep", "k_win", "v_win",
               "q_pos", "keep_pos", "counts", "col_scores", "thresh", "err_flag")


class hq_cache(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int32) for n in ("B", "Hkv", "D", "window", "cap_q", "cap_keep", "cap_probe", "dt")]
                + [(n, ctypes.c_void_p) for n in _CACHE_PTRS]
                + [("q_tile_off", ctypes.c_void_p), ("q_tiles_total", ctypes.c_int64)])


class hq_cache_sizes(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int32) for n in ("cap_q", "cap_keep", "cap_probe")]
                + [(n, ctypes.c_size_t) for n in _CACHE_PTRS])


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python kv_cache_amd/build.py`")
    # torch first: the library then binds to the HIP runtime torch has
    # loaded, so both see the same devices, memory and streams (loaded the
    # other way round, the library's calls find no device).
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, S, V = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
    pol = ctypes.POINTER(hq_policy)
    sig = {
        "hq_probe_select": (I, [P, P, P, I, I, I, I, I, I, pol, F, P, P, P, P, P, S, V]),
        "hq_probe_ws_bytes": (S, [I, I, I, I, I, pol]),
        "hq_quantize_kv": (I, [P, P, P, I, P, P, P, P, pol, ctypes.POINTER(hq_cache), V]),
        "hq_append_kv": (I, [ctypes.POINTER(hq_cache), P, P, V]),
        "hq_decode_attn": (I, [ctypes.POINTER(hq_cache), P, I, F, P, I, P, S, V]),
        "hq_decode_ws_bytes": (S, [ctypes.POINTER(hq_cache), I]),
        "hq_decode_attn_noalloc": (I, [ctypes.POINTER(hq_cache), P, I, F, P, I, V]),
        "hq_prefill_attn": (I, [P, P, P, I, I, I, I, I, I, pol, P, P, F, P, I, P, S, V]),
        "hq_prefill_ws_bytes": (S, [I, I, I, I, I, pol]),
        "hq_cache_layout": (I, [I, I, I, I, I, I, pol, ctypes.POINTER(hq_cache_sizes)]),
        "hq_cache_layout_ragged": (I, [I, I, I, ctypes.POINTER(ctypes.c_int32), I, I, pol,
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(hq_cache_sizes)]),
        "hq_sel_stride": (I, [I, pol]),
        "hq_last_error": (ctypes.c_char_p, []),
        "hq_diag_read_int4": (I, [ctypes.POINTER(hq_cache), P, S, V]),
        "hq_diag_read_int4_sink_bytes": (S, [ctypes.POINTER(hq_cache)]),
        "hq_diag_exp2_error": (I, [F, F, P, S, V]),
        "hq_reprobe": (I, [ctypes.POINTER(hq_cache), P, I, pol, F, P, P, P, P, P, P, S, V]),
        "hq_reprobe_ws_bytes": (S, [ctypes.POINTER(hq_cache), I, pol]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(status: int):
    if status != HQ_OK:
        raise HQError(status, lib.hq_last_error().decode())


# ---------------------------------------------------------------------------
# torch-facing helpers (argument marshalling only)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Policy:
    keep_num: int = 5
    keep_den: int = 100
    window: int = 128
    probe_rows: int = 64
    low_fmt: int = HQ_LOW_INT8   # prefill's low-precision path (HQ_LOW_INT8 / HQ_LOW_FP8)
    tile_num: int = 0            # prefill tile routing fraction (0 = off)
    tile_den: int = 100

    def c(self) -> hq_policy:
        return hq_policy(self.keep_num, self.keep_den, self.window, self.probe_rows, self.low_fmt,
                         self.tile_num, self.tile_den)


def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return HQ_BF16
    if t.dtype == torch.float16:
        return HQ_F16
    if t.dtype == torch.float32:
        return HQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def sel_stride(T: int, policy: Policy = Policy()) -> int:
    return int(lib.hq_sel_stride(T, ctypes.byref(policy.c())))


def probe_select(q_probe, k, seq_lens, policy: Policy = Policy(), sm_scale: float | None = None):
    """hq_probe_select. q_probe [B][Hq][R][D], k [B][Hkv][Tmax][D] (bf16/f16),
    seq_lens [B] int32. Returns (col_scores f32 [B][Hkv][Tmax], sel_idx int32
    [B][Hkv][stride], sel_count int32 [B][Hkv], thresh int32 [B][Hkv][2])."""
    torch = _torch()
    _need_contig(q_probe, k, seq_lens)
    B, Hq, R, D = q_probe.shape
    _, Hkv, Tmax, _ = k.shape
    if R != policy.probe_rows:
        raise ValueError("q_probe rows must equal policy.probe_rows")
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    dev = k.device
    stride = sel_stride(Tmax, policy)
    col = torch.empty((B, Hkv, Tmax), dtype=torch.float32, device=dev)
    sel = torch.empty((B, Hkv, stride), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    thr = torch.empty((B, Hkv, 2), dtype=torch.int32, device=dev)
    pc = policy.c()
    nws = lib.hq_probe_ws_bytes(B, Hq, Hkv, Tmax, D, ctypes.byref(pc))
    ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
    _check(lib.hq_probe_select(_ptr(q_probe), _ptr(k), _ptr(seq_lens), B, Hq, Hkv, Tmax, D, _dt(k),
                               ctypes.byref(pc), sm, _ptr(col), _ptr(sel), _ptr(cnt), _ptr(thr), _ptr(ws),
                               ws.numel(), _stream()))
    return col, sel, cnt, thr


class HybridCache:
    """Caller-owned buffers of the hybrid KV cache (hq_cache). cap_tokens is
    one capacity for every sequence (the uniform layout) or a list of B
    capacities (the ragged INT4 layout of hq_cache_layout_ragged)."""

    def __init__(self, B: int, Hkv: int, cap_tokens, cap_probe: int, dtype, device,
                 policy: Policy = Policy(), D: int = 128):
        torch = _torch()
        self.policy = policy
        dt = HQ_BF16 if dtype == torch.bfloat16 else HQ_F16 if dtype == torch.float16 else None
        if dt is None:
            raise TypeError("cache dtype must be bf16 or fp16")
        sz = hq_cache_sizes()
        ragged = not isinstance(cap_tokens, int)
        if ragged:
            caps = (ctypes.c_int32 * B)(*[int(x) for x in cap_tokens])
            offs = (ctypes.c_int64 * (B * Hkv + 1))()
            _check(lib.hq_cache_layout_ragged(B, Hkv, D, caps, cap_probe, dt, ctypes.byref(policy.c()), offs,
                                              ctypes.byref(sz)))
            self.q_tile_off = list(offs)
        else:
            _check(lib.hq_cache_layout(B, Hkv, D, cap_tokens, cap_probe, dt, ctypes.byref(policy.c()),
                                       ctypes.byref(sz)))
            self.q_tile_off = None
        self.sizes = sz
        self.bufs = {}
        c = hq_cache(B=B, Hkv=Hkv, D=D, window=policy.window, cap_q=sz.cap_q, cap_keep=sz.cap_keep,
                     cap_probe=sz.cap_probe, dt=dt)
        for name in _CACHE_PTRS:
            nbytes = max(int(getattr(sz, name)), 256)
            t = torch.zeros(nbytes, dtype=torch.uint8, device=device)
            self.bufs[name] = t
            setattr(c, name, t.data_ptr())
        if ragged:
            t = torch.tensor(self.q_tile_off, dtype=torch.int64, device=device)
            self.bufs["q_tile_off"] = t
            c.q_tile_off = t.data_ptr()
            c.q_tiles_total = self.q_tile_off[-1]
        self.c = c
        self.B, self.Hkv, self.D, self.dtype, self.device = B, Hkv, D, dtype, device
        self._ws = None

    # canonical read-back helpers (device tensors; no computation)
    def counts(self):
        torch = _torch()
        return self.bufs["counts"][: self.B * self.Hkv * 16].view(torch.int32).view(self.B, self.Hkv, 4)

    def err_flag(self) -> int:
        torch = _torch()
        return int(self.bufs["err_flag"][:4].view(torch.int32)[0].item())

    def ptr(self):
        return ctypes.byref(self.c)


def quantize_kv(cache: HybridCache, k, v, seq_lens, sel_idx, sel_count, col_scores, thresh):
    _need_contig(k, v, seq_lens, sel_idx, sel_count, col_scores, thresh)
    Tmax = k.shape[2]
    _check(lib.hq_quantize_kv(_ptr(k), _ptr(v), _ptr(seq_lens), Tmax, _ptr(sel_idx), _ptr(sel_count),
                              _ptr(col_scores), _ptr(thresh), ctypes.byref(cache.policy.c()), cache.ptr(),
                              _stream()))


def append_kv(cache: HybridCache, k_new, v_new):
    _need_contig(k_new, v_new)
    _check(lib.hq_append_kv(cache.ptr(), _ptr(k_new), _ptr(v_new), _stream()))


def decode_ws(cache: HybridCache, Hq: int):
    torch = _torch()
    n = lib.hq_decode_ws_bytes(cache.ptr(), Hq)
    if cache._ws is None or cache._ws.numel() < n:
        cache._ws = torch.empty(max(n, 256), dtype=torch.uint8, device=cache.device)
    return cache._ws


def decode_attn(cache: HybridCache, q, sm_scale: float | None = None, out=None, out_dtype=None):
    """hq_decode_attn. q [B][Hq][D] in the cache dtype; returns out [B][Hq][D]."""
    torch = _torch()
    _need_contig(q)
    B, Hq, D = q.shape
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or torch.float32, device=q.device)
    ws = decode_ws(cache, Hq)
    _check(lib.hq_decode_attn(cache.ptr(), _ptr(q), Hq, sm, _ptr(out), _dt(out), _ptr(ws), ws.numel(),
                              _stream()))
    return out


def decode_attn_noalloc(cache: HybridCache, q, sm_scale: float | None = None, out=None, out_dtype=None):
    """hq_decode_attn_noalloc: as decode_attn, with the split partials in the
    library's static scratch array (no workspace). q [B][Hq][D]; returns out."""
    torch = _torch()
    _need_contig(q)
    B, Hq, D = q.shape
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    if out is None:
        out = torch.empty((B, Hq, D), dtype=out_dtype or torch.float32, device=q.device)
    _check(lib.hq_decode_attn_noalloc(cache.ptr(), _ptr(q), Hq, sm, _ptr(out), _dt(out), _stream()))
    return out


def reprobe_tcap(cache: HybridCache) -> int:
    """Position stride of hq_reprobe's outputs: cap_q + cap_keep + window."""
    return int(cache.c.cap_q + cache.c.cap_keep + cache.c.window)


def reprobe(cache: HybridCache, q_recent, sm_scale: float | None = None, policy: Policy | None = None, ws=None):
    """hq_reprobe. q_recent [B][Hq][R][D] in the cache dtype (R = policy.probe_rows).
    Returns (col_scores f32 [B][Hkv][Tcap], sel_idx int32 [B][Hkv][stride],
    sel_count int32 [B][Hkv], thresh int32 [B][Hkv][2], n_persist int32 [B][Hkv],
    ws uint8; its first B*Hkv*Tcap*D*2 bytes are the expanded keys)."""
    torch = _torch()
    _need_contig(q_recent)
    B, Hq, R, D = q_recent.shape
    policy = policy or cache.policy
    if R != policy.probe_rows:
        raise ValueError("q_recent rows must equal policy.probe_rows")
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    dev = q_recent.device
    tcap = reprobe_tcap(cache)
    stride = sel_stride(tcap, policy)
    col = torch.empty((B, cache.Hkv, tcap), dtype=torch.float32, device=dev)
    sel = torch.empty((B, cache.Hkv, stride), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, cache.Hkv), dtype=torch.int32, device=dev)
    thr = torch.empty((B, cache.Hkv, 2), dtype=torch.int32, device=dev)
    npers = torch.empty((B, cache.Hkv), dtype=torch.int32, device=dev)
    pc = policy.c()
    n = lib.hq_reprobe_ws_bytes(cache.ptr(), Hq, ctypes.byref(pc))
    if ws is None or ws.numel() < n:
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    _check(lib.hq_reprobe(cache.ptr(), _ptr(q_recent), Hq, ctypes.byref(pc), sm, _ptr(col), _ptr(sel), _ptr(cnt),
                          _ptr(thr), _ptr(npers), _ptr(ws), ws.numel(), _stream()))
    return col, sel, cnt, thr, npers, ws


def diag_read_int4(cache: HybridCache, sink=None):
    """hq_diag_read_int4 (measurement helper): streams the cache's INT4 store
    in the decode kernel's access pattern; returns the sink tensor."""
    torch = _torch()
    n = lib.hq_diag_read_int4_sink_bytes(cache.ptr())
    if sink is None or sink.numel() < n:
        sink = torch.empty(max(n, 256), dtype=torch.uint8, device=cache.device)
    _check(lib.hq_diag_read_int4(cache.ptr(), _ptr(sink), sink.numel(), _stream()))
    return sink


def diag_exp2_error(lo: float = -0.5, hi: float = 0.5, nblocks: int = 4096) -> float:
    """hq_diag_exp2_error (measurement helper): the largest relative error of
    the hardware base-2 exponential over every fp32 input in [lo, hi]."""
    torch = _torch()
    out = torch.zeros(nblocks, dtype=torch.float64, device="cuda")
    _check(lib.hq_diag_exp2_error(lo, hi, _ptr(out), nblocks, _stream()))
    return float(out.max().item())


def prefill_attn(q, k, v, sel_idx, sel_count, policy: Policy = Policy(), sm_scale: float | None = None,
                 out=None, out_dtype=None, ws=None):
    """hq_prefill_attn. q [B][Hq][T][D], k/v [B][Hkv][T][D]; returns out [B][Hq][T][D]."""
    torch = _torch()
    _need_contig(q, k, v, sel_idx, sel_count)
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    sm = 1.0 / math.sqrt(D) if sm_scale is None else sm_scale
    if out is None:
        out = torch.empty((B, Hq, T, D), dtype=out_dtype or torch.float32, device=q.device)
    pc = policy.c()
    n = lib.hq_prefill_ws_bytes(B, Hq, Hkv, T, D, ctypes.byref(pc))
    if ws is None or ws.numel() < n:
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    _check(lib.hq_prefill_attn(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, T, D, _dt(q), ctypes.byref(pc),
                               _ptr(sel_idx), _ptr(sel_count), sm, _ptr(out), _dt(out), _ptr(ws), ws.numel(),
                               _stream()))
    return out
