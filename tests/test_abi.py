"""The C ABI: the shared library loads, exports every function include/hq.h
declares, sizes the cache in closed form, and rejects bad arguments on the
host (before any GPU work) with the documented status codes. CPU only."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kv_cache_amd", "libhyquant.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libhyquant.so not built")


@pytest.fixture(scope="module")
def hq():
    import kv_cache_amd
    return kv_cache_amd


def _declared():
    names = set()
    for h in ("hq.h", "hq_diag.h"):
        with open(os.path.join(ROOT, "include", h)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(hq_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_exports_every_declared_symbol(hq):
    names = _declared()
    assert set(hq.EXPORTED) == set(names), names
    raw = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(raw, n), n


def test_nm_lists_symbols_as_text():
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    for n in _declared():
        assert re.search(rf"\sT\s{n}$", out, re.M), n


def test_cache_layout_closed_form(hq):
    pol = hq.Policy()
    sz = hq.hq_cache_sizes()
    assert hq.lib.hq_cache_layout(16, 8, 128, 32768, 32768, hq.HQ_BF16, ctypes.byref(pol.c()), ctypes.byref(sz)) == 0
    BG = 16 * 8
    assert sz.cap_q == 32768
    assert sz.cap_keep == 1792                     # round64(1638 + 128)
    assert sz.k_codes == BG * 32768 * 64           # 64 B of K codes per token
    assert sz.k_meta == BG * 32768 * 16            # 4 groups x (fp16 s, fp16 z)
    assert sz.k_win == BG * 128 * 256
    # per-token traffic of the decode kernel: 160 B quantized, 512 B 16-bit
    assert (sz.k_codes + sz.v_codes + sz.k_meta + sz.v_meta) // (BG * 32768) == 160
    assert (sz.k_keep + sz.v_keep) // (BG * 1792) == 512


def test_sel_stride(hq):
    pol = hq.Policy()
    assert hq.sel_stride(32768, pol) == 1638
    assert hq.sel_stride(10, pol) == 1


def _null():
    return ctypes.c_void_p(0)


FAKE = ctypes.c_void_p(0x100000)       # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x100004)


def _probe(hq, **kw):
    a = dict(q=FAKE, k=FAKE, lens=FAKE, B=1, Hq=4, Hkv=1, Tmax=256, D=128, dt=hq.HQ_BF16, pol=hq.Policy().c(),
             sm=0.088, col=FAKE, sel=FAKE, cnt=FAKE, thr=FAKE, ws=FAKE, wsb=0)
    a.update(kw)
    return hq.lib.hq_probe_select(a["q"], a["k"], a["lens"], a["B"], a["Hq"], a["Hkv"], a["Tmax"], a["D"],
                                  a["dt"], ctypes.byref(a["pol"]), a["sm"], a["col"], a["sel"], a["cnt"],
                                  a["thr"], a["ws"], a["wsb"], None)


def test_probe_validation(hq):
    assert _probe(hq, q=_null()) == hq.HQ_ERR_INVALID_ARG
    assert "q_probe is null" in hq.lib.hq_last_error().decode()
    assert _probe(hq, k=MISALIGNED) == hq.HQ_ERR_INVALID_ARG
    assert "aligned" in hq.lib.hq_last_error().decode()
    assert _probe(hq, D=64) == hq.HQ_ERR_UNSUPPORTED
    assert _probe(hq, Hq=6, Hkv=4) == hq.HQ_ERR_UNSUPPORTED
    assert _probe(hq, Hq=48, Hkv=3) == hq.HQ_ERR_UNSUPPORTED          # group of 16
    assert _probe(hq, dt=hq.HQ_F32) == hq.HQ_ERR_UNSUPPORTED
    assert _probe(hq, pol=hq.hq_policy(5, 0, 128, 64)) == hq.HQ_ERR_INVALID_ARG
    assert _probe(hq, pol=hq.hq_policy(5, 100, 100, 64)) == hq.HQ_ERR_INVALID_ARG   # window % 64
    assert _probe(hq, pol=hq.hq_policy(101, 100, 128, 64)) == hq.HQ_ERR_INVALID_ARG
    assert _probe(hq, sm=-1.0) == hq.HQ_ERR_INVALID_ARG
    assert _probe(hq, Tmax=0) == hq.HQ_ERR_INVALID_ARG
    assert _probe(hq, wsb=16) == hq.HQ_ERR_CAPACITY                      # workspace too small
    assert "workspace" in hq.lib.hq_last_error().decode()


def _cache(hq, **kw):
    sz = hq.hq_cache_sizes()
    pol = hq.Policy()
    assert hq.lib.hq_cache_layout(1, 1, 128, 1024, 1024, hq.HQ_BF16, ctypes.byref(pol.c()), ctypes.byref(sz)) == 0
    c = hq.hq_cache(B=1, Hkv=1, D=128, window=128, cap_q=sz.cap_q, cap_keep=sz.cap_keep, cap_probe=sz.cap_probe,
                    dt=hq.HQ_BF16)
    for n in hq._CACHE_PTRS:
        setattr(c, n, 0x100000)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_cache_validation(hq):
    q = FAKE
    ws = FAKE
    for bad, code in [(dict(D=64), hq.HQ_ERR_UNSUPPORTED), (dict(k_codes=0), hq.HQ_ERR_INVALID_ARG),
                      (dict(v_meta=0x100008), hq.HQ_ERR_INVALID_ARG), (dict(cap_q=100), hq.HQ_ERR_INVALID_ARG),
                      (dict(window=100), hq.HQ_ERR_INVALID_ARG), (dict(dt=hq.HQ_F32), hq.HQ_ERR_UNSUPPORTED),
                      (dict(cap_probe=5000), hq.HQ_ERR_INVALID_ARG)]:
        c = _cache(hq, **bad)
        assert hq.lib.hq_decode_attn(ctypes.byref(c), q, 4, 0.088, FAKE, hq.HQ_F32, ws, 1 << 30, None) == code, bad
        assert hq.lib.hq_append_kv(ctypes.byref(c), FAKE, FAKE, None) == code, bad
    c = _cache(hq)
    assert hq.lib.hq_decode_attn(ctypes.byref(c), q, 6, 0.088, FAKE, hq.HQ_F32, ws, 1 << 30, None) == hq.HQ_ERR_UNSUPPORTED
    assert hq.lib.hq_decode_attn(ctypes.byref(c), q, 4, 0.088, FAKE, hq.HQ_F32, ws, 16, None) == hq.HQ_ERR_CAPACITY
    assert hq.lib.hq_decode_attn(ctypes.byref(c), _null(), 4, 0.088, FAKE, hq.HQ_F32, ws, 1 << 30, None) == hq.HQ_ERR_INVALID_ARG
    assert hq.lib.hq_append_kv(ctypes.byref(c), FAKE, _null(), None) == hq.HQ_ERR_INVALID_ARG
    assert hq.lib.hq_append_kv(None, FAKE, FAKE, None) == hq.HQ_ERR_INVALID_ARG
    # quantize: Tmax beyond the probe capacity, policy/window mismatch
    pol = hq.Policy().c()
    assert hq.lib.hq_quantize_kv(FAKE, FAKE, FAKE, 4096, FAKE, FAKE, FAKE, FAKE, ctypes.byref(pol),
                                 ctypes.byref(c), None) == hq.HQ_ERR_CAPACITY
    pol2 = hq.hq_policy(5, 100, 64, 64)
    assert hq.lib.hq_quantize_kv(FAKE, FAKE, FAKE, 512, FAKE, FAKE, FAKE, FAKE, ctypes.byref(pol2),
                                 ctypes.byref(c), None) == hq.HQ_ERR_INVALID_ARG


def test_prefill_validation(hq):
    pol = hq.Policy().c()

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, B=1, Hq=32, Hkv=8, T=1024, D=128, dt=hq.HQ_BF16, sel=FAKE, cnt=FAKE,
                 sm=0.088, out=FAKE, odt=hq.HQ_F32, ws=FAKE, wsb=0)
        a.update(kw)
        return hq.lib.hq_prefill_attn(a["q"], a["k"], a["v"], a["B"], a["Hq"], a["Hkv"], a["T"], a["D"], a["dt"],
                                      ctypes.byref(pol), a["sel"], a["cnt"], a["sm"], a["out"], a["odt"], a["ws"],
                                      a["wsb"], None)
    assert call(v=_null()) == hq.HQ_ERR_INVALID_ARG
    assert call(D=256) == hq.HQ_ERR_UNSUPPORTED
    assert call(odt=7) == hq.HQ_ERR_UNSUPPORTED
    assert call(T=0) == hq.HQ_ERR_INVALID_ARG
    assert call(wsb=1) == hq.HQ_ERR_CAPACITY


def test_layout_rejects_bad_sizes(hq):
    sz = hq.hq_cache_sizes()
    pol = hq.Policy().c()
    assert hq.lib.hq_cache_layout(1, 1, 128, 100, 200, hq.HQ_BF16, ctypes.byref(pol), ctypes.byref(sz)) == hq.HQ_ERR_INVALID_ARG
    assert hq.lib.hq_cache_layout(1, 1, 96, 100, 100, hq.HQ_BF16, ctypes.byref(pol), ctypes.byref(sz)) == hq.HQ_ERR_UNSUPPORTED
    assert hq.lib.hq_cache_layout(1, 1, 128, 100, 100, hq.HQ_BF16, ctypes.byref(pol), None) == hq.HQ_ERR_INVALID_ARG
