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
    assert sz.cap_q == 32768 - 128                 # every position outside the window
    assert sz.cap_keep == 1792                     # round64(1638 + 128): selected + flagged departures
    assert sz.k_codes == BG * sz.cap_q * 64        # 64 B of K codes per token
    assert sz.k_meta == BG * sz.cap_q * 16         # 4 groups x (fp16 s, fp16 z)
    assert sz.k_win == BG * 128 * 256
    # per-token traffic of the decode kernel: 160 B quantized, 512 B 16-bit
    assert (sz.k_codes + sz.v_codes + sz.k_meta + sz.v_meta) // (BG * sz.cap_q) == 160
    assert (sz.k_keep + sz.v_keep) // (BG * 1792) == 512
    # a context shorter than the window: the INT4 store keeps its minimum tile
    assert hq.lib.hq_cache_layout(1, 1, 128, 100, 100, hq.HQ_BF16, ctypes.byref(pol.c()), ctypes.byref(sz)) == 0
    assert sz.cap_q == 64 and sz.cap_keep == 128
    # capacities are bounded by the 32-bit byte offsets of the INT4 store
    assert hq.lib.hq_cache_layout(1, 1, 128, (1 << 24) + 1, 1000, hq.HQ_BF16, ctypes.byref(pol.c()),
                                  ctypes.byref(sz)) == hq.HQ_ERR_CAPACITY
    assert "2^24" in hq.lib.hq_last_error().decode() or "16777216" in hq.lib.hq_last_error().decode()


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
    assert _probe(hq, pol=hq.hq_policy(5, 100, 128, 64, 2)) == hq.HQ_ERR_UNSUPPORTED     # low_fmt
    assert _probe(hq, sm=-1.0) == hq.HQ_ERR_INVALID_ARG
    assert _probe(hq, Tmax=0) == hq.HQ_ERR_INVALID_ARG
    assert _probe(hq, wsb=16) == hq.HQ_ERR_CAPACITY                      # workspace too small
    assert "workspace" in hq.lib.hq_last_error().decode()
    # probe shapes: G x probe_rows a multiple of 16, at most 512
    assert _probe(hq, pol=hq.hq_policy(5, 100, 128, 10)) == hq.HQ_ERR_UNSUPPORTED   # 4 x 10 = 40
    assert "multiple of 16" in hq.lib.hq_last_error().decode()
    assert _probe(hq, Hq=8, pol=hq.hq_policy(5, 100, 128, 128)) == hq.HQ_ERR_UNSUPPORTED   # 8 x 128 = 1024
    assert "at most 512" in hq.lib.hq_last_error().decode()
    assert hq.lib.hq_probe_ws_bytes(1, 4, 1, 256, 128, ctypes.byref(hq.hq_policy(5, 100, 128, 10))) == 0
    assert _probe(hq, pol=hq.hq_policy(5, 100, 128, 4), wsb=16) == hq.HQ_ERR_CAPACITY  # 4 x 4 = 16 is accepted


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
                      (dict(cap_probe=5000), hq.HQ_ERR_INVALID_ARG),
                      (dict(cap_q=1 << 25), hq.HQ_ERR_CAPACITY), (dict(cap_keep=1 << 25), hq.HQ_ERR_CAPACITY)]:
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
    # tile routing: a valid fraction, the INT8 path, T <= 2^18
    for bad, code in [(hq.hq_policy(5, 100, 128, 64, 0, 5, 0), hq.HQ_ERR_INVALID_ARG),
                      (hq.hq_policy(5, 100, 128, 64, 0, 7, 5), hq.HQ_ERR_INVALID_ARG),
                      (hq.hq_policy(5, 100, 128, 64, 1, 5, 100), hq.HQ_ERR_UNSUPPORTED)]:
        assert hq.lib.hq_prefill_attn(FAKE, FAKE, FAKE, 1, 32, 8, 1024, 128, hq.HQ_BF16, ctypes.byref(bad), FAKE,
                                      FAKE, 0.088, FAKE, hq.HQ_F32, FAKE, 1 << 40, None) == code
    tp = hq.hq_policy(5, 100, 128, 64, 0, 5, 100)
    assert hq.lib.hq_prefill_attn(FAKE, FAKE, FAKE, 1, 32, 8, (1 << 18) + 1, 128, hq.HQ_BF16, ctypes.byref(tp), FAKE,
                                  FAKE, 0.088, FAKE, hq.HQ_F32, FAKE, 1 << 40, None) == hq.HQ_ERR_UNSUPPORTED


def test_layout_rejects_bad_sizes(hq):
    sz = hq.hq_cache_sizes()
    pol = hq.Policy().c()
    assert hq.lib.hq_cache_layout(1, 1, 128, 100, 200, hq.HQ_BF16, ctypes.byref(pol), ctypes.byref(sz)) == hq.HQ_ERR_INVALID_ARG
    assert hq.lib.hq_cache_layout(1, 1, 96, 100, 100, hq.HQ_BF16, ctypes.byref(pol), ctypes.byref(sz)) == hq.HQ_ERR_UNSUPPORTED
    assert hq.lib.hq_cache_layout(1, 1, 128, 100, 100, hq.HQ_BF16, ctypes.byref(pol), None) == hq.HQ_ERR_INVALID_ARG


def test_decode_noalloc_validation(hq):
    """hq_decode_attn_noalloc validates like hq_decode_attn on the host, and
    rejects a cache whose split partials exceed the static scratch."""
    c = _cache(hq)
    q = FAKE
    assert hq.lib.hq_decode_attn_noalloc(ctypes.byref(c), _null(), 4, 0.088, FAKE, hq.HQ_F32, None) == \
        hq.HQ_ERR_INVALID_ARG
    assert hq.lib.hq_decode_attn_noalloc(ctypes.byref(c), q, 6, 0.088, FAKE, hq.HQ_F32, None) == hq.HQ_ERR_UNSUPPORTED
    assert hq.lib.hq_decode_attn_noalloc(None, q, 4, 0.088, FAKE, hq.HQ_F32, None) == hq.HQ_ERR_INVALID_ARG
    bad = _cache(hq, k_codes=0)
    assert hq.lib.hq_decode_attn_noalloc(ctypes.byref(bad), q, 4, 0.088, FAKE, hq.HQ_F32, None) == \
        hq.HQ_ERR_INVALID_ARG
    # a cache far beyond the scratch: 64 x 64 (b, g) of 1M tokens, 8 query heads each
    sz = hq.hq_cache_sizes()
    pol = hq.Policy()
    assert hq.lib.hq_cache_layout(64, 64, 128, 1 << 20, 1 << 20, hq.HQ_BF16, ctypes.byref(pol.c()),
                                  ctypes.byref(sz)) == 0
    big = hq.hq_cache(B=64, Hkv=64, D=128, window=128, cap_q=sz.cap_q, cap_keep=sz.cap_keep, cap_probe=sz.cap_probe,
                      dt=hq.HQ_BF16)
    for n in hq._CACHE_PTRS:
        setattr(big, n, 0x100000)
    need = hq.lib.hq_decode_ws_bytes(ctypes.byref(big), 512)
    assert need > (16 << 20)
    assert hq.lib.hq_decode_attn_noalloc(ctypes.byref(big), q, 512, 0.088, FAKE, hq.HQ_F32, None) == \
        hq.HQ_ERR_CAPACITY
    assert "static scratch" in hq.lib.hq_last_error().decode()
    # the workspace entry point still requires its workspace
    assert hq.lib.hq_decode_attn(ctypes.byref(c), q, 4, 0.088, FAKE, hq.HQ_F32, None, 1 << 30, None) == \
        hq.HQ_ERR_INVALID_ARG


def test_diag_exp2_error_validation(hq):
    """hq_diag_exp2_error rejects an empty or out-of-limit range, a NaN bound,
    a bad workgroup count and a null output on the host."""
    d = FAKE
    f = hq.lib.hq_diag_exp2_error
    assert f(0.5, -0.5, d, 16, None) == hq.HQ_ERR_INVALID_ARG
    assert f(-65.0, 0.0, d, 16, None) == hq.HQ_ERR_INVALID_ARG
    assert f(0.0, 64.5, d, 16, None) == hq.HQ_ERR_INVALID_ARG
    assert f(float("nan"), 0.5, d, 16, None) == hq.HQ_ERR_INVALID_ARG
    assert f(-0.5, 0.5, d, 0, None) == hq.HQ_ERR_INVALID_ARG
    assert f(-0.5, 0.5, d, 65537, None) == hq.HQ_ERR_INVALID_ARG
    assert f(-0.5, 0.5, None, 16, None) == hq.HQ_ERR_INVALID_ARG
    assert "hq_diag_exp2_error" in hq.lib.hq_last_error().decode()


def test_reprobe_validation(hq):
    """hq_reprobe checks the cache, the policy against it, the probe's shape
    rule, the workspace and its alignment before anything is launched."""
    c = _cache(hq)
    pol = hq.Policy().c()
    need = hq.lib.hq_reprobe_ws_bytes(ctypes.byref(c), 4, ctypes.byref(pol))
    tcap = c.cap_q + c.cap_keep + c.window
    assert need >= tcap * 128 * 2 + tcap

    def call(cache=c, Hq=4, p=pol, sm=0.088, ws=FAKE, wsb=None, **ptrs):
        a = dict(q=FAKE, col=FAKE, sel=FAKE, cnt=FAKE, thr=FAKE, npers=FAKE)
        a.update(ptrs)
        return hq.lib.hq_reprobe(ctypes.byref(cache) if cache is not None else None, a["q"], Hq, ctypes.byref(p), sm,
                                 a["col"], a["sel"], a["cnt"], a["thr"], a["npers"], ws,
                                 need if wsb is None else wsb, None)
    assert call(cache=None) == hq.HQ_ERR_INVALID_ARG
    assert call(cache=_cache(hq, k_codes=0)) == hq.HQ_ERR_INVALID_ARG
    assert call(Hq=6) == hq.HQ_ERR_UNSUPPORTED
    assert call(p=hq.hq_policy(5, 100, 64, 64)) == hq.HQ_ERR_INVALID_ARG          # window != cache window
    assert call(p=hq.hq_policy(5, 100, 128, 10)) == hq.HQ_ERR_UNSUPPORTED         # 4 x 10 rows
    assert call(sm=0.0) == hq.HQ_ERR_INVALID_ARG
    assert call(npers=_null()) == hq.HQ_ERR_INVALID_ARG
    assert call(q=_null()) == hq.HQ_ERR_INVALID_ARG
    assert call(ws=ctypes.c_void_p(0x100010)) == hq.HQ_ERR_INVALID_ARG            # not 256-byte aligned
    assert call(wsb=need - 1) == hq.HQ_ERR_CAPACITY
    big = _cache(hq, cap_q=(1 << 24) - 64, cap_keep=128)
    assert call(cache=big) == hq.HQ_ERR_CAPACITY
    assert hq.lib.hq_reprobe_ws_bytes(ctypes.byref(big), 4, ctypes.byref(pol)) == 0


def test_cache_layout_ragged_closed_form(hq):
    """Per-sequence INT4 capacities round64(cap - min(W, cap)) (at least 64),
    packed back to back in (b, g) order; every other buffer as the uniform
    layout of the longest sequence; equal capacities give the uniform sizes."""
    pol = hq.Policy()
    caps = [700, 3000, 129, 64]
    B, Hkv = len(caps), 3
    c_caps = (ctypes.c_int32 * B)(*caps)
    offs = (ctypes.c_int64 * (B * Hkv + 1))()
    rg, un = hq.hq_cache_sizes(), hq.hq_cache_sizes()
    assert hq.lib.hq_cache_layout_ragged(B, Hkv, 128, c_caps, 2000, hq.HQ_BF16, ctypes.byref(pol.c()), offs,
                                         ctypes.byref(rg)) == 0
    assert hq.lib.hq_cache_layout(B, Hkv, 128, 3000, 2000, hq.HQ_BF16, ctypes.byref(pol.c()), ctypes.byref(un)) == 0
    tiles = [max(64, -(-(cap - min(128, cap)) // 64) * 64) // 64 for cap in caps]
    assert tiles == [9, 45, 1, 1]
    expect = [0]
    for b in range(B):
        for _ in range(Hkv):
            expect.append(expect[-1] + tiles[b])
    assert list(offs) == expect
    total = expect[-1]
    assert rg.k_codes == rg.v_codes == total * 4096 and rg.k_meta == rg.v_meta == total * 1024
    assert rg.q_pos == total * 64 * 4
    assert rg.cap_q == un.cap_q == 45 * 64
    for n in ("k_keep", "v_keep", "k_win", "v_win", "keep_pos", "counts", "col_scores", "thresh", "err_flag"):
        assert getattr(rg, n) == getattr(un, n), n
    assert rg.k_codes < un.k_codes
    same = (ctypes.c_int32 * B)(*([3000] * B))
    assert hq.lib.hq_cache_layout_ragged(B, Hkv, 128, same, 2000, hq.HQ_BF16, ctypes.byref(pol.c()), offs,
                                         ctypes.byref(rg)) == 0
    for n in hq._CACHE_PTRS:
        assert getattr(rg, n) == getattr(un, n), n
    bad = (ctypes.c_int32 * B)(700, 0, 129, 64)
    assert hq.lib.hq_cache_layout_ragged(B, Hkv, 128, bad, 2000, hq.HQ_BF16, ctypes.byref(pol.c()), offs,
                                         ctypes.byref(rg)) == hq.HQ_ERR_INVALID_ARG
    c = _cache(hq, q_tile_off=0x100000, q_tiles_total=0)
    assert hq.lib.hq_append_kv(ctypes.byref(c), FAKE, FAKE, None) == hq.HQ_ERR_INVALID_ARG


def test_host_layer_under_address_and_undefined_sanitizers(tmp_path):
    """The library's sources and tests/abi_host_check.cpp built with
    AddressSanitizer and UndefinedBehaviorSanitizer on the host side (device
    code is compiled as usual and never run), then run with every device
    hidden: size and layout queries and every validation path, on bad and
    edge arguments, must finish with no sanitizer report."""
    import glob
    import shutil
    import subprocess
    from concurrent.futures import ThreadPoolExecutor
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    base = [hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-fno-omit-frame-pointer",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + san
    srcs = sorted(glob.glob(os.path.join(ROOT, "kv_cache_amd", "csrc", "*.hip")))
    srcs.append(os.path.join(ROOT, "tests", "abi_host_check.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run(base + ["-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return obj
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "abi_host_check")
    r = subprocess.run([hipcc, "--offload-arch=gfx950"] + san + objs + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host checks passed" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-2000:]
