"""Pins for the oracle's quantizers (INT4 cache format, INT8 prefill blocks).

Every check here fixes the oracle against something other than itself:
the error bound that follows from the definition, brute force over all
candidate codes, special cases, and an exhaustive integer-arithmetic proof of
the two-step fp32/fp16 scale rounding.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle as O
from synth import bf16_bits_from_f32, f16_bits_from_f32

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _data(seed, n=4096, outliers=True, dtype="bf16"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128), dtype=np.float32)
    if outliers:
        x[:, [3, 40, 77, 100]] *= 20
    bits = bf16_bits_from_f32(x) if dtype == "bf16" else f16_bits_from_f32(x)
    return O.to_f64(bits, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_int4_error_bound(dtype):
    """|x - x_hat| <= s/2 elementwise (s in fp16's normal range)."""
    x = _data(1, dtype=dtype)
    codes, s, z = O.int4_quantize(x)
    xh = O.int4_dequantize(codes, s, z)
    sb = np.repeat(s.astype(np.float64), 32, axis=-1)
    assert np.all(s.astype(np.float64) >= 2.0 ** -14)
    assert np.all(np.abs(x - xh) <= sb / 2)
    # zero point is the exact group minimum for these inputs
    assert np.array_equal(z.astype(np.float64), x.reshape(-1, 4, 32).min(-1))


def test_int4_codes_are_nearest_grid_point_brute_force():
    """code = argmin_c |x - (c*s + z)| over the 16 candidates, ties to even."""
    x = _data(2, n=512)
    codes, s, z = O.int4_quantize(x)
    g = x.reshape(-1, 4, 32)
    cand = np.arange(16, dtype=np.float64)
    grid = cand[None, None, :] * s.astype(np.float64)[..., None] + z.astype(np.float64)[..., None]
    err = np.abs(g[..., :, None] - grid[..., None, :])          # [n][4][32][16]
    best = err.min(-1, keepdims=True)
    is_best = err == best
    # among equally near candidates pick the even one (round half to even)
    even_pref = np.where(is_best & (cand % 2 == 0), cand, np.where(is_best, cand + 100, 1000))
    ref = even_pref.min(-1)
    ref = np.where(ref >= 100, ref - 100, ref).astype(np.uint8)
    assert np.array_equal(codes.reshape(-1, 4, 32), ref)


def test_int4_constant_group():
    x = np.full((3, 128), 0.75)
    x[1] = -2.5
    codes, s, z = O.int4_quantize(x)
    assert np.all(s == 0) and np.all(codes == 0)
    assert np.array_equal(O.int4_dequantize(codes, s, z), x)


def test_int4_known_group():
    """Hand-worked group: values 0..15 step 0.5 around -3 -> s = 0.5, z = -3."""
    x = np.zeros((1, 128))
    x[0, :32] = -3.0 + 0.5 * (np.arange(32) % 16)
    x[0, 32:] = 1.0
    codes, s, z = O.int4_quantize(x)
    assert float(s[0, 0]) == 0.5 and float(z[0, 0]) == -3.0
    assert list(codes[0, :32]) == list(np.arange(32) % 16)
    # exact half-way case: x = z + 7.5 s rounds to even code 8; 6.5 s -> 6
    y = np.ones((1, 128))
    y[0, 0], y[0, 1], y[0, 2], y[0, 3] = 0.0, 15.0, 7.5, 6.5
    c2, s2, z2 = O.int4_quantize(y)
    assert float(s2[0, 0]) == 1.0 and float(z2[0, 0]) == 0.0
    assert c2[0, 2] == 8 and c2[0, 3] == 6


def test_int4_pack_layout():
    codes = np.array([[1, 2, 3, 4, 15, 0, 9, 10]], dtype=np.uint8)
    packed = O.int4_pack(codes)
    assert list(packed[0]) == [0x21, 0x43, 0x0F, 0xA9]
    assert np.array_equal(O.int4_unpack(packed), codes)


def _scale_tool(tmp_path):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    exe = os.path.join(ROOT, "oracle", "scale_exhaustive")
    if not os.path.exists(exe):
        exe = str(tmp_path / "scale_exhaustive")
        subprocess.check_call([cc, "-O2", "-fopenmp", os.path.join(ROOT, "oracle", "scale_exhaustive.c"),
                               "-o", exe])
    return exe


def test_scale_two_step_rounding_matches_exact_rational(tmp_path):
    """numpy's fp16(fp32(d)/15) path equals fp16_rne(d/15) computed with
    integer arithmetic, on a spread of ranges d."""
    exe = _scale_tool(tmp_path)
    rng = np.random.default_rng(3)
    d = np.concatenate([
        np.exp(rng.uniform(np.log(1e-9), np.log(1e6), 20000)).astype(np.float32),
        np.float32([1.0, 15.0, 7.5, 0.1, 65504.0, 983040.0, 2.0 ** -24, 6e-8, 1e-45]),
    ])
    bits = d.view(np.uint32)
    out = subprocess.run([exe, "exact"], input="\n".join(f"{b:08x}" for b in bits),
                         capture_output=True, text=True, check=True).stdout.split()
    exact = np.array([int(h, 16) for h in out], dtype=np.uint16)
    ours = (d / np.float32(15.0)).astype(np.float16).view(np.uint16)
    assert np.array_equal(exact, ours)


def test_scale_exhaustive_all_fp32(tmp_path):
    """Every positive finite fp32 d: fp16(fp32(d/15)) == fp16(exact d/15)."""
    exe = _scale_tool(tmp_path)
    r = subprocess.run([exe, "all"], capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "checked 2139095039 mismatches 0"


# ---------------------------------------------------------------- INT8 blocks


def test_int8_block_bound_and_brute_force():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((200, 128), dtype=np.float32)
    x[:, 5] *= 20
    xv = O.bf16_to_f64(bf16_bits_from_f32(x))
    codes, s = O.int8_block_quantize(xv)
    assert codes.shape == (200, 128) and s.shape == (4,)
    for b in range(4):
        blk = xv[b * 64:(b + 1) * 64]
        sb = float(s[b])
        assert sb == float(np.float32(np.float32(np.abs(blk).max()) / np.float32(127)))
        recon = codes[b * 64:(b + 1) * 64].astype(np.float64) * sb
        assert np.all(np.abs(blk - recon) <= sb / 2 * (1 + 1e-6))
        # brute force nearest over all 255 codes (exact halves do not occur here)
        cand = np.arange(-127, 128, dtype=np.float64) * sb
        near = np.abs(blk[..., None] - cand).argmin(-1) - 127
        assert np.array_equal(near, codes[b * 64:(b + 1) * 64])
    assert np.abs(codes).max() == 127


def test_int8_zero_block():
    x = np.zeros((70, 128))
    x[64:, 0] = 1.0
    codes, s = O.int8_block_quantize(x)
    assert s[0] == 0 and np.all(codes[:64] == 0)
    assert codes[64, 0] == 127 and float(s[1]) == float(np.float32(1) / np.float32(127))
