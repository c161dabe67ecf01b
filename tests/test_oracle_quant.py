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


# ---- O9 reference line: uniform per-token INT8 ----

def test_int8_token_closed_form_and_exact_dequant():
    """A token whose values are m * 2^e with max |m| = 127 has s = 2^e
    exactly and codes m: the dequantized token equals the input."""
    rng = np.random.default_rng(91)
    m = rng.integers(-127, 128, size=(5, 128))
    m[:, 7] = 127 * np.array([1, -1, 1, -1, 1])  # the maximum magnitude of each token
    e = np.array([-3, 0, 2, -10, 5])
    x = m * np.ldexp(1.0, e)[:, None]
    codes, s = O.int8_token_quantize(x)
    assert np.array_equal(s.astype(np.float64), np.ldexp(1.0, e))
    assert np.array_equal(codes.astype(np.int64), m)
    assert np.array_equal(codes.astype(np.float64) * s.astype(np.float64)[:, None], x)


def test_int8_token_half_integer_quotients_round_to_even():
    """s = 1 (max |x| = 127): quotients k + 0.5 go to the even neighbour."""
    x = np.zeros((1, 128))
    x[0, 0] = 127.0
    x[0, 1:7] = [2.5, 3.5, -2.5, -3.5, 0.5, 126.5]
    codes, s = O.int8_token_quantize(x)
    assert s[0] == 1.0
    assert codes[0, :7].tolist() == [127, 2, 4, -2, -4, 0, 126]


def test_int8_token_error_bound_and_zero_token():
    """|x - code * s| <= s / 2 + 2^-23 |x| for 16-bit inputs (exact in
    fp32), per token: the fp32 quotient x / s can move a value that sits on a
    half-integer by 2^-24 relative (x = max / 2 lands there exactly); an
    all-zero token has s = 0 and codes 0."""
    rng = np.random.default_rng(92)
    x = O.to_f64(bf16_bits_from_f32(rng.standard_normal((64, 128)).astype(np.float32) * 3.0), "bf16")
    x[5] = 0.0
    codes, s = O.int8_token_quantize(x)
    err = np.abs(x - codes.astype(np.float64) * s.astype(np.float64)[:, None])
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 + np.ldexp(np.abs(x), -23))
    assert s[5] == 0 and not codes[5].any()
    # brute force: each code is a nearest of the 255 levels to the fp32
    # quotient (ties: the even one)
    lv = np.arange(-127, 128, dtype=np.float64)
    for t in (0, 17, 63):
        qt = (x[t].astype(np.float32) / s[t]).astype(np.float64)
        d = np.abs(qt[:, None] - lv[None, :])
        best = d.min(axis=1)
        ok = np.abs(qt - codes[t].astype(np.float64)) == best
        assert ok.all()


def test_uniform_int8_attention_reduces_to_softmax_attention():
    """When every token is exactly representable the INT8 reference line is
    plain softmax attention; otherwise it is within a small error of it."""
    rng = np.random.default_rng(93)
    m = rng.integers(-127, 128, size=(300, 128)).astype(np.float64)
    m[:, 0] = 127
    K = m * 0.03125
    V = np.roll(m, 3, axis=1) * 0.0625
    q = rng.standard_normal((4, 128))
    a = O.uniform_int8_attention(q, K, V, 0.088)
    b = O.softmax_attention(q, K, V, 0.088)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


# ---- O11: OCP FP8 (E4M3) prefill blocks ----

def test_fp8_decode_closed_forms():
    """Values the E4M3 definition fixes: 1.0, 1.5, -1, the largest finite
    (448), the smallest normal (2^-6), the smallest and largest subnormals
    (2^-9, 7 x 2^-9), signed zero, and the two NaN patterns; the 127
    non-negative finite patterns increase with the code."""
    d = O.fp8_e4m3_decode(np.arange(256, dtype=np.uint8))
    fixed = {0x38: 1.0, 0x3C: 1.5, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x00: 0.0, 0x40: 2.0, 0x77: 240.0}
    for c, val in fixed.items():
        assert d[c] == val, hex(c)
    assert np.signbit(d[0x80]) and d[0x80] == 0.0
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.sum(np.isnan(d)) == 2
    assert np.all(np.diff(d[:0x7F]) > 0)
    assert np.array_equal(d[0x80:0xFF], -d[:0x7F])


def test_fp8_encode_round_trip_ties_and_nearest():
    d = O.fp8_e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = np.nonzero(~np.isnan(d))[0].astype(np.uint8)
    assert np.array_equal(O.fp8_e4m3_encode(d[finite].astype(np.float32)), finite)
    pos = d[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)     # exact in fp32
    enc = O.fp8_e4m3_encode(mid)
    assert np.all((enc & 1) == 0)                             # ties go to the even mantissa
    assert np.all((enc == np.arange(0x00, 0x7E)) | (enc == np.arange(0x01, 0x7F)))
    # just off the midpoints: the nearer neighbour
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(-np.inf))
    assert np.array_equal(O.fp8_e4m3_encode(up), np.arange(0x01, 0x7F))
    assert np.array_equal(O.fp8_e4m3_encode(dn[1:]), np.arange(0x01, 0x7E))
    assert O.fp8_e4m3_encode(np.float32(463.9)) == 0x7E and O.fp8_e4m3_encode(np.float32(-1e-4)) == 0x80


def test_fp8_encode_matches_torch_cast():
    """A library routine that implements the same format: torch's fp32 ->
    float8_e4m3fn cast (round to nearest even) on the CPU."""
    import torch
    rng = np.random.default_rng(11)
    mags = rng.choice([1e-4, 1e-3, 1e-2, 0.1, 1.0, 10.0, 100.0], 60000)
    x = np.concatenate([rng.standard_normal(60000) * mags, rng.uniform(-448, 448, 20000),
                        np.ldexp(rng.uniform(-1, 1, 20000), -7)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_e4m3_encode(x), ref)


def test_fp8_block_brute_force_and_bound():
    """Per block: the scale's definition, the block maximum on +-448, each
    code the nearest E4M3 value to fp32(x / s) by exhaustive search (ties,
    which do not occur here, aside), and |x - decode(code) s| <= 2^-4 |x| +
    2^-10 s (half a spacing, relative in the normal range, absolute in the
    subnormal one)."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((150, 128), dtype=np.float32)
    x[:, 9] *= 30
    x[3, :] *= 1e-4
    xv = O.bf16_to_f64(bf16_bits_from_f32(x))
    codes, s = O.fp8_block_quantize(xv)
    assert codes.shape == (150, 128) and s.shape == (3,)
    table = O.fp8_e4m3_decode(np.arange(256, dtype=np.uint8))
    fin = np.nonzero(~np.isnan(table))[0]
    for b in range(3):
        blk = xv[b * 64:(b + 1) * 64]
        sb = np.float32(s[b])
        assert sb == np.float32(np.float32(np.abs(blk).max()) / np.float32(448))
        c = codes[b * 64:(b + 1) * 64]
        assert np.abs(O.fp8_e4m3_decode(c)).max() == 448.0
        qv = (blk.astype(np.float32) / sb).astype(np.float64)
        dist = np.abs(qv[..., None] - table[fin])
        best = dist.min(-1, keepdims=True)
        ok = dist == best
        chosen = (fin[None, None, :] == c[..., None].astype(np.int64))
        assert np.all((ok & chosen).any(-1)), b
        recon = O.fp8_e4m3_decode(c) * float(sb)
        assert np.all(np.abs(blk - recon) <= 2.0 ** -4 * np.abs(blk) + 2.0 ** -10 * float(sb) + 1e-300)


def test_fp8_zero_block_and_signed_zero():
    x = np.zeros((70, 128))
    x[64:, 0] = -2.0
    x[64:, 1] = -0.0
    codes, s = O.fp8_block_quantize(x)
    assert s[0] == 0 and np.all(codes[:64] == 0)
    assert codes[64, 0] == 0xFE and codes[64, 1] == 0x80 and codes[64, 2] == 0x00
    assert float(s[1]) == float(np.float32(2) / np.float32(448))
