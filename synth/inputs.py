"""Seeded synthetic workloads shaped like the long-context Llama-3.1-8B
attention the HyQuant pages evaluate on.

The pages ("How HyQuant uses hybrid-precision attention to cut decode
compute", section "What the authors tested") measure on real models and
public benchmarks that are not available here. These tensors stand in for
them: the attention shapes (32 query / 8 KV heads, head_dim 128, the 70B-like
64 / 8 variant), the context lengths of the pages' speed table (1K-32K) and
beyond, heavy outlier channels in K (the failure mode the pages' TL;DR
describes for uniform low-bit grids), and planted "vertical line" key
columns that every query attends to (the structure the probe looks for).

Recipe (identical for every consumer):
  * master seed per workload; ``np.random.SeedSequence(seed).spawn(8)`` gives
    streams in a fixed order: 0 lengths, 1 outlier channels, 2 probe
    queries, 3 decode queries, 4 K, 5 V, 6 planted positions, 7 appended
    tokens;
  * values are drawn in fp32 and rounded once, round-to-nearest-even, to the
    16-bit storage type (bf16, or fp16 for the 1-head correctness workload);
  * Q, V ~ N(0, 1); K ~ N(0, 1) with ``n_outlier`` channels per KV head
    multiplied by ``outlier_scale`` (shared across batch and tokens);
  * planted columns per (batch, KV head): token 0 plus distinct random
    positions in [1, T - window); their key is
    ``4 * sqrt(D) * u + eps`` where ``u`` is the unit mean direction of the
    group's probe queries and ``eps`` is drawn like any other key, so the
    planted logit gain is about 4 * (q . u) in softmax units;
  * ragged batches draw T_b uniformly in [t_min, t_max] and pad to t_max.

Nothing here computes any part of the hybrid attention method.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# ---------------------------------------------------------------------------
# 16-bit storage rounding (data preparation only)
# ---------------------------------------------------------------------------


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to IEEE fp16 (nearest, ties to even); uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_from_f32(x)
    if dtype == "f16":
        return f16_bits_from_f32(x)
    raise ValueError(dtype)


def _bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    # Used only to build the planted direction from already-rounded queries.
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


# ---------------------------------------------------------------------------
# Workload definitions
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int                      # context length (t_max for ragged batches)
    D: int = 128
    dtype: str = "bf16"
    n_outlier: int = 4
    outlier_scale: float = 20.0
    plant_count: int | None = None     # fixed total per (b, g), incl. token 0
    plant_frac: float | None = None    # else round(frac * T_b) total
    ragged_min: int | None = None      # ragged: T_b ~ U[ragged_min, T]
    window: int = 128
    probe_rows: int = 64
    append_steps: int = 0
    seed: int = 20260911


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int = 128
    dtype: str = "bf16"
    n_outlier: int = 4
    outlier_scale: float = 20.0
    plant_frac: float = 0.005
    plant_count: int | None = None
    window: int = 128
    probe_rows: int = 64
    seed: int = 20260911


# The five workloads: 1-head 4K correctness case, the 8B GQA 32K decode
# (headline), 8B GQA 128K decode with appends, the 16K causal prefill, and
# the ragged 70B-like decode.
CONFIGS = {
    "decode_4k_1head": DecodeSpec(
        name="decode_4k_1head", B=1, Hq=1, Hkv=1, T=4096, dtype="f16",
        plant_count=21, seed=20260911 + 1),
    "decode_8b_32k": DecodeSpec(
        name="decode_8b_32k", B=16, Hq=32, Hkv=8, T=32768,
        plant_frac=0.005, seed=20260911 + 2),
    "decode_8b_128k_append": DecodeSpec(
        name="decode_8b_128k_append", B=4, Hq=32, Hkv=8, T=131072,
        plant_frac=0.005, append_steps=64, seed=20260911 + 3),
    "prefill_8b_16k": PrefillSpec(
        name="prefill_8b_16k", B=1, Hq=32, Hkv=8, T=16384,
        plant_frac=0.005, seed=20260911 + 4),
    "decode_70b_ragged_64k": DecodeSpec(
        name="decode_70b_ragged_64k", B=8, Hq=64, Hkv=8, T=65536,
        n_outlier=8, outlier_scale=30.0, plant_frac=0.01, ragged_min=16384,
        seed=20260911 + 5),
}


@dataclasses.dataclass
class DecodeInputs:
    spec: DecodeSpec
    seq_lens: np.ndarray        # [B] int32
    q_probe: np.ndarray         # [B][Hq][R][D] uint16 bits; row r is position T_b - R + r
    q: np.ndarray               # [B][Hq][D] uint16 bits (the decode query)
    k: np.ndarray               # [B][Hkv][Tmax][D] uint16 bits (zero beyond T_b)
    v: np.ndarray               # [B][Hkv][Tmax][D] uint16 bits
    planted: list               # [B][Hkv] -> sorted int array of planted positions
    outlier_channels: np.ndarray  # [Hkv][n_outlier]


@dataclasses.dataclass
class PrefillInputs:
    spec: PrefillSpec
    q: np.ndarray               # [B][Hq][T][D] uint16 bits
    k: np.ndarray               # [B][Hkv][T][D]
    v: np.ndarray               # [B][Hkv][T][D]
    planted: list
    outlier_channels: np.ndarray


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(8)]


def _outliers(rng, Hkv, D, n):
    return np.stack([np.sort(rng.choice(D, size=n, replace=False)) for _ in range(Hkv)]) \
        if n > 0 else np.zeros((Hkv, 0), dtype=np.int64)


def _plant_positions(rng, T_b, window, count):
    hi = max(1, T_b - window)
    count = max(1, min(count, hi))
    extra = rng.choice(np.arange(1, hi), size=count - 1, replace=False) if count > 1 else []
    return np.sort(np.concatenate([[0], np.asarray(extra, dtype=np.int64)])).astype(np.int64)


def _plant_count(spec, T_b):
    if spec.plant_count is not None:
        return spec.plant_count
    return max(1, int(round(spec.plant_frac * T_b)))


def _draw_keys(rng, n, D, out_ch, scale):
    x = rng.standard_normal((n, D), dtype=np.float32)
    if len(out_ch):
        x[:, out_ch] *= np.float32(scale)
    return x


def _unit_mean_dir(q_bits_group, dtype):
    """Unit vector along the mean of a group's probe queries (fp32)."""
    qf = _bits_to_f32(q_bits_group, dtype).reshape(-1, q_bits_group.shape[-1])
    m = qf.astype(np.float64).mean(axis=0)
    n = np.linalg.norm(m)
    return (m / n if n > 0 else m).astype(np.float32)


def _fill_kv(spec, s_out, s_k, s_v, s_plant, lens, q_probe_bits, Tmax):
    B, Hkv, D = spec.B, spec.Hkv, spec.D
    G = spec.Hq // Hkv
    out_ch = _outliers(s_out, Hkv, D, spec.n_outlier)
    k = np.zeros((B, Hkv, Tmax, D), dtype=np.uint16)
    v = np.zeros((B, Hkv, Tmax, D), dtype=np.uint16)
    planted = []
    amp = np.float32(4.0 * math.sqrt(D))
    for b in range(B):
        T_b = int(lens[b])
        row = []
        for g in range(Hkv):
            kf = _draw_keys(s_k, T_b, D, out_ch[g], spec.outlier_scale)
            pos = _plant_positions(s_plant, T_b, spec.window, _plant_count(spec, T_b))
            u = _unit_mean_dir(q_probe_bits[b, g * G:(g + 1) * G], spec.dtype)
            kf[pos] += amp * u[None, :]
            k[b, g, :T_b] = _to_bits(kf, spec.dtype)
            vf = s_v.standard_normal((T_b, D), dtype=np.float32)
            v[b, g, :T_b] = _to_bits(vf, spec.dtype)
            row.append(pos)
        planted.append(row)
    return k, v, planted, out_ch


def make_decode_inputs(spec: DecodeSpec) -> DecodeInputs:
    """Build the decode workload described by ``spec`` (deterministic)."""
    st = _streams(spec.seed)
    B, Hq, D, R = spec.B, spec.Hq, spec.D, spec.probe_rows
    if spec.ragged_min is not None:
        lens = st[0].integers(spec.ragged_min, spec.T + 1, size=B).astype(np.int32)
    else:
        lens = np.full(B, spec.T, dtype=np.int32)
    Tmax = spec.T
    q_probe = _to_bits(st[2].standard_normal((B, Hq, R, D), dtype=np.float32), spec.dtype)
    q = _to_bits(st[3].standard_normal((B, Hq, D), dtype=np.float32), spec.dtype)
    k, v, planted, out_ch = _fill_kv(spec, st[1], st[4], st[5], st[6], lens, q_probe, Tmax)
    return DecodeInputs(spec, lens, q_probe, q, k, v, planted, out_ch)


def make_append_tokens(spec: DecodeSpec, outlier_channels: np.ndarray, steps: int | None = None):
    """New K/V tokens and decode queries for ``steps`` consecutive appends.

    Returns (k_new [S][B][Hkv][D], v_new [S][B][Hkv][D], q [S][B][Hq][D]) as
    uint16 bits, drawn from stream 7 like ordinary (unplanted) tokens.
    """
    steps = spec.append_steps if steps is None else steps
    rng = _streams(spec.seed)[7]
    B, Hkv, Hq, D = spec.B, spec.Hkv, spec.Hq, spec.D
    kn = np.empty((steps, B, Hkv, D), dtype=np.uint16)
    vn = np.empty((steps, B, Hkv, D), dtype=np.uint16)
    qn = np.empty((steps, B, Hq, D), dtype=np.uint16)
    for s in range(steps):
        for g in range(Hkv):
            kn[s, :, g] = _to_bits(_draw_keys(rng, B, D, outlier_channels[g], spec.outlier_scale), spec.dtype)
        vn[s] = _to_bits(rng.standard_normal((B, Hkv, D), dtype=np.float32), spec.dtype)
        qn[s] = _to_bits(rng.standard_normal((B, Hq, D), dtype=np.float32), spec.dtype)
    return kn, vn, qn


def make_prefill_inputs(spec: PrefillSpec) -> PrefillInputs:
    """Causal prefill workload; the probe rows are the last rows of Q itself."""
    st = _streams(spec.seed)
    B, Hq, Hkv, T, D, R = spec.B, spec.Hq, spec.Hkv, spec.T, spec.D, spec.probe_rows
    q = _to_bits(st[2].standard_normal((B, Hq, T, D), dtype=np.float32), spec.dtype)
    lens = np.full(B, T, dtype=np.int32)
    q_probe = q[:, :, T - min(R, T):, :]
    k, v, planted, out_ch = _fill_kv(spec, st[1], st[4], st[5], st[6], lens, q_probe, T)
    return PrefillInputs(spec, q, k, v, planted, out_ch)


def small_decode_inputs(B=2, Hq=8, Hkv=2, T=700, D=128, dtype="bf16", window=128,
                        probe_rows=64, n_outlier=4, outlier_scale=20.0,
                        plant_frac=0.01, ragged_min=None, seed=1234) -> DecodeInputs:
    """Small decode workload with the same distributions (for parity tests)."""
    spec = DecodeSpec(name="small", B=B, Hq=Hq, Hkv=Hkv, T=T, D=D, dtype=dtype,
                      n_outlier=n_outlier, outlier_scale=outlier_scale,
                      plant_frac=plant_frac, ragged_min=ragged_min, window=window,
                      probe_rows=probe_rows, seed=seed)
    return make_decode_inputs(spec)
