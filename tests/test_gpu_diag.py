"""The streaming-read helper hq_diag_read_int4 (measurement aid, not a step
of the method) reads exactly the INT4 store it claims to: the XOR of every
word it writes to its sink equals the XOR of every 32-bit word of the
n_q/64 leading tiles of K codes, V codes, K scale/zero and V scale/zero of
each (b, g), computed on the host from the same cache buffers."""
import numpy as np
import pytest

from synth import small_decode_inputs

from test_gpu_cache_decode import _run_quantize

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kw", [dict(B=2, Hq=8, Hkv=2, T=700, ragged_min=389, seed=31),
                                dict(B=1, Hq=4, Hkv=1, T=3000, seed=32)])
def test_diag_read_int4_reads_the_int4_store(kw):
    import torch
    import kv_cache_amd as hq
    inp = small_decode_inputs(**kw)
    cache, _, _ = _run_quantize(inp, 128, (5, 100))
    sink = hq.diag_read_int4(cache)
    torch.cuda.synchronize()
    n = hq.lib.hq_diag_read_int4_sink_bytes(cache.ptr())
    got = np.bitwise_xor.reduce(sink[:n].cpu().numpy().view(np.uint32))
    counts = cache.counts().cpu().numpy().reshape(-1, 4)
    qt = cache.c.cap_q // 64
    want = np.uint32(0)
    for name, per_tile in (("k_codes", 4096), ("v_codes", 4096), ("k_meta", 1024), ("v_meta", 1024)):
        buf = cache.bufs[name].cpu().numpy()[: counts.shape[0] * qt * per_tile].reshape(counts.shape[0], qt * per_tile)
        for bg in range(counts.shape[0]):
            nqt = (int(counts[bg, 1]) + 63) // 64
            want ^= np.bitwise_xor.reduce(buf[bg, : nqt * per_tile].view(np.uint32))
    assert got == want
    assert cache.err_flag() == 0


def test_hw_exp2_error_within_the_probe_bound():
    """The probe's first pass takes 2^f, |f| <= 1/2, with the hardware base-2
    exponential; its score bound counts that instruction's relative error as
    at most 1.5 2^-24 there. Checked over every fp32 input in [-1/2, 1/2]
    (2.1e9 values) against the fp64 exponential."""
    import kv_cache_amd as hq
    from gpu_common import HW_EXP2_REL
    err = hq.diag_exp2_error(-0.5, 0.5)
    print(f"hardware exp2 on [-1/2, 1/2]: largest relative error {err:.4e} ({err / 2.0 ** -24:.3f} x 2^-24)")
    assert 0.0 < err <= HW_EXP2_REL
    # a one-point range still reports that point's error (2^0 is exact)
    assert hq.diag_exp2_error(0.0, 0.0, nblocks=4) == 0.0
