"""Read-back helpers for tests: turn the library's tiled cache buffers into the
canonical per-position view the oracle uses. Pure data movement following the
byte layout documented in include/hq.h (no attention arithmetic here)."""
import numpy as np

TILE = 64


def _mf_nib(e):
    return 16 * (e & 1) + 4 * (e >> 1)


def _int4_maps():
    """(word index, nibble shift) of every (slot, channel) of a 4096-byte
    K-code and V-code tile, and the dword index of every (slot, group) of the
    K / V metadata blocks (the layouts documented in include/hq.h)."""
    t = np.arange(TILE)[:, None]
    c = np.arange(128)[None, :]
    kw = ((t >> 4) * 1024 + ((t & 15) + 16 * ((c >> 3) & 3)) * 16 + (c >> 5) * 4) // 4
    ks = _mf_nib(c & 7) + 0 * t
    vw = ((c >> 5) * 1024 + ((c & 15) + 16 * ((t >> 3) & 3)) * 16 + ((((c >> 4) & 1) << 1) | (t >> 5)) * 4) // 4
    vs = _mf_nib(t & 7) + 0 * c
    j = np.arange(4)[None, :]
    km = ((t & 15) + 16 * j) * 4 + (t >> 4)
    vm = t * 4 + j
    return kw, ks, vw, vs, km, vm


_KW, _KS, _VW, _VS, _KM, _VM = _int4_maps()


def _unpack_codes(buf, BG, cap_q, widx, shift):
    nt = cap_q // TILE
    w = buf.view(np.uint32).reshape(BG, nt, 1024)[:, :, widx]          # [BG][nt][64][128]
    return ((w >> shift.astype(np.uint32)) & 0xF).astype(np.uint8).reshape(BG, cap_q, 128)


def unpack_k_codes(kc: np.ndarray, BG: int, cap_q: int) -> np.ndarray:
    """[BG*cap_q/64*4096] bytes -> canonical codes [BG][cap_q][128] uint8."""
    return _unpack_codes(kc, BG, cap_q, _KW, _KS)


def unpack_v_codes(vc: np.ndarray, BG: int, cap_q: int) -> np.ndarray:
    return _unpack_codes(vc, BG, cap_q, _VW, _VS)


def _unpack_meta(meta, BG, cap_q, idx):
    nt = cap_q // TILE
    m = meta.view(np.uint32).reshape(BG, nt, 256)[:, :, idx].reshape(BG, cap_q, 4)
    h = m.view(np.uint16).reshape(BG, cap_q, 4, 2).view(np.float16)
    return h[..., 0], h[..., 1]


def unpack_meta(meta: np.ndarray, BG: int, cap_q: int, which: str = "k"):
    """-> (s, z) float16 [BG][cap_q][4] of the K ('k') or V ('v') metadata."""
    return _unpack_meta(meta, BG, cap_q, _KM if which == "k" else _VM)


def unpack_k16(buf: np.ndarray, BG: int, cap: int) -> np.ndarray:
    """16-bit K tiles -> [BG][cap][128] uint16 bits."""
    nt = cap // TILE
    x = buf.view(np.uint16).reshape(BG, nt, 16, TILE, 8).transpose(0, 1, 3, 2, 4)
    return x.reshape(BG, cap, 128)


def unpack_v16(buf: np.ndarray, BG: int, cap: int) -> np.ndarray:
    nt = cap // TILE
    x = buf.view(np.uint16).reshape(BG, nt, 16, 4, 16, 8).transpose(0, 1, 3, 2, 4, 5)
    return x.reshape(BG, cap, 128)


def read_cache(cache) -> dict:
    """Copy a kv_cache_amd.HybridCache to host and decode every buffer."""
    import torch  # noqa: F401
    c = cache.c
    BG = c.B * c.Hkv
    host = {k: v.cpu().numpy() for k, v in cache.bufs.items()}
    if getattr(cache, "q_tile_off", None) is not None:
        # ragged INT4 pools: each (b, g)'s span copied into the uniform
        # [BG][cap_q] arrangement (zero past its capacity)
        off, qt = cache.q_tile_off, c.cap_q // 64
        for name, per_tile in (("k_codes", 4096), ("v_codes", 4096), ("k_meta", 1024), ("v_meta", 1024),
                               ("q_pos", 256)):
            dense = np.zeros(BG * qt * per_tile, dtype=np.uint8)
            for bg in range(BG):
                a, b = off[bg], off[bg + 1]
                dense[bg * qt * per_tile:(bg * qt + b - a) * per_tile] = host[name][a * per_tile:b * per_tile]
            host[name] = dense
    d = {
        "counts": host["counts"][: BG * 16].view(np.int32).reshape(c.B, c.Hkv, 4),
        "k_codes": unpack_k_codes(host["k_codes"][: BG * c.cap_q * 64], BG, c.cap_q),
        "v_codes": unpack_v_codes(host["v_codes"][: BG * c.cap_q * 64], BG, c.cap_q),
        "q_pos": host["q_pos"][: BG * c.cap_q * 4].view(np.int32).reshape(BG, c.cap_q),
        "keep_pos": host["keep_pos"][: BG * c.cap_keep * 4].view(np.int32).reshape(BG, c.cap_keep),
        "k_keep": unpack_k16(host["k_keep"][: BG * c.cap_keep * 256], BG, c.cap_keep),
        "v_keep": unpack_v16(host["v_keep"][: BG * c.cap_keep * 256], BG, c.cap_keep),
        "err_flag": int(host["err_flag"][:4].view(np.int32)[0]),
        "thresh": host["thresh"][: BG * 8].view(np.int32).reshape(BG, 2),
        "col_scores": host["col_scores"][: BG * c.cap_probe * 4].view(np.float32).reshape(BG, c.cap_probe),
    }
    d["k_s"], d["k_z"] = unpack_meta(host["k_meta"][: BG * c.cap_q * 16], BG, c.cap_q, "k")
    d["v_s"], d["v_z"] = unpack_meta(host["v_meta"][: BG * c.cap_q * 16], BG, c.cap_q, "v")
    if c.window > 0:
        d["k_win"] = unpack_k16(host["k_win"][: BG * c.window * 256], BG, c.window)
        d["v_win"] = unpack_v16(host["v_win"][: BG * c.window * 256], BG, c.window)
    return d
