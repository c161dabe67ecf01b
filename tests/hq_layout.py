"""Read-back helpers for tests: turn the library's tiled cache buffers into the
canonical per-position view the oracle uses. Pure data movement following the
byte layout documented in include/hq.h (no attention arithmetic here)."""
import numpy as np

TILE = 64


def _vcode_word_index():
    """word index (uint32) inside a 4096-byte V-code tile for (pair P, quad Q)."""
    P = np.arange(32)[:, None]
    Q = np.arange(32)[None, :]
    u, j, c8, e = P // 8, P % 8, Q // 2, Q % 2
    off = (j // 2) * 1024 + (16 * u + c8) * 16 + ((j % 2) * 2 + e) * 4
    return off // 4


_VIDX = _vcode_word_index()


def unpack_k_codes(kc: np.ndarray, BG: int, cap_q: int) -> np.ndarray:
    """[BG*cap_q/64*4096] bytes -> canonical codes [BG][cap_q][128] uint8."""
    nt = cap_q // TILE
    b = kc.reshape(BG, nt, 4, TILE, 16).transpose(0, 1, 3, 2, 4).reshape(BG, cap_q, 64)
    out = np.empty((BG, cap_q, 128), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def unpack_v_codes(vc: np.ndarray, BG: int, cap_q: int) -> np.ndarray:
    nt = cap_q // TILE
    w = vc.view(np.uint32).reshape(BG, nt, 1024)[:, :, _VIDX]          # [BG][nt][P][Q]
    halves = np.stack([w & 0xFFFF, w >> 16], axis=2)                  # [BG][nt][half][P][Q]
    nib = np.stack([(halves >> (4 * n)) & 0xF for n in range(4)], axis=-1)  # [..][Q][4]
    # slot = P + 32 * half
    return nib.reshape(BG, nt, 2, 32, 128).reshape(BG, cap_q, 128).astype(np.uint8)


def unpack_meta(meta: np.ndarray, BG: int, cap_q: int):
    """-> (s, z) float16 [BG][cap_q][4]."""
    m = meta.view(np.float16).reshape(BG, cap_q, 4, 2)
    return m[..., 0], m[..., 1]


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
    d["k_s"], d["k_z"] = unpack_meta(host["k_meta"][: BG * c.cap_q * 16], BG, c.cap_q)
    d["v_s"], d["v_z"] = unpack_meta(host["v_meta"][: BG * c.cap_q * 16], BG, c.cap_q)
    if c.window > 0:
        d["k_win"] = unpack_k16(host["k_win"][: BG * c.window * 256], BG, c.window)
        d["v_win"] = unpack_v16(host["v_win"][: BG * c.window * 256], BG, c.window)
    return d
