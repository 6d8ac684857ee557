"""Unpacking of the library's packed FP8 operand layouts (as stated in
include/vc_attn.h) into the oracle's logical layouts, for comparisons."""
import numpy as np


def sw(r):
    r = np.asarray(r)
    return ((r >> 1) & 7) ^ ((r & 1) << 2)


kswz = sw
vswz = sw


def vkey_of_pos(p):
    """Key (within the tile) stored at byte position p of a packed V row."""
    p = np.asarray(p)
    return (p & 64) + 16 * ((p >> 2) & 3) + 4 * ((p >> 4) & 3) + (p & 3)


def unpack_k(packed: np.ndarray, D: int) -> np.ndarray:
    """[..., S_pad, D] packed K codes -> logical row-major codes."""
    S_pad = packed.shape[-2]
    ncl = D // 16
    x = packed.reshape(packed.shape[:-2] + (S_pad, ncl, 16))
    rows = np.arange(S_pad) % 128
    swr = kswz(rows) if D == 128 else (kswz(rows) & 3)
    out = np.empty_like(x)
    for c in range(ncl):
        out[..., c, :] = x[..., np.arange(S_pad), c ^ swr, :]  # logical chunk c sits at c ^ swizzle(row)
    return out.reshape(packed.shape)


def unpack_v(packed: np.ndarray, D: int) -> np.ndarray:
    """[..., D, S_pad] buffer holding packed V tiles [nblk][D][128] ->
    logical key-contiguous codes [..., D, S_pad]."""
    S_pad = packed.shape[-1]
    nblk = S_pad // 128
    lead = packed.shape[:-2]
    x = packed.reshape(lead + (nblk, D, 8, 16))
    sw = vswz(np.arange(D))
    pos = np.empty_like(x)
    swd = vswz(np.arange(D))
    for c in range(8):
        pos[..., :, :, c, :] = x[..., :, np.arange(D), c ^ swd, :]
    pos = pos.reshape(lead + (nblk, D, 128))  # by byte position inside the tile row
    out = np.empty_like(pos)
    out[..., vkey_of_pos(np.arange(128))] = pos  # position p holds key vkey_of_pos(p)
    # [..., nblk, D, 128] -> [..., D, nblk*128]
    out = np.moveaxis(out, -3, -2)
    return out.reshape(lead + (D, S_pad))


def k_matches(packed: np.ndarray, D: int, codes: np.ndarray, S: int) -> bool:
    """vc_quantize's packed K against the oracle's row-major K codes: rows
    < S equal, rows S .. S_pad - 1 copies of row S - 1 (the library pads K
    with the last key; the oracle with zeros, which the method never reads)."""
    got = unpack_k(packed, D)
    return bool((got[..., :S, :] == codes[..., :S, :]).all()
                and (got[..., S:, :] == got[..., S - 1:S, :]).all())
