"""The packed-code layout as the mlx-cpu 0.30.1 ``quantized.h`` page states it.

``affine_dequantize`` on that page reads packed bytes pack by pack: for 2-, 4-
and 8-bit codes one byte holds 8/bits codes, code i at bit ``bits*i``; for
3-bit codes 3 bytes hold 8 codes, for 5-bit 5 bytes hold 8 codes, for 6-bit 3
bytes hold 4 codes, with the field masks listed there.  The tables below
restate those masks as (byte, first bit, width, destination bit) pieces.
They are used only to pin the oracle's generic bit-stream pack and unpack,
which never look at these tables.
"""
import numpy as np

# code j of a pack <- list of (byte index, low bit in byte, n bits, dest bit)
_STRADDLE = {
    3: (3, [
        [(0, 0, 3, 0)],
        [(0, 3, 3, 0)],
        [(0, 6, 2, 0), (1, 0, 1, 2)],
        [(1, 1, 3, 0)],
        [(1, 4, 3, 0)],
        [(1, 7, 1, 0), (2, 0, 2, 1)],
        [(2, 2, 3, 0)],
        [(2, 5, 3, 0)],
    ]),
    5: (5, [
        [(0, 0, 5, 0)],
        [(0, 5, 3, 0), (1, 0, 2, 3)],
        [(1, 2, 5, 0)],
        [(1, 7, 1, 0), (2, 0, 4, 1)],
        [(2, 4, 4, 0), (3, 0, 1, 4)],
        [(3, 1, 5, 0)],
        [(3, 6, 2, 0), (4, 0, 3, 2)],
        [(4, 3, 5, 0)],
    ]),
    6: (3, [
        [(0, 0, 6, 0)],
        [(0, 6, 2, 0), (1, 0, 4, 2)],
        [(1, 4, 4, 0), (2, 0, 2, 4)],
        [(2, 2, 6, 0)],
    ]),
}


def decode_row_bytes(row_bytes: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Decode packed bytes [..., K*bits/8] into codes [..., K] per the page."""
    b = np.asarray(row_bytes, dtype=np.uint8)
    lead = b.shape[:-1]
    if bits in (2, 4, 8):
        per = 8 // bits
        mask = (1 << bits) - 1
        out = np.empty(lead + (K,), np.uint8)
        for i in range(per):
            out[..., i::per] = (b >> (bits * i)) & mask
        return out
    nbytes, pieces = _STRADDLE[bits]
    per = len(pieces)
    packs = b.reshape(lead + (K // per, nbytes)).astype(np.uint32)
    out = np.zeros(lead + (K // per, per), np.uint32)
    for j, plist in enumerate(pieces):
        for (byte, lo, width, dest) in plist:
            field = (packs[..., byte] >> lo) & ((1 << width) - 1)
            out[..., j] |= field << dest
    return out.reshape(lead + (K,)).astype(np.uint8)


def decode_words(w_q: np.ndarray, K: int, bits: int) -> np.ndarray:
    """uint32 words [..., K*bits/32] -> codes, reading the words as LE bytes."""
    w = np.ascontiguousarray(w_q, dtype="<u4")
    return decode_row_bytes(w.view(np.uint8), K, bits)
