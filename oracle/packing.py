"""Code bitstream: the packing layout of the integer codes (oracle side).

TEST INFRASTRUCTURE (see the package docstring).

[BAL] section 1 says a format must state its packing layout, and section 6
that unpacking costs time at inference; neither gives a layout. Reading R17:
per output row, code k (original column order) occupies bits
[k*b, k*b + b) of a little-endian stream of uint32 words, least significant
bit first; a code whose bits cross a word boundary continues at bit 0 of the
next word. A row holds ceil(n_quant * b / 32) words.
"""
import numpy as np


def words_per_row(n_quant, bits):
    return (n_quant * bits + 31) // 32


def pack(codes, bits):
    """uint8 codes (rows x n_quant) -> uint32 words (rows x words_per_row)."""
    codes = np.asarray(codes, dtype=np.uint64)
    rows, nq = codes.shape
    words = np.zeros((rows, words_per_row(nq, bits)), np.uint64)
    for k in range(nq):
        off = k * bits
        w, sh = off // 32, off % 32
        val = (codes[:, k] & np.uint64((1 << bits) - 1)) << np.uint64(sh)
        words[:, w] |= val & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:
            words[:, w + 1] |= val >> np.uint64(32)
    return words.astype(np.uint32)


def unpack(words, nq, bits):
    """Inverse of :func:`pack`."""
    words = np.asarray(words, dtype=np.uint64)
    rows = words.shape[0]
    out = np.zeros((rows, nq), np.uint8)
    mask = np.uint64((1 << bits) - 1)
    for k in range(nq):
        off = k * bits
        w, sh = off // 32, off % 32
        val = words[:, w] >> np.uint64(sh)
        if sh + bits > 32:
            val |= words[:, w + 1] << np.uint64(32 - sh)
        out[:, k] = (val & mask).astype(np.uint8)
    return out
