"""Code packing oracle -- test infrastructure only.

The pages fix no on-disk format for the quantized checkpoint (OneComp v1.1.0
release post, "one-line core": the first quantized checkpoint is the
deployable artefact; OneComp hub article, "code architecture": a Quantizer
exposes quantize() and save()).  The reading taken here: per row, the codes
form one little-endian bitstream -- code i occupies bits [i*b, (i+1)*b) of the
row -- cut into 32-bit words, word w holding stream bits [32w, 32w+32).  For
b = 3 a group of 32 codes fills exactly three words.
"""

from __future__ import annotations

import numpy as np


def pack_ref(codes, bits: int) -> np.ndarray:
    """codes [rows, cols] (values < 2**bits) -> uint32 [rows, cols*bits/32]."""
    codes = np.asarray(codes, dtype=np.int64)
    rows, cols = codes.shape
    if (cols * bits) % 32:
        raise ValueError("cols * bits must be a multiple of 32")
    if codes.size and (codes.min() < 0 or codes.max() >= (1 << bits)):
        raise ValueError("code out of range")
    k = np.arange(bits, dtype=np.int64)
    stream = ((codes[:, :, None] >> k) & 1).reshape(rows, cols * bits)
    nw = cols * bits // 32
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    words = (stream.reshape(rows, nw, 32).astype(np.uint64) * weights).sum(axis=2)
    return words.astype(np.uint32)


def unpack_ref(packed, cols: int, bits: int) -> np.ndarray:
    """Inverse of pack_ref."""
    packed = np.asarray(packed, dtype=np.uint32)
    rows, nw = packed.shape
    bitpos = np.arange(32, dtype=np.uint32)
    stream = ((packed[:, :, None] >> bitpos) & 1).reshape(rows, nw * 32)[:, :cols * bits]
    weights = np.int64(1) << np.arange(bits, dtype=np.int64)
    return (stream.reshape(rows, cols, bits).astype(np.int64) * weights).sum(axis=2)
