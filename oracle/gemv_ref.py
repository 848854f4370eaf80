"""Dequantizing matrix-vector product oracle -- test infrastructure only.

The serving side of a quantized layer (OneComp hub article, quantizer table and
"code architecture": the quantized weights are saved and later run for
inference; OneComp v1.1.0 release post, vLLM plugins for GPTQ models).  The
pages fix no kernel and no format beyond the group-wise asymmetric grid: a
weight is w^ = s_g (q - z_g) with the scale s_g and zero z_g of its group.
Reading taken here: the product consumes exactly what the quantizer and the
packer produce -- the per-row little-endian bitstream of b-bit codes
(pack_ref), fp32 scales [rows, G] and integer zeros [rows, G] -- and returns
y = W^ x in float64 (no rounding of W^ or of the sum before the end).
"""

from __future__ import annotations

import numpy as np

from .pack_ref import unpack_ref


def dequant_ref(codes, scales, zeros, groupsize: int) -> np.ndarray:
    """w^[r, j] = scales[r, j // g] * (codes[r, j] - zeros[r, j // g]) in float64 (g = cols if groupsize == -1)."""
    codes = np.asarray(codes, dtype=np.float64)
    rows, cols = codes.shape
    g = cols if groupsize == -1 else groupsize
    gi = np.arange(cols) // g
    s = np.asarray(scales, dtype=np.float64)[:, gi]
    z = np.asarray(zeros, dtype=np.float64)[:, gi]
    return s * (codes - z)


def dequant_gemv_ref(packed, scales, zeros, bits: int, groupsize: int, x, cols: int) -> np.ndarray:
    """y = W^ x for the packed codes of a [rows, cols] layer; x [cols] (or [cols, k] for several vectors)."""
    codes = unpack_ref(packed, cols, bits)
    return dequant_ref(codes, scales, zeros, groupsize) @ np.asarray(x, dtype=np.float64)
