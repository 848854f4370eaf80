"""Pins of the dequantizing product oracle (CPU only)."""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dequant_gemv_ref, dequant_ref, pack_ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_4x8_2bit_g4.json")


def test_dequant_matches_hand_worked_w_hat():
    # the hand-traced 4x8 example: its codes, scales and zeros decode to its w^ exactly
    gd = json.load(open(GOLDEN))
    scales = [[float(Fraction(v)) for v in row] for row in gd["scales"]]
    wh = dequant_ref(gd["codes"], scales, gd["zeros"], gd["parameters"]["groupsize"])
    np.testing.assert_array_equal(wh, np.array(gd["w_hat"], dtype=np.float64))


def test_gemv_hand_vector():
    # one 32-column row, 4-bit, groups of 32: codes 0..15 twice, s = 1/2, z = 3,
    # x = 1 on the first 16 columns: y = (1/2) * sum_{q=0}^{15} (q - 3) = (1/2) * 72 = 36
    codes = np.array([list(range(16)) * 2])
    x = np.r_[np.ones(16), np.zeros(16)]
    y = dequant_gemv_ref(pack_ref(codes, 4), [[0.5]], [[3]], 4, 32, x, 32)
    assert y.shape == (1,) and y[0] == 36.0


@pytest.mark.parametrize("bits,g", [(2, 32), (3, 64), (4, 128), (8, -1)])
def test_gemv_invariants(bits, g):
    rng = np.random.default_rng(bits)
    rows, cols = 5, 256
    G = 1 if g == -1 else cols // g
    codes = rng.integers(0, 2 ** bits, size=(rows, cols))
    scales = rng.uniform(0.01, 0.1, size=(rows, G))
    zeros = rng.integers(0, 2 ** bits, size=(rows, G))
    p = pack_ref(codes, bits)
    # unit vectors pick the dequantized columns; zero codes at the zero point vanish
    for j in (0, 31, 32, 255):
        e = np.zeros(cols)
        e[j] = 1.0
        gj = 0 if g == -1 else j // g
        np.testing.assert_array_equal(dequant_gemv_ref(p, scales, zeros, bits, g, e, cols),
                                      scales[:, gj] * (codes[:, j] - zeros[:, gj]))
    zc = np.repeat(zeros, cols // G, axis=1)
    assert np.all(dequant_gemv_ref(pack_ref(zc, bits), scales, zeros, bits, g, rng.standard_normal(cols), cols) == 0)
    # linear in x, and several vectors at once agree with one at a time
    X = rng.standard_normal((cols, 3))
    Y = dequant_gemv_ref(p, scales, zeros, bits, g, X, cols)
    for k in range(3):
        np.testing.assert_allclose(Y[:, k], dequant_gemv_ref(p, scales, zeros, bits, g, X[:, k], cols), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dequant_gemv_ref(p, scales, zeros, bits, g, X[:, 0] + 2 * X[:, 1], cols),
                               Y[:, 0] + 2 * Y[:, 1], rtol=1e-12, atol=1e-12)


def test_gemv_brute_force_small():
    # element-by-element definition on a tiny 3-bit layer
    rng = np.random.default_rng(7)
    rows, cols, g = 2, 64, 32
    codes = rng.integers(0, 8, size=(rows, cols))
    scales = rng.uniform(0.1, 1.0, size=(rows, 2))
    zeros = rng.integers(0, 8, size=(rows, 2))
    x = rng.standard_normal(cols)
    y = dequant_gemv_ref(pack_ref(codes, 3), scales, zeros, 3, g, x, cols)
    for r in range(rows):
        acc = 0.0
        for j in range(cols):
            acc += scales[r, j // g] * (codes[r, j] - zeros[r, j // g]) * x[j]
        assert abs(acc - y[r]) <= 1e-12 * max(1.0, abs(acc))


# planted mistakes in a copy of the dequantization: each must fail a pin above
GEMV_MUTANTS = ["zero_added", "group_of_next_column", "scale_of_column_index", "codes_msb_first"]


def _dequant_mut(codes, scales, zeros, groupsize, mut):
    codes = np.asarray(codes, dtype=np.float64)
    rows, cols = codes.shape
    g = cols if groupsize == -1 else groupsize
    gi = np.arange(cols) // g
    if mut == "group_of_next_column":
        gi = np.minimum(np.arange(1, cols + 1) // g, scales.shape[1] - 1)
    s = np.asarray(scales, dtype=np.float64)[:, gi]
    z = np.asarray(zeros, dtype=np.float64)[:, gi]
    if mut == "scale_of_column_index":
        s = np.asarray(scales, dtype=np.float64)[:, np.minimum(np.arange(cols), scales.shape[1] - 1)]
    if mut == "zero_added":
        return s * (codes + z)
    if mut == "codes_msb_first":
        codes = codes[:, ::-1]
    return s * (codes - z)


@pytest.mark.parametrize("mut", GEMV_MUTANTS)
def test_each_planted_dequant_mistake_is_caught(mut):
    gd = json.load(open(GOLDEN))
    scales = np.array([[float(Fraction(v)) for v in row] for row in gd["scales"]])
    wh = _dequant_mut(gd["codes"], scales, np.array(gd["zeros"]), gd["parameters"]["groupsize"], mut)
    assert not np.array_equal(wh, np.array(gd["w_hat"], dtype=np.float64))
    assert np.array_equal(_dequant_mut(gd["codes"], scales, np.array(gd["zeros"]), 4, None),
                          np.array(gd["w_hat"], dtype=np.float64))
