"""CPU checks behind the GPU grid-edge cases: the oracle on the same inputs.

The padded worked example must reproduce the hand-worked values of tests/golden (so the padding
argument holds), and the edge rows must reach the branch each GPU assertion names (so the GPU
cases test what they claim).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from oracle import gptq_quantize
from test_gpu_grid_edges import _POS, degenerate_grid, edge_layer, expected_branches, padded_worked_example


@pytest.mark.parametrize("decision", [np.float64, np.float32])
def test_padded_worked_example_reproduces_golden(decision):
    gold, W, H = padded_worked_example()
    o = gptq_quantize(W.astype(np.float64), H, 2, 32, 0.01, decision=decision)
    assert o["lam"] == 1.0
    np.testing.assert_array_equal(o["codes"][:, _POS], np.array(gold["codes"]))
    np.testing.assert_array_equal(o["zeros"], np.array(gold["zeros"]))
    s_gold = np.array([[float(Fraction(t)) for t in row] for row in gold["scales"]])
    np.testing.assert_allclose(o["scales"], s_gold, rtol=1e-7 if decision is np.float32 else 1e-15)
    np.testing.assert_allclose(o["what"][:, _POS], np.array(gold["w_hat"]), rtol=1e-7, atol=1e-12)
    np.testing.assert_allclose(o["loss"], np.array(gold["row_loss"]), rtol=1e-12)
    pad = [c for c in range(64) if c not in _POS]
    assert np.all(o["what"][:, pad] == 0.0)
    # the padded columns are uncoupled in the factor
    U = o["U"]
    assert np.all(U[np.ix_(_POS, pad)] == 0.0)


@pytest.mark.parametrize("bits,g", [(2, 32), (3, 64), (4, 128), (4, -1), (8, 32), (3, -1)])
def test_edge_rows_reach_their_branches(bits, g):
    rpk, cols = 8, 384
    W, H32 = edge_layer(rpk, cols, seed=bits * 10 + (g % 7))
    o = gptq_quantize(W.astype(np.float64), H32.astype(np.float64), bits, g, 0.01, decision=np.float32)
    kind = expected_branches(rpk, cols, bits, g)
    s0, z0 = degenerate_grid(bits)
    zero = kind == "zero"
    assert np.all(o["scales"][zero].astype(np.float32) == s0) and np.all(o["zeros"][zero] == z0)
    assert (kind == "pos").any() and (kind == "neg").any()
    assert np.all(o["zeros"][kind == "pos"] == 0)
    assert np.all(o["zeros"][kind == "neg"] == 2 ** bits - 1)
