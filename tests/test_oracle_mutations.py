"""Planted mistakes: each plausible slip in the oracle's loop must fail a pin (CPU only).

``_loop`` is a copy of the oracle's per-column GPTQ loop with switches that
plant one mistake each (a dropped term, a wrong sign or index, a transposed
operand, the wrong rounding or range).  With no switch set it must pass the
hand-worked example; with any one switch set the worked example, the OBS
identity or the exact rational route must reject it.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import damp_ref, factor_ref
from oracle.gptq_exact import gptq_exact

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_4x8_2bit_g4.json")

MUTANTS = ["transposed_factor", "feedback_sign", "error_times_ujj", "feedback_index_shift",
           "raw_weight_groups", "zero_not_forced", "zero_point_floor", "round_half_away",
           "no_damping", "loss_missing_half", "group_window_shift"]


def _loop(W, H, bits, g, damp, mut=None):
    Hd, Ws, _, _ = damp_ref(H, W, 0.0 if mut == "no_damping" else damp)
    U = factor_ref(Hd)
    if mut == "transposed_factor":
        U = U.T.copy()
    W = Ws.copy()
    W_raw = Ws.copy()
    rows, n = W.shape
    maxq = 2 ** bits - 1
    codes = np.zeros((rows, n), dtype=np.int64)
    what = np.zeros((rows, n))
    loss = np.zeros(rows)
    rnd = (lambda x: np.floor(x + 0.5) if mut == "round_half_away" else np.rint(x))
    for j in range(n):
        if j % g == 0:
            src = W_raw if mut == "raw_weight_groups" else W
            lo = j + 1 if mut == "group_window_shift" else j
            grp = src[:, lo:lo + g] if lo < n else src[:, j:j + 1]
            if mut == "zero_not_forced":
                xmin, xmax = grp.min(1), grp.max(1)
            else:
                xmin, xmax = np.minimum(grp.min(1), 0), np.maximum(grp.max(1), 0)
            deg = (xmin == 0) & (xmax == 0)
            xmin = np.where(deg, -1.0, xmin)
            xmax = np.where(deg, 1.0, xmax)
            s = (xmax - xmin) / maxq
            z = np.floor(-xmin / s) if mut == "zero_point_floor" else rnd(-xmin / s)
        q = np.clip(rnd(W[:, j] / s) + z, 0, maxq)
        wh = s * (q - z)
        d = W[:, j] - wh
        e = d * U[j, j] if mut == "error_times_ujj" else d / U[j, j]
        sign = -1.0 if mut == "feedback_sign" else 1.0
        if mut == "feedback_index_shift":
            W[:, j + 1:] -= sign * np.outer(e, np.append(U[j, j + 2:], 0.0))
        else:
            W[:, j + 1:] -= sign * np.outer(e, U[j, j + 1:])
        codes[:, j] = q
        what[:, j] = wh
        half = 1.0 if mut == "loss_missing_half" else 2.0
        loss += d * d / (half * U[j, j] ** 2)
    return codes, what, loss, Hd, Ws


def _worked():
    with open(GOLD) as f:
        g = json.load(f)
    H = np.diag([100.0] * 8)
    for a, b in g["pairs"]:
        H[a, b] = H[b, a] = 50.5
    return g, np.array(g["W"]), H


def _pins_pass(mut):
    g, W, H = _worked()
    codes, what, loss, Hd, Ws = _loop(W, H, 2, 4, 0.01, mut)
    ok = np.array_equal(codes, np.array(g["codes"]))
    ok &= np.allclose(what, g["w_hat"], rtol=0, atol=1e-12)
    ok &= np.allclose(loss, g["row_loss"], rtol=1e-12)
    # OBS identity on the mutant's own outputs
    D = what - Ws
    ok &= np.allclose(loss, 0.5 * np.einsum("ri,ik,rk->r", D, Hd, D), rtol=1e-9)
    # an exact rounding tie with H = I (w/s = 0.5 rounds to the even 0)
    c, _, _, _, _ = _loop(np.array([[-0.25, 0.0, 0.5, 0.125]]), np.eye(4), 2, 4, 0.01, mut)
    ok &= np.array_equal(c, [[0, 1, 3, 1]])
    # exact rational route on small random dyadic layers
    for seed in range(3):
        rng = np.random.default_rng(100 + seed)
        Wr = rng.integers(-64, 65, size=(3, 8)) / 64.0
        X = rng.integers(-4, 5, size=(24, 8)).astype(np.float64)
        Hr = 2.0 * X.T @ X
        ex = gptq_exact(Wr.tolist(), [[Fraction(int(v)) for v in r] for r in Hr], 3, 4)
        c, _, l, _, _ = _loop(Wr, Hr, 3, 4, 0.01, mut)
        ok &= np.array_equal(c, np.array(ex["codes"]))
        ok &= np.allclose(l, [float(v) for v in ex["loss"]], rtol=1e-9)
    return bool(ok)


def test_unmutated_copy_passes():
    assert _pins_pass(None)


@pytest.mark.parametrize("mut", MUTANTS)
def test_each_planted_mistake_is_caught(mut):
    assert not _pins_pass(mut), f"planted mistake {mut} slipped through every pin"


def test_hessian_missing_factor_two_is_caught():
    from oracle import hessian_ref
    X = np.eye(3)
    assert np.array_equal(hessian_ref([X], 3), 2 * np.eye(3))
    assert not np.array_equal(X.T @ X, 2 * np.eye(3))
