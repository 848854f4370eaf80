"""Pins of the error-propagation correction oracle (CPU only)."""

import numpy as np
import pytest

from oracle import cross_ref, hessian_ref, qep_correct_ref


def _data(seed, tokens=200, n=24, rows=5, noise=0.05):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((tokens, n))
    Xq = X + noise * rng.standard_normal((tokens, n))
    W = rng.standard_normal((rows, n))
    return W, X, Xq


def _corr(W, X, Xq, alpha, damp):
    n = X.shape[1]
    return qep_correct_ref(W, hessian_ref([Xq], n), cross_ref([(X, Xq)], n), alpha, damp)


def test_cross_by_hand():
    X = np.array([[1.0, 2.0], [3.0, -1.0]])
    Xq = np.array([[0.5, 1.0], [2.0, 0.0]])
    # 2 X^T Xq = 2 [[1*0.5+3*2, 1*1+3*0], [2*0.5-1*2, 2*1-1*0]] = [[13, 2], [-2, 4]]
    np.testing.assert_array_equal(cross_ref([(X, Xq)], 2), [[13.0, 2.0], [-2.0, 4.0]])
    # chunks add up
    np.testing.assert_array_equal(cross_ref([(X[:1], Xq[:1]), (X[1:], Xq[1:])], 2), cross_ref([(X, Xq)], 2))


def test_no_error_no_correction_and_zero_strength():
    W, X, Xq = _data(1)
    np.testing.assert_allclose(_corr(W, X, X, 1.0, 0.01), W, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(_corr(W, X, Xq, 0.0, 0.01), W)


def test_full_strength_is_the_ridge_optimum():
    """Gradient of ||X W^T - X^ V^T||^2 + (lambda/2)||V - W||^2 vanishes at V = W_1."""
    W, X, Xq = _data(2)
    n = X.shape[1]
    H = hessian_ref([Xq], n)
    lam = 0.01 * np.mean(np.diag(H))
    V = _corr(W, X, Xq, 1.0, 0.01)
    grad = -2.0 * (X @ W.T - Xq @ V.T).T @ Xq + lam * (V - W)
    scale = 2.0 * np.abs(X @ W.T).T @ np.abs(Xq)
    assert np.max(np.abs(grad) / scale) < 1e-12


def test_undamped_limit_is_least_squares():
    """damp = 0 with full-rank X^: V^T = lstsq(X^, X W^T)."""
    W, X, Xq = _data(3, tokens=300, n=16)
    V = _corr(W, X, Xq, 1.0, 0.0)
    ref = np.linalg.lstsq(Xq, X @ W.T, rcond=None)[0].T
    np.testing.assert_allclose(V, ref, rtol=1e-9, atol=1e-10)


def test_square_inputs_reproduce_the_outputs():
    """tokens = n, X^ invertible, damp = 0: the corrected layer gives X W^T from X^ exactly."""
    W, X, Xq = _data(4, tokens=12, n=12)
    V = _corr(W, X, Xq, 1.0, 0.0)
    np.testing.assert_allclose(Xq @ V.T, X @ W.T, rtol=0, atol=1e-8)


def test_strength_is_linear():
    W, X, Xq = _data(5)
    V1 = _corr(W, X, Xq, 1.0, 0.01)
    np.testing.assert_allclose(_corr(W, X, Xq, 0.3, 0.01), W + 0.3 * (V1 - W), rtol=0, atol=1e-12)


def test_dead_input_column_contributes_nothing():
    """A column of X^ that is all zero is a dead column of H^: its G column is zero and the
    correction does not read it."""
    W, X, Xq = _data(6)
    Xq[:, 3] = 0.0
    n = X.shape[1]
    C = cross_ref([(X, Xq)], n)
    H = hessian_ref([Xq], n)
    np.testing.assert_array_equal((C - H)[:, 3], 0.0)
    V = _corr(W, X, Xq, 1.0, 0.01)
    assert np.all(np.isfinite(V))


# planted mistakes in a copy of the correction: each must fail a pin above
MUTANTS = ["cross_transposed", "cross_without_2", "undamped_solve", "correction_left_multiplied"]


def _corr_mut(W, X, Xq, alpha, damp, mut):
    n = X.shape[1]
    H = hessian_ref([Xq], n)
    lam = damp * np.mean(np.diag(H))
    C = cross_ref([(X, Xq)], n)
    if mut == "cross_transposed":
        C = C.T
    if mut == "cross_without_2":
        C = C / 2.0
    G = C - H
    Hd = H + (0.0 if mut == "undamped_solve" else lam) * np.eye(n)
    if mut == "correction_left_multiplied":
        return W + alpha * (W @ np.linalg.inv(Hd) @ G)
    return W + alpha * (W @ G) @ np.linalg.inv(Hd)


@pytest.mark.parametrize("mut", MUTANTS)
def test_each_planted_correction_mistake_is_caught(mut):
    W, X, Xq = _data(7)
    n = X.shape[1]
    H = hessian_ref([Xq], n)
    lam = 0.01 * np.mean(np.diag(H))
    V = _corr_mut(W, X, Xq, 1.0, 0.01, mut)
    grad = -2.0 * (X @ W.T - Xq @ V.T).T @ Xq + lam * (V - W)
    scale = 2.0 * np.abs(X @ W.T).T @ np.abs(Xq)
    assert np.max(np.abs(grad) / scale) > 1e-6, mut
