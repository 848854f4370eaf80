"""Pins of the Hadamard rotation oracle (CPU only)."""

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard_matrix, rotate_hessian_ref, rotate_rows_ref, rotation_ref


def _signs(n, seed):
    return np.where(np.random.default_rng(seed).random(n) < 0.5, -1.0, 1.0)


def test_small_hadamard_by_hand():
    np.testing.assert_array_equal(hadamard_matrix(1), [[1.0]])
    np.testing.assert_array_equal(hadamard_matrix(2), [[1, 1], [1, -1]])
    np.testing.assert_array_equal(hadamard_matrix(4), [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


@pytest.mark.parametrize("b", [1, 2, 8, 64, 512, 4096])
def test_hadamard_is_the_library_sylvester_matrix(b):
    np.testing.assert_array_equal(hadamard_matrix(b), scipy.linalg.hadamard(b))


@pytest.mark.parametrize("n,block", [(8, 8), (12, 4), (256, 256), (384, 128), (96, 1)])
def test_rotation_is_orthogonal(n, block):
    Q = rotation_ref(n, _signs(n, n + block), block)
    np.testing.assert_allclose(Q.T @ Q, np.eye(n), rtol=0, atol=1e-12)
    np.testing.assert_allclose(Q @ Q.T, np.eye(n), rtol=0, atol=1e-12)


def test_closed_forms_on_basis_and_ones():
    n, b = 16, 8
    ones = np.ones(n)
    e0 = np.zeros((1, n))
    e0[0, 0] = 1.0
    # the first row of H_b is all ones: e_0 spreads 1/sqrt(b) over its block only
    np.testing.assert_allclose(rotate_rows_ref(e0, ones, b)[0], np.r_[np.full(b, b ** -0.5), np.zeros(n - b)],
                               rtol=0, atol=1e-15)
    # the columns of H_b past the first sum to zero: a constant block goes to sqrt(b) e_0
    c = np.r_[np.ones(b), np.zeros(n - b)][None, :]
    np.testing.assert_allclose(rotate_rows_ref(c, ones, b)[0], np.r_[np.sqrt(b), np.zeros(n - 1)], rtol=0,
                               atol=1e-14)
    # a sign flips the row it multiplies before the transform
    s = ones.copy()
    s[0] = -1.0
    np.testing.assert_allclose(rotate_rows_ref(e0, s, b), -rotate_rows_ref(e0, ones, b), rtol=0, atol=0)


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    n, b = 8, 4
    A = rng.standard_normal((3, n))
    d = _signs(n, 1)
    out = rotate_rows_ref(A, d, b)
    hb = scipy.linalg.hadamard(b)
    for r in range(3):
        for j in range(n):
            acc = 0.0
            for k in range(n):
                if k // b == j // b:
                    acc += A[r, k] * d[k] * hb[k % b, j % b]
            assert abs(acc / np.sqrt(b) - out[r, j]) <= 1e-14


@pytest.mark.parametrize("n,block", [(64, 64), (96, 32), (48, 16)])
def test_layer_output_and_hessian_routes_agree(n, block):
    rng = np.random.default_rng(n)
    d = _signs(n, 7)
    W = rng.standard_normal((5, n))
    X = rng.standard_normal((40, n))
    Wr, Xr = rotate_rows_ref(W, d, block), rotate_rows_ref(X, d, block)
    # W' x' = W x for every token
    np.testing.assert_allclose(Xr @ Wr.T, X @ W.T, rtol=0, atol=1e-10)
    # the Hessian of rotated activations is the two-sided rotation of the Hessian
    H = 2.0 * X.T @ X
    Hr = rotate_hessian_ref(H, d, block)
    np.testing.assert_allclose(2.0 * Xr.T @ Xr, Hr, rtol=0, atol=1e-9)
    np.testing.assert_allclose(np.trace(Hr), np.trace(H), rtol=1e-13)
    np.testing.assert_allclose(np.linalg.norm(Hr), np.linalg.norm(H), rtol=1e-13)
    np.testing.assert_allclose(Hr, Hr.T, rtol=0, atol=1e-10)


# planted mistakes in a copy of the rotation: each must fail a pin above
MUTANTS = ["no_normalisation", "signs_after_transform", "q_h_qt", "blocks_shifted"]


def _rot_mut(n, d, b, mut):
    hb = scipy.linalg.hadamard(b).astype(np.float64)
    if mut != "no_normalisation":
        hb = hb / np.sqrt(b)
    q = np.kron(np.eye(n // b), hb)
    if mut == "blocks_shifted":
        q = np.roll(q, 1, axis=1)
    if mut == "signs_after_transform":
        return q * np.asarray(d)[None, :]
    return np.asarray(d)[:, None] * q


def _brute_rows(A, d, b):
    """A Q element by element: sum over k in j's block of A[r, k] d[k] H_b[k mod b, j mod b] / sqrt(b)."""
    hb = scipy.linalg.hadamard(b)
    m, n = A.shape
    out = np.zeros((m, n))
    for r in range(m):
        for j in range(n):
            out[r, j] = sum(A[r, k] * d[k] * hb[k % b, j % b] for k in range(n) if k // b == j // b) / np.sqrt(b)
    return out


@pytest.mark.parametrize("mut", MUTANTS)
def test_each_planted_rotation_mistake_is_caught(mut):
    """A mutant rotation Qm is run through the independent pins: orthogonality, the
    element-by-element definition, and the two Hessian routes."""
    n, b = 16, 8
    d = _signs(n, 5)
    Qm = _rot_mut(n, d, b, mut)
    rng = np.random.default_rng(2)
    A = rng.standard_normal((3, n))
    X = rng.standard_normal((30, n))
    H = 2.0 * X.T @ X
    Hm = Qm @ H @ Qm.T if mut == "q_h_qt" else Qm.T @ H @ Qm
    caught = [
        not np.allclose(Qm.T @ Qm, np.eye(n), atol=1e-12),
        not np.allclose(A @ Qm, _brute_rows(A, d, b), atol=1e-12),
        not np.allclose(2.0 * (X @ Qm).T @ (X @ Qm), Hm, atol=1e-9),
    ]
    assert any(caught), mut


def test_pins_pass_on_the_oracle():
    """The same three checks hold for the oracle's own rotation."""
    n, b = 16, 8
    d = _signs(n, 5)
    Q = rotation_ref(n, d, b)
    rng = np.random.default_rng(2)
    A = rng.standard_normal((3, n))
    X = rng.standard_normal((30, n))
    np.testing.assert_allclose(Q.T @ Q, np.eye(n), atol=1e-12)
    np.testing.assert_allclose(rotate_rows_ref(A, d, b), _brute_rows(A, d, b), atol=1e-12)
    np.testing.assert_allclose(2.0 * (X @ Q).T @ (X @ Q), rotate_hessian_ref(2.0 * X.T @ X, d, b), atol=1e-9)
