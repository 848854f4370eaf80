"""Fixed randomised Hadamard rotation oracle -- test infrastructure only.

The OneComp hub article lists rotation preprocessing (rotations chosen before
quantization and absorbed into the weights, with online Hadamard hooks
registered at load) and, in its code-architecture listing, a pre-processing
package for rotation matrices and the Hadamard transform.  The pages define no
rotation; the learned ones need training.  Reading taken here: a fixed
orthogonal

    Q = D . blockdiag(H_b, ..., H_b) / sqrt(b),

D = diag(signs) with signs drawn by the caller (+-1 for a rotation), H_b the
Sylvester Hadamard matrix of order b (a power of two that divides n; H_1 = [1],
H_2m = [[H_m, H_m], [H_m, -H_m]]).  A layer y = W x is rewritten as
W' = W Q and x' = Q^T x, so W' x' = W x; activation rows X [tokens, n] become
X' = X Q and the Hessian becomes H' = 2 X'^T X' = Q^T H Q.  Everything is fp64.
"""

from __future__ import annotations

import numpy as np


def hadamard_matrix(b: int) -> np.ndarray:
    """H_b by the Sylvester doubling, b a power of two."""
    if b < 1 or b & (b - 1):
        raise ValueError("b must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < b:
        h = np.block([[h, h], [h, -h]])
    return h


def rotation_ref(n: int, signs, block: int) -> np.ndarray:
    """Q [n, n] = diag(signs) . blockdiag(H_block) / sqrt(block)."""
    if n % block:
        raise ValueError("block must divide n")
    hb = hadamard_matrix(block) / np.sqrt(block)
    q = np.kron(np.eye(n // block), hb)
    return np.asarray(signs, dtype=np.float64)[:, None] * q


def rotate_rows_ref(A, signs, block: int) -> np.ndarray:
    """A Q: every row of A [m, n] rotated (weights W -> W Q, activations X -> X Q)."""
    A = np.asarray(A, dtype=np.float64)
    return A @ rotation_ref(A.shape[1], signs, block)


def rotate_hessian_ref(H, signs, block: int) -> np.ndarray:
    """Q^T H Q for H [n, n]."""
    H = np.asarray(H, dtype=np.float64)
    Q = rotation_ref(H.shape[0], signs, block)
    return Q.T @ H @ Q
