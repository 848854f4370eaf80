"""The factor's blocking, modelled in fp64 on the host: the schedule k_factor.hip runs, checked exact.

The device factor is a right-looking blocked Cholesky of the reversed damped Hessian A with the
transposed inverse L^-T folded into A's upper triangle.  Per block column k (columns [k0, c1)):

  * the block column solve: rows of the block become rows of L_kk^-T, every other row r takes
    A[r, k0:c1] L_kk^-T (panel rows below, inverse rows above);
  * the diagonal block of block k+1 is updated with every pending panel, then factored;
  * the GEMM A[r, j] -= A[r, kp:c1] L[j, kp:c1]^T over the pending panels kp .. c1: on block
    column k+1 at every step, on the columns past it only when the step flushes (every
    `lazy` panels, at the last steps, or when the step's GEMM is small), lower tiles of the
    trailing matrix only, and a pending panel's own rows starting their K range at their own
    block (before it their entries right of the diagonal were above the trailing triangle).

The model follows those rules with numpy products, as the host code of factor_run and the
tile enumeration of k_factor_step lay them out, and must reproduce numpy's Cholesky factor
and inverse to rounding.  Dropping the K floor must break it.
"""

from __future__ import annotations

import numpy as np
import pytest


def blocked_factor(H, NB, lazy, tiles_limit=0, k_floor=True):
    n = H.shape[0]
    A = np.tril(H).copy()
    nk = -(-n // NB)
    Lkk = {}

    def potrf(k):
        k0 = k * NB
        kb = min(NB, n - k0)
        D = A[k0:k0 + kb, k0:k0 + kb]
        Lkk[k] = np.linalg.cholesky(np.tril(D) + np.tril(D, -1).T)

    potrf(0)
    kp = 0  # first column of the pending panels
    for k in range(nk):
        k0 = k * NB
        kb = min(NB, n - k0)
        c1 = k0 + kb
        rest = n - c1
        Linv_T = np.linalg.inv(Lkk[k]).T
        for r in range(n):  # the block column solve
            if k0 <= r < c1:
                A[r, k0:c1] = Linv_T[r - k0]
            else:
                A[r, k0:c1] = A[r, k0:c1] @ Linv_T
        if rest <= 0:
            break
        kb1 = min(rest, NB)
        kn = c1 - kp
        nt = -(-rest // NB)
        tiles = (c1 // NB) * nt + nt * (nt + 1) // 2 - 1
        flush = kn >= lazy * NB or rest <= kb1 or tiles <= tiles_limit
        # the next diagonal block, with every pending panel
        P = A[c1:c1 + kb1, kp:c1]
        D = A[c1:c1 + kb1, c1:c1 + kb1] - P @ P.T
        A[c1:c1 + kb1, c1:c1 + kb1] = np.tril(D) + np.triu(A[c1:c1 + kb1, c1:c1 + kb1], 1)
        # the step GEMM: block column k+1 always, the columns past it on a flush
        jend = n if flush else c1 + kb1
        for tm in range(0, n, NB):
            rows = slice(tm, min(tm + NB, n))
            kbeg = tm if (k_floor and kp <= tm < c1) else kp
            upd = A[rows, kbeg:c1] @ A[c1:jend, kbeg:c1].T
            for jt in range(c1, jend, NB):
                if tm >= c1 and (jt > tm or (tm == c1 and jt == c1)):
                    continue  # upper tiles of the trailing matrix; its first block by the diagonal update
                cols = slice(jt, min(jt + NB, jend))
                A[rows, cols] -= upd[:, cols.start - c1:cols.stop - c1]
        potrf(k + 1)
        if flush:
            kp = c1
    L = np.tril(A)
    for k, Lk in Lkk.items():
        k0 = k * NB
        L[k0:k0 + Lk.shape[0], k0:k0 + Lk.shape[0]] = Lk
    return L, np.triu(A)


def _spd(n, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((2 * n, n)) * (1.0 + 3.0 * rng.random(n))
    return X.T @ X + 0.01 * n * np.eye(n)


@pytest.mark.parametrize("n,NB,lazy,tiles_limit", [
    (300, 32, 2, 0), (512, 64, 2, 0), (520, 64, 3, 0), (384, 128, 2, 0), (1000, 128, 2, 0),
    (700, 32, 2, 60),   # the size rule mixes deferred and immediate steps
    (610, 32, 4, 0), (900, 32, 8, 0), (257, 32, 1, 0),
])
def test_blocked_factor_is_exact(n, NB, lazy, tiles_limit):
    H = _spd(n, n + NB)
    L_ref = np.linalg.cholesky(H)
    Y_ref = np.linalg.inv(L_ref).T
    L, Y = blocked_factor(H, NB, lazy, tiles_limit)
    assert np.abs(L - L_ref).max() <= 1e-12 * np.abs(L_ref).max()
    assert np.abs(Y - Y_ref).max() <= 1e-12 * np.abs(Y_ref).max()


def test_size_rule_defers_some_steps_and_not_others():
    # the mixed case above must really contain both kinds of step
    n, NB, lazy, limit = 700, 32, 2, 60
    kinds = set()
    kp = 0
    nk = -(-n // NB)
    for k in range(nk - 1):
        c1 = min((k + 1) * NB, n)
        rest = n - c1
        nt = -(-rest // NB)
        tiles = (c1 // NB) * nt + nt * (nt + 1) // 2 - 1
        flush = (c1 - kp) >= lazy * NB or rest <= min(rest, NB) or tiles <= limit
        kinds.add(("flush" if flush else "defer", tiles <= limit))
        if flush:
            kp = c1
    assert ("defer", False) in kinds and ("flush", True) in kinds


def test_dropping_the_k_floor_breaks_the_inverse():
    H = _spd(300, 7)
    L_ref = np.linalg.cholesky(H)
    Y_ref = np.linalg.inv(L_ref).T
    _, Y = blocked_factor(H, 32, 2, k_floor=False)
    assert np.abs(Y - Y_ref).max() > 1e-6 * np.abs(Y_ref).max()
