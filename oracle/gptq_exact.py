"""Exact rational GPTQ for tiny inputs -- test infrastructure only.

The same method as ``gptq_ref`` (per-column GPTQ with group-wise asymmetric
min/max grids; the OneComp hub article's quantizer table names it as the
Hessian-guided 2-4 bit quantizer), reached by a different route so that the
two check each other:

* no Cholesky factor and no square root.  Row j of the upper factor U of
  inv(H_d) is the first row of inv(H_d[j:, j:]) divided by the square root of
  its first entry (the Schur complement of a leading block of an inverse is
  the inverse of the trailing block).  Hence the feedback coefficient
  U_jk / U_jj equals x_k / x_j and U_jj^2 equals x_j, where x solves
  H_d[j:, j:] x = e_1 -- all rational;
* every value is a ``fractions.Fraction``; rint is half-to-even on the exact
  value.

Inputs must be exactly representable rationals (dyadic weights, integer or
dyadic Hessians); damp is a Fraction (0.01 is Fraction(1, 100)).
"""

from __future__ import annotations

from fractions import Fraction
from math import floor


def rint_half_even(x: Fraction) -> int:
    f = floor(x)
    rem = x - f
    if rem < Fraction(1, 2):
        return f
    if rem > Fraction(1, 2):
        return f + 1
    return f if f % 2 == 0 else f + 1


def _solve_first_unit(A):
    """Solve A x = e_1 for a small dense rational matrix by Gauss-Jordan elimination."""
    m = len(A)
    M = [list(A[i]) + [Fraction(1 if i == 0 else 0)] for i in range(m)]
    for c in range(m):
        p = next((r for r in range(c, m) if M[r][c] != 0), None)
        if p is None:
            raise ZeroDivisionError("singular trailing block")
        M[c], M[p] = M[p], M[c]
        piv = M[c][c]
        M[c] = [v / piv for v in M[c]]
        for r in range(m):
            if r != c and M[r][c] != 0:
                f = M[r][c]
                M[r] = [a - f * b for a, b in zip(M[r], M[c])]
    return [M[i][m] for i in range(m)]


def gptq_exact(W, H, bits: int, groupsize: int, damp=Fraction(1, 100)):
    """Exact per-column GPTQ.  W: rows x cols, H: cols x cols, nested lists of Fractions.

    Returns dict with codes, scales, zeros (per row per group), what, loss
    (per row, sum of d^2 / (2 U_jj^2)), and the damped Hessian.
    """
    W = [[Fraction(v) for v in row] for row in W]
    H = [[Fraction(v) for v in row] for row in H]
    rows, n = len(W), len(H)
    maxq = 2 ** bits - 1
    g = n if groupsize == -1 else groupsize
    for i in range(n):
        if H[i][i] == 0:
            H[i][i] = Fraction(1)
            for r in range(rows):
                W[r][i] = Fraction(0)
    lam = Fraction(damp) * sum(H[i][i] for i in range(n)) / n
    Hd = [[H[i][k] + (lam if i == k else 0) for k in range(n)] for i in range(n)]
    G = -(-n // g)
    codes = [[0] * n for _ in range(rows)]
    what = [[Fraction(0)] * n for _ in range(rows)]
    scales = [[Fraction(0)] * G for _ in range(rows)]
    zeros = [[0] * G for _ in range(rows)]
    loss = [Fraction(0)] * rows
    for j in range(n):
        x = _solve_first_unit([row[j:] for row in Hd[j:]])
        ujj2 = x[0]
        if ujj2 <= 0:
            raise ValueError("damped Hessian is not positive definite")
        ratio = [xk / x[0] for xk in x]
        for r in range(rows):
            if j % g == 0:
                grp = W[r][j:j + g]
                xmin = min(min(grp), Fraction(0))
                xmax = max(max(grp), Fraction(0))
                if xmin == 0 and xmax == 0:
                    xmin, xmax = Fraction(-1), Fraction(1)
                s = (xmax - xmin) / maxq
                scales[r][j // g] = s
                zeros[r][j // g] = rint_half_even(-xmin / s)
            s = scales[r][j // g]
            z = zeros[r][j // g]
            q = min(max(rint_half_even(W[r][j] / s) + z, 0), maxq)
            wh = s * (q - z)
            d = W[r][j] - wh
            codes[r][j] = q
            what[r][j] = wh
            loss[r] += d * d / (2 * ujj2)
            for k in range(j + 1, n):
                W[r][k] -= d * ratio[k - j]
    return {"codes": codes, "scales": scales, "zeros": zeros, "what": what, "loss": loss, "Hd": Hd}
