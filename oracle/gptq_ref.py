"""fp64 NumPy oracle for GPTQ layer quantization -- test infrastructure only.

What is computed.  The pages name GPTQ as a 2-4 bit quantizer that rounds
weights "optimally" with the help of a Hessian matrix, slow but accurate
(OneComp hub article, "core features", item 2: the quantizer table), driven by
the knobs ``wbits`` and ``groupsize`` (same article, item 3: the LPCD example,
``GPTQ(wbits=3, groupsize=128)``), used layer by layer (same article,
"limitations", point 3), with RTN as the round-to-nearest baseline (quantizer
table).  The pages do not write the mathematics out; this module follows the
published method they name (GPTQ, Frantar et al. 2022) in its plainest form:

  H   = 2 X^T X over all calibration tokens, X [tokens, in_features]
  dead columns (H_ii == 0): H_ii := 1 and W[:, i] := 0
  H_d = H + lambda I,  lambda = damp * mean(diag H)
  U   = the upper-triangular factor with positive diagonal, U^T U = H_d^{-1}
  for j = 0 .. cols-1 in natural order:
      at a group start (j % g == 0): per-row asymmetric min/max grid from
      the CURRENT (error-updated) weights of the group's columns
      q_j = clamp(rint(w_j / s) + z, 0, maxq),  w^_j = s (q_j - z)
      e_j = (w_j - w^_j) / U_jj
      w_k -= e_j U_jk  for every k > j
      loss += (w_j - w^_j)^2 / (2 U_jj^2)

The grid (asymmetric min/max, zero forced into the range, integer zero
point) is the group-wise quantizer the release post names for 4-bit,
groupsize-128 group quantization (OneComp v1.1.0 release post, "new
quantization methods", Enhanced JointQ bullet).

Decisions.  Where floating point decides an integer (the grid, the rounding
of w/s, the zero point), ``decision`` selects the precision in which that
decision is taken: float64 gives the method's exact-as-possible value;
float32 takes it in the precision a float32 implementation uses (the current
weight is rounded to float32 first, then every grid operation is a float32
operation).  Error feedback and the loss always stay in float64.
"""

from __future__ import annotations

import numpy as np


class NotPositiveDefinite(ValueError):
    """The damped Hessian has no Cholesky factor."""


# ---------------------------------------------------------------------------
# Hessian and damping
# ---------------------------------------------------------------------------

def hessian_ref(chunks, n: int) -> np.ndarray:
    """H = 2 * sum over chunks of X_c^T X_c, accumulated in float64.

    Each chunk is an array [tokens_c, n] of any float dtype; values are widened
    exactly to float64 before the product.
    """
    H = np.zeros((n, n), dtype=np.float64)
    for X in chunks:
        X64 = np.asarray(X, dtype=np.float64)
        if X64.shape[1] != n:
            raise ValueError("chunk width does not match n")
        H += 2.0 * (X64.T @ X64)
    return H


def damp_ref(H, W, damp: float):
    """Dead-column fix then damping.

    Columns with H_ii == 0 never see a non-zero input: their diagonal is set
    to 1 and their weights to 0 before damping, so lambda is taken over the
    fixed diagonal.  Returns (H_d, W_staged, dead_mask, lambda).
    """
    Hd = np.array(H, dtype=np.float64, copy=True)
    Ws = np.array(W, dtype=np.float64, copy=True)
    n = Hd.shape[0]
    dead = np.diag(Hd) == 0.0
    di = np.nonzero(dead)[0]
    Hd[di, di] = 1.0
    Ws[:, dead] = 0.0
    lam = damp * np.mean(np.diag(Hd)) if n else 0.0
    Hd[np.diag_indices(n)] += lam
    return Hd, Ws, dead, lam


# ---------------------------------------------------------------------------
# Factor
# ---------------------------------------------------------------------------

def factor_ref(Hd) -> np.ndarray:
    """U upper with positive diagonal and U^T U = inv(H_d): invert, then Cholesky.

    Raises NotPositiveDefinite when H_d (or its inverse) has no Cholesky factor.
    """
    try:
        np.linalg.cholesky(Hd)
        Hinv = np.linalg.inv(Hd)
        L = np.linalg.cholesky(Hinv)
    except np.linalg.LinAlgError as exc:  # pragma: no cover - message only
        raise NotPositiveDefinite(str(exc)) from exc
    return np.ascontiguousarray(L.T)


def factor_ref_reverse(Hd) -> np.ndarray:
    """The same U by a second route: H_d = R R^T with R upper, then U = R^{-1}.

    R comes from the ordinary lower Cholesky factor of the index-reversed
    matrix, flipped back.  inv(H_d) = R^{-T} R^{-1} = (R^{-1})^T (R^{-1}),
    and R^{-1} is upper with a positive diagonal, so it is the unique U.
    """
    try:
        Lr = np.linalg.cholesky(Hd[::-1, ::-1])
    except np.linalg.LinAlgError as exc:  # pragma: no cover
        raise NotPositiveDefinite(str(exc)) from exc
    R = Lr[::-1, ::-1]
    return np.ascontiguousarray(np.linalg.inv(R))


def factor_ref_large(Hd) -> np.ndarray:
    """The reverse route of factor_ref_reverse on PyTorch's CPU LAPACK, in fp64.

    For the wide layers (n in the tens of thousands) where NumPy's general
    inverse takes minutes: the lower Cholesky factor of the index-reversed
    H_d flipped back gives the upper R with H_d = R R^T, and U = R^{-1} comes
    from one upper-triangular solve against the identity.  Same U as
    factor_ref up to rounding.
    """
    import torch
    H = torch.from_numpy(np.ascontiguousarray(Hd, dtype=np.float64))
    Lr, info = torch.linalg.cholesky_ex(H.flip(0, 1).contiguous())
    if int(info) != 0:
        raise NotPositiveDefinite(f"leading minor {int(info)} is not positive definite")
    R = Lr.flip(0, 1).contiguous()
    del Lr
    n = R.shape[0]
    eye = torch.eye(n, dtype=torch.float64)
    U = torch.linalg.solve_triangular(R, eye, upper=True)
    return U.numpy()


# ---------------------------------------------------------------------------
# Grid
# ---------------------------------------------------------------------------

def grid_params(wgroup, maxq: int, decision=np.float64):
    """Per-row asymmetric min/max grid of one group, shape [rows, group_width].

    xmin = min(min w, 0), xmax = max(max w, 0); an all-zero group uses [-1, 1];
    s = (xmax - xmin) / maxq; z = rint(-xmin / s) (half to even).
    All operations in the ``decision`` dtype.  Returns (s, z).
    """
    dt = decision
    w = np.asarray(wgroup).astype(dt)
    xmin = np.minimum(w.min(axis=1), dt(0))
    xmax = np.maximum(w.max(axis=1), dt(0))
    degenerate = (xmin == 0) & (xmax == 0)
    xmin = np.where(degenerate, dt(-1), xmin).astype(dt)
    xmax = np.where(degenerate, dt(1), xmax).astype(dt)
    s = ((xmax - xmin) / dt(maxq)).astype(dt)
    z = np.rint(-xmin / s).astype(dt)
    return s, z


def quantize_column(w, s, z, maxq: int, decision=np.float64):
    """q = clamp(rint(w / s) + z, 0, maxq) and w^ = s (q - z), in the decision dtype."""
    dt = decision
    r = (np.asarray(w).astype(dt) / s).astype(dt)
    q = np.clip(np.rint(r) + z, dt(0), dt(maxq)).astype(dt)
    what = (s * (q - z)).astype(dt)
    return q, what, r


def _group(groupsize: int, cols: int) -> int:
    g = cols if groupsize == -1 else groupsize
    if g <= 0:
        raise ValueError("groupsize must be positive or -1")
    return max(g, 1)


# ---------------------------------------------------------------------------
# GPTQ
# ---------------------------------------------------------------------------

def gptq_from_factor(W, U, bits: int, groupsize: int, blocksize: int | None = None,
                     decision=np.float64):
    """Quantize W [rows, cols] (already dead-zeroed) against the factor U [cols, cols].

    blocksize None runs the per-column definition.  A positive blocksize runs
    the lazy-batch form: in-block feedback per column, then one trailing
    product W[:, b1:] -= E U[b0:b1, b1:] per block, which equals the
    per-column form in exact arithmetic; it requires group starts to fall on
    block starts or groups to lie inside blocks.

    Returns a dict: codes (int64 [rows, cols]), scales and zeros (float64
    [rows, G]), what (float64 [rows, cols]), loss (float64 [rows]) and err
    (the scaled errors e, float64 [rows, cols]).
    """
    W = np.array(W, dtype=np.float64, copy=True)
    U = np.asarray(U, dtype=np.float64)
    rows, cols = W.shape
    maxq = 2 ** bits - 1
    g = _group(groupsize, cols)
    G = -(-cols // g) if cols else 0
    codes = np.zeros((rows, cols), dtype=np.int64)
    what = np.zeros((rows, cols), dtype=np.float64)
    err = np.zeros((rows, cols), dtype=np.float64)
    scales = np.zeros((rows, G), dtype=np.float64)
    zeros = np.zeros((rows, G), dtype=np.float64)
    loss = np.zeros(rows, dtype=np.float64)
    s = z = None

    def step(j, b1):
        nonlocal s, z
        if j % g == 0:
            s, z = grid_params(W[:, j:j + g], maxq, decision)
            scales[:, j // g] = s
            zeros[:, j // g] = z
        q, wh, _ = quantize_column(W[:, j], s, z, maxq, decision)
        wh = wh.astype(np.float64)
        d = W[:, j] - wh
        e = d / U[j, j]
        W[:, j + 1:b1] -= np.outer(e, U[j, j + 1:b1])
        codes[:, j] = q.astype(np.int64)
        what[:, j] = wh
        err[:, j] = e
        loss[:] += d * d / (2.0 * U[j, j] * U[j, j])

    if blocksize is None:
        for j in range(cols):
            step(j, cols)
    else:
        B = int(blocksize)
        if not (g % B == 0 or B % g == 0 or g >= cols):
            raise ValueError("lazy-batch form needs block-aligned groups")
        for b0 in range(0, cols, B):
            b1 = min(b0 + B, cols)
            for j in range(b0, b1):
                step(j, b1)
            if b1 < cols:
                W[:, b1:] -= err[:, b0:b1] @ U[b0:b1, b1:]
    return {"codes": codes, "scales": scales, "zeros": zeros, "what": what,
            "loss": loss, "err": err}


def gptq_quantize(W, H, bits: int, groupsize: int, damp: float = 0.01,
                  blocksize: int | None = None, decision=np.float64, route: str = "inv-chol"):
    """Full layer: dead-column fix, damping, factor, then the GPTQ loop.

    ``route`` picks the factor route ("inv-chol" or "reverse"); both give the
    same U up to rounding.  The result dict also carries U, H_d, the staged W,
    the dead mask and lambda.
    """
    Hd, Ws, dead, lam = damp_ref(H, W, damp)
    U = factor_ref(Hd) if route == "inv-chol" else factor_ref_reverse(Hd)
    out = gptq_from_factor(Ws, U, bits, groupsize, blocksize, decision)
    out.update({"U": U, "Hd": Hd, "W_staged": Ws, "dead": dead, "lam": lam})
    return out


def rtn_ref(W, bits: int, groupsize: int, decision=np.float64):
    """Round-to-nearest baseline: the same grid on the raw weights, no feedback."""
    W = np.asarray(W, dtype=np.float64)
    rows, cols = W.shape
    maxq = 2 ** bits - 1
    g = _group(groupsize, cols)
    G = -(-cols // g) if cols else 0
    codes = np.zeros((rows, cols), dtype=np.int64)
    what = np.zeros((rows, cols), dtype=np.float64)
    scales = np.zeros((rows, G), dtype=np.float64)
    zeros = np.zeros((rows, G), dtype=np.float64)
    for gi in range(G):
        c0, c1 = gi * g, min(gi * g + g, cols)
        s, z = grid_params(W[:, c0:c1], maxq, decision)
        scales[:, gi], zeros[:, gi] = s, z
        for j in range(c0, c1):
            q, wh, _ = quantize_column(W[:, j], s, z, maxq, decision)
            codes[:, j] = q.astype(np.int64)
            what[:, j] = wh
    return {"codes": codes, "scales": scales, "zeros": zeros, "what": what}


def layer_error(W0, What, H0) -> float:
    """Relative layer output error tr(D H0 D^T) / tr(W0 H0 W0^T), D = W0 - What.

    With the undamped H0 = 2 X^T X this equals ||(W0 - What) X^T||_F^2 / ||W0 X^T||_F^2.
    """
    W0 = np.asarray(W0, dtype=np.float64)
    D = W0 - np.asarray(What, dtype=np.float64)
    H0 = np.asarray(H0, dtype=np.float64)
    return float(np.sum((D @ H0) * D) / np.sum((W0 @ H0) * W0))


# ---------------------------------------------------------------------------
# Replay comparison against another implementation's codes
# ---------------------------------------------------------------------------

def _tie_distance(r):
    """Distance of r from the nearest rounding boundary (a half-integer), in code units."""
    r = np.asarray(r, dtype=np.float64)
    return np.abs(r - np.floor(r) - 0.5)


def replay_compare(W, U, bits: int, groupsize: int, codes, scales, zeros, tau: float,
                   decision=np.float32, rows_sel=None, blocksize: int | None = None):
    """Run the per-column loop, adopting the other side's codes as it goes.

    At every (row, column) the oracle's own code is computed from its own
    state; if the other side's code differs, the flip is a tie flip when the
    oracle's pre-rounding value w/s lies within ``tau`` code units of a
    rounding boundary and a hard flip otherwise.  The loop then continues
    with the other side's code, so one flip never contaminates later
    comparisons.  Zero points are treated the same way (-xmin/s is their
    pre-rounding value).  Scales are compared relatively on this aligned
    history.

    ``codes``, ``scales``, ``zeros`` hold the other side's outputs for the
    rows in ``rows_sel`` (all rows when None); W and U are the staged weights
    of those rows and the full factor.

    ``blocksize`` selects the lazy-batch form of the same loop, as in
    gptq_from_factor: feedback inside the block per column, the rest of the
    row once per block.  Both forms give the same result in exact arithmetic;
    the per-column form (None) is the definition.
    """
    W = np.array(W, dtype=np.float64, copy=True)
    if rows_sel is not None:
        W = W[rows_sel]
    U = np.asarray(U, dtype=np.float64)
    codes = np.asarray(codes, dtype=np.int64)
    scales = np.asarray(scales, dtype=np.float64)
    zeros = np.asarray(zeros, dtype=np.float64)
    rows, cols = W.shape
    dt = decision
    maxq = 2 ** bits - 1
    g = _group(groupsize, cols)
    st = {"total": rows * cols, "mismatch": 0, "tie_flips": 0, "hard_flips": 0,
          "zero_mismatch": 0, "zero_hard": 0, "max_scale_rel": 0.0, "min_tie_gap": np.inf,
          "groups": 0}
    what = np.zeros((rows, cols), dtype=np.float64)
    err = np.zeros((rows, cols), dtype=np.float64)
    s = z = None
    B = cols if blocksize is None else int(blocksize)
    if blocksize is not None and not (g % B == 0 or B % g == 0 or g >= cols):
        raise ValueError("lazy-batch form needs block-aligned groups")

    def step(j, b1):
        nonlocal s, z
        if j % g == 0:
            s, z = grid_params(W[:, j:j + g], maxq, dt)
            gi = j // g
            s_o = scales[:, gi].astype(dt)
            z_o = zeros[:, gi].astype(dt)
            rel = np.abs(s_o.astype(np.float64) - s.astype(np.float64)) / np.abs(s.astype(np.float64))
            st["max_scale_rel"] = max(st["max_scale_rel"], float(rel.max(initial=0.0)))
            zm = z_o != z
            if zm.any():
                xmin = np.minimum(W[:, j:j + g].astype(dt).min(axis=1), dt(0))
                rz = (-xmin / s).astype(dt)
                tie = _tie_distance(rz) <= tau
                st["zero_mismatch"] += int(zm.sum())
                st["zero_hard"] += int((zm & ~tie).sum())
            z = z_o
            st["groups"] += rows
        q, _, r = quantize_column(W[:, j], s, z, maxq, dt)
        qo = codes[:, j]
        mm = q.astype(np.int64) != qo
        if mm.any():
            gap = _tie_distance(r[mm])
            tie = gap <= tau
            st["mismatch"] += int(mm.sum())
            st["tie_flips"] += int(tie.sum())
            st["hard_flips"] += int((~tie).sum())
            st["min_tie_gap"] = min(st["min_tie_gap"], float(gap.min()))
        qa = qo.astype(dt)
        wh = (s * (qa - z)).astype(dt).astype(np.float64)
        d = W[:, j] - wh
        e = d / U[j, j]
        W[:, j + 1:b1] -= np.outer(e, U[j, j + 1:b1])
        what[:, j] = wh
        err[:, j] = e

    if blocksize is None:
        for j in range(cols):
            step(j, cols)
    else:
        for b0 in range(0, cols, B):
            b1 = min(b0 + B, cols)
            for j in range(b0, b1):
                step(j, b1)
            if b1 < cols:
                W[:, b1:] -= err[:, b0:b1] @ U[b0:b1, b1:]
    st["identical_frac"] = 1.0 - st["mismatch"] / max(st["total"], 1)
    st["what"] = what
    return st
