"""Error-propagation correction before GPTQ -- test infrastructure only.

The OneComp pages describe QEP (quantization error propagation) only as an
idea: the error that quantizing the earlier layers leaves in a layer's inputs
is carried into that layer's own correction, so the quantized model tracks the
full-precision one; they cite the method's paper and code, which are not part
of the pages.  Reading taken here, the plainest one that idea supports: with
X [tokens, n] the layer's inputs in the full-precision model and X^ those in
the partly quantized model, the layer's weights are first moved to

    W' = argmin_V  || X W^T - X^ V^T ||_F^2 + (lambda / 2) || V - W ||_F^2
       = W + W G H_d^-1,      G = 2 (X - X^)^T X^,   H_d = 2 X^T X^ + lambda I

(the normal equations, with GPTQ's own damping lambda = damp * mean diag and
its dead-column rule on H^ = 2 X^T X^), blended by a propagation strength
alpha in [0, 1]:  W_alpha = W + alpha W G H_d^-1; then W_alpha is quantized by
GPTQ against H^.  Everything is fp64.
"""

from __future__ import annotations

import numpy as np

from .gptq_ref import damp_ref, gptq_quantize, hessian_ref


def cross_ref(chunks, n: int) -> np.ndarray:
    """C = 2 sum over chunks of X_c^T X^_c; chunks are pairs (X_c, X^_c) [tokens_c, n]."""
    C = np.zeros((n, n), dtype=np.float64)
    for X, Xq in chunks:
        C += 2.0 * (np.asarray(X, dtype=np.float64).T @ np.asarray(Xq, dtype=np.float64))
    return C


def qep_correct_ref(W, H_hat, C, alpha: float, damp: float = 0.01) -> np.ndarray:
    """W + alpha W G H_d^-1 with G = C - H^ (= 2 (X - X^)^T X^), H_d the damped H^."""
    W = np.asarray(W, dtype=np.float64)
    Hd, _, _, _ = damp_ref(H_hat, W, damp)
    G = np.asarray(C, dtype=np.float64) - np.asarray(H_hat, dtype=np.float64)
    # (W G) H_d^-1 by a solve: H_d symmetric, so (W G) H_d^-1 = (H_d^-1 (W G)^T)^T
    return W + alpha * np.linalg.solve(Hd, (W @ G).T).T


def qep_quantize_ref(W, X, Xq, alpha: float, bits: int, groupsize: int, damp: float = 0.01, blocksize=None):
    """Correct W from (X, X^), then GPTQ against H^ = 2 X^T X^."""
    n = np.asarray(X).shape[1]
    H_hat = hessian_ref([Xq], n)
    Wc = qep_correct_ref(W, H_hat, cross_ref([(X, Xq)], n), alpha, damp)
    out = gptq_quantize(Wc, H_hat, bits, groupsize, damp, blocksize=blocksize)
    out["W_corrected"] = Wc
    return out
