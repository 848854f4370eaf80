"""Oracle for the GPTQ layer quantizer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation of what the HIP path
computes, written from the method's definition.  Only the test suite,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
or run anything in this package; the product path never does, and this
package imports nothing from the product path.

Modules
  gptq_ref    fp64 NumPy: Hessian, damping, factor, per-column GPTQ and its
              lazy-batch variant, RTN, layer error, replay comparison.
  gptq_exact  exact rational GPTQ (fractions.Fraction) for tiny dyadic inputs,
              reached through a different route (trailing principal inverses
              instead of a Cholesky factor).
  pack_ref    LSB-first per-row bitstream packing and unpacking.
  gemv_ref    dequantization of packed codes and the product y = W^ x.
  hadamard_ref  the fixed randomised Hadamard rotation Q and W Q, Q^T H Q.
  qep_ref     the error-propagation correction of W from full-precision and
              quantized-model inputs, before GPTQ.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against closed forms, the hand-worked 4x8 example in ``tests/golden``,
invariants and the exact rational route.  No function is left unpinned.
"""

from .gptq_ref import (  # noqa: F401
    NotPositiveDefinite,
    damp_ref,
    factor_ref,
    factor_ref_reverse,
    factor_ref_large,
    gptq_from_factor,
    gptq_quantize,
    grid_params,
    hessian_ref,
    layer_error,
    quantize_column,
    replay_compare,
    rtn_ref,
)
from .pack_ref import pack_ref, unpack_ref  # noqa: F401
from .gemv_ref import dequant_gemv_ref, dequant_ref  # noqa: F401
from .qep_ref import cross_ref, qep_correct_ref, qep_quantize_ref  # noqa: F401
from .hadamard_ref import hadamard_matrix, rotate_hessian_ref, rotate_rows_ref, rotation_ref  # noqa: F401
