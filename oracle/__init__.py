"""CPU oracle for the VJP ops -- TEST INFRASTRUCTURE, not part of the product.

A plain, slow, fp64 numpy statement of what each forward and backward
computes, written from the definitions on the source pages:

* "Backward in Triton -- autograd.Function and the backward grid"
  (fused scaled-SiLU, fp32 gradient accumulation, ``+=`` into gradients);
* "Writing Triton Kernels with Autograd: A Minimal End-to-End Example"
  (row-wise weighted sum, two-stage grad_w reduction);
* "Backprop for kernel writers" (the VJP contract, the softmax collapse,
  the fused softmax-cross-entropy, logsumexp statistics, LayerNorm's
  two-row-scalar backward, the scatter-add backward of a gather; RMSNorm's
  dw reduction from "Backward in Triton").

Every function takes and returns float64 arrays and computes the plain
definition of its result; there is no tiling, fusion or reordering beyond
what the definition states.  Outputs are rounded to a storage dtype only by
:func:`oracle.rounding.round_to` (direct fp64 -> dtype, round to nearest
even), so no result is rounded twice.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path
(``row_wise_backward_amd``) and imports nothing from it.

Parity status: every function here is pinned by tests that do not re-type
its formula (finite differences, brute-force Jacobians, library routines,
invariants, special cases, the weighted-sum page's worked tiling example,
exhaustive rounding enumeration).  No function is "parity unpinned".
"""
from . import gather, norms, rounding, scaled_silu, softmax, softmax_xent, weighted_sum  # noqa: F401
