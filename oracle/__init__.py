"""CPU oracle for the LLM.int8() decomposed matmul -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product (the HIP library and its Python binding)
never imports, calls or links anything from here, and this package imports
nothing from the product.

* ``int8mm_ref``  -- plain numpy implementation of every step, in the order
  the pages give it (fp32 IEEE division, round-half-even, exact integer
  accumulation, fp32 epilogue).
* ``bruteforce``  -- pure-Python ``fractions.Fraction`` arithmetic for tiny
  shapes; pins the numpy oracle to the exact rational definition.

Every oracle function is pinned by CPU tests against things other than
itself: the brute force, closed forms, special thresholds that reduce to
textbook matmuls, invariants of the quantizer and the error bound of the
method.  Parity left unpinned: the low-order bits of the fp16 output Y, which
depend on fp32 summation order and are checked only by tolerance.
"""

from .int8mm_ref import (  # noqa: F401
    Q_MAX,
    quantize_rows_ref,
    prepare_weight_ref,
    outlier_mask_ref,
    quantize_activation_ref,
    outlier_slices_ref,
    int8_gemm_ref,
    outlier_gemm_ref,
    epilogue_ref,
    int8_matmul_ref,
    tolerance_bound,
)
