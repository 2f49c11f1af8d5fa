"""CPU oracle for the 4-bit (HiFA4-style) FlashAttention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP library (no kernels, no
headers, no constant tables, no pre/post-processing); the only shared module is
the seeded input generator ``synth``, which holds none of the method's
arithmetic.

The oracle is plain NumPy.  Arithmetic is FP64 with every rounding to a narrow
format made explicit; where the GPU computes a value in FP32 that later decides
an integer (a 4-bit code, a scale exponent, the running max), the oracle takes
that decision in FP32 too, emulating each FP32 operation exactly (``fp.py``).

Sources (cited by title and section):
  [HiFA4]  "HiFA4: Training-Free 4-bit FlashAttention on Ascend HIF4 NPUs for
           LLM Inference" (arXiv 2607.04302v1), Abstract and Section 1.
  [FA4P]   "Hardware-Aware FP4 FlashAttention-4" (arXiv 2609.04105), Abstract
           (prior art: mapping scores straight to FP4 probabilities).

Modules:
  fp         exact FP32 / FP16 rounding helpers (fma, two-operand sums, fract)
  mx         E2M1 codes with a power-of-two scale per 32-element block
  smooth     Smooth-QK calibration and the element-wise rescale
  rope       the FP32 rotate-half RoPE of the fused prologue (RoPE, then Smooth-QK,
             then quantization, from pre-RoPE FP16 inputs)
  attention  the tiled recurrence with P-Reordering, split-KV merge, the
             inconsistent-normalizer variant, epsilon statistics and the
             unquantized FP32 reference

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, invariants, textbook reductions).  The one
exception is the accumulator of the scaled MFMA (``attention.mfma_seq``): the
pages say nothing about it, so its rule (exact block products taken in block
order; operands far below the block's exponent anchor truncated; one FP32
rounding per block) comes from probing the instruction, and it is pinned on
the GPU by crafted operands through the library, not on the CPU.
"""

from . import fp, mx, smooth, attention  # noqa: F401
