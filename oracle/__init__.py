"""CPU oracle for the OFT dequant-GEMM path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, fp64 numpy code that states what the GPU library computes.  It
shares no code with the library (``orthogonal_fine_tuning_amd``) and neither
imports the other; both read their inputs from ``oft_inputs``.  Only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path never calls it and has no CPU fallback.

Sources.  The method is the OFT adapter of the Orbit pages:
  [P1] the Synced article on Orbit ("Orbit: first single-node RL of a
       trillion-parameter model", mirror at m.xxlwj.com), section
       "Technical details" (active-expert-chunked dequantisation;
       bypass-base-weight-grad GEMM backward);
  [P2] the chooseai.io news page "Sphere AI Lab releases Orbit, an open-source
       RL training framework built on OFT adapters", sections "Technical
       principles" (frozen low-precision base, BF16 OFT adapter carries every
       gradient), "Five design features of the adapter-first architecture"
       (custom split-projection adapter kernels), "Architectural advantages of
       OFT over LoRA" (each sub-space of a fused tensor gets its own orthogonal
       rotation) and "Dedicated optimisation for low-precision MoE models"
       (router-selected experts, fixed-size batches, temporary dequantisation,
       grouped GEMM).

The pages print no formula.  The readings this library implements:
  * each projection segment's output channels carry a block-diagonal
    orthogonal R with blocks of size b, each block the Cayley map
    R = (I + Q)(I - Q)^-1 of a skew-symmetric Q given by the bf16 parameters
    of its strict upper triangle;
  * y = rot_R(x . dequant(W0)^T): per token and block, y_blk = R . z_blk
    (row-major: Y_blk = Z_blk R^T);
  * training needs dX and dQ only; dW0 is never formed (frozen base).

Parity pins (``tests/test_oracle_*.py``): library casts for the number
codecs, closed forms for the Cayley map, Q = 0 reducing to the plain
dequantised GEMM, norm preservation, the adjoint identity, central finite
differences for dX / dQ / dw, a brute-force all-experts evaluation of the MoE
layer and library sorting for the routing.  Readings no page can pin (which
side is rotated, R versus R^T, the parameter packing, the INT4 nibble order,
the dequant rounding, per-expert adapters, SwiGLU, un-renormalised combine
weights) are "parity unpinned" by the pages: they are fixed by the tests only
as this library's stated convention.
"""
from . import codec, dense, moe, policy  # noqa: F401
