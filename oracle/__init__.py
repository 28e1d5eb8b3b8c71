"""CPU oracle for the SubSpec substitute-draft step.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow reference that the HIP
path is checked against. Only the tests, the package smoke check and the bench's
CPU-baseline leg may import it; the product path never does. It shares no code
with the HIP library or its binding.

Pages cited (by title, then section):
  [Review]   "SubSpec: Using the Target Model's Own Low-Bit Shadow as Its Draft Model"
             (tabzhangjx.github.io blog review of the SubSpec paper)
  [Summary]  "Speculate Deep and Accurate: Lossless and Training-Free Acceleration for
             Offloaded LLMs via Substitute Speculative Decoding" (atlas.scime.ai summary)
  [Abstract] the arXiv abstract of the same paper on its mlsanity.com page

Precision: integer and bit operations are exact; steps whose result must match the
kernels bit for bit (quantize, dequantize, draft selection) run in IEEE fp32 with
one rounding per operation and no fused multiply-add, as NumPy float32 arithmetic
does; every float reference (matmul, attention, layer) runs in fp64.

Parity pins: every function is pinned by the CPU tests in tests/test_oracle_*.py
against brute force, closed forms, special cases and library routines. The
whole-stack composition (`stack64`) is pinned by zero-projection layers (the stack
reduces to embedding, final norm and head) and by an independent float64
implementation with torch primitives (complex-rotation RoPE, parent-walk tree mask,
masked scaled-dot-product attention) over three non-trivial layers with distinct
caches.
"""

from .fp import bf16_to_f32, bf16_to_f64, f32_to_bf16  # noqa: F401
from .quant import quantize, pack_int4, unpack_int4, dequantize_f16, dequant_exact64  # noqa: F401
from .linalg import matmul64, w4a16_matmul64  # noqa: F401
from .tree import validate_tree, tree_mask, tree_depth, accept, kv_commit  # noqa: F401
from .attention import tree_attention64, tree_attention_loop64  # noqa: F401
from .layer import rmsnorm64, rope64, silu64, swiglu64, layer64, stack64  # noqa: F401
from .select import row_argmax, draft_select  # noqa: F401
