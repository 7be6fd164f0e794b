"""CPU oracle for the sparse MoE layer — TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The HIP
library never routes through it and shares no code with it: no kernels,
headers, tables, constants or pre/post-processing.  Inputs come from the
seeded generators in ``synth`` (which hold none of the layer's arithmetic).

What it computes (the FreeToken pages describe the method; they print no
formula for it, so each step is the plain textbook definition named in its
docstring):
  * router logits, top-k routing with softmax weights   (formats: none)
  * the token -> expert permutation (stable counting sort)
  * the expert-id -> slot LRU lookup shared across layers
  * dequantisation of MXFP4 / NVFP4 / BF16 expert weights
  * the SwiGLU expert FFN, per expert, looping per token
  * the weighted combine back to token order
  * (FP4-MFMA prefill mode) the MXFP4 activation quantiser

Precision: floating point is evaluated in float64 (exact dequantised weights,
float64 dot products); decisions that the kernels take in float32 (top-k keys,
the MXFP4 encoding of the intermediate activation) are taken on float32 values.

Parity status: every public function is pinned by ``tests/test_oracle_*.py``
against closed forms, torch's independent float4/float8 dtypes, brute force on
tiny inputs or invariants.  Nothing here is "parity unpinned" except the
throughput figures, which are not computed here.
"""
from . import formats, lru, moe, quant  # noqa: F401
