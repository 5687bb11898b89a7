"""CPU oracle for the routed-expert W4A16 grouped matmul (test infrastructure).

This package is test infrastructure, not part of the product.  Only the test
suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import it.  It is a plain, slow, float64 numpy restatement of what the
routed-expert path computes, written from these pages:

* "Running DeepSeek V4 Flash on TPU v6" (mainlymatmul.com), section
  "1. Four bits that v6e can't hold": expert-sorted token bands, the grouped
  matmul loop nest, the e2m1 code semantics and the per-32 block scale applied
  before the matmul; section "Grouped matmul performance vs bf16": the NVFP4
  variant (e2m1 codes with per-16 E4M3 block scales) and the bf16-weight
  grouped matmul it is compared with.
* "DeepSeek-V4-Flash-0731-NVFP4" (model card), section "The lossless weight
  cast": the MXFP4 -> NVFP4 power-of-two scale mapping; section
  "Verification": the -0 -> +0 canonicalisation note.
* "DeepSeek-V4-Flash" (PocketLLM docs), section "Correctness and precision":
  the expert reduction is deterministic (fixed order, no atomics).
* The gate/up activation after the fused w13 matmul, which the pages name but
  do not define: the SiLU-gated product of the two column halves (act.py).
* "DeepSeek-V4-Flash-0731-NVFP4": the W4A4 execution with 4-bit activations,
  here with MXFP4 (power-of-two block scale) activation quantization
  (quant.py).

It shares no code with the HIP path and imports nothing from it.
"""

from .formats import (  # noqa: F401
    E2M1_MAGNITUDES,
    unpack_nibbles,
    e2m1_decode,
    e8m0_decode,
    e4m3_decode,
    e4m3_encode_pow2,
    decode_mxfp4,
    decode_nvfp4,
    mxfp4_to_nvfp4,
)
from .route import route_sort  # noqa: F401
from .gmm import gmm, gmm_w4a4, gmm_sampled, dense_weights  # noqa: F401
from .quant import nearest_e2m1, quantize_mxfp4_rows, dequantize_mxfp4_rows  # noqa: F401
from .combine import combine  # noqa: F401
from .act import silu, silu_mul  # noqa: F401
