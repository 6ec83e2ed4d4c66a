"""CPU oracle for the W8A8 INT8 linear-layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls, links or
runs anything in this package.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may use it.
It shares no code with the HIP library (no kernels, headers, helpers, tables
or constant generators), and it never imports the HIP package.

What it computes is the plain definition of the method described on the page
"DeepSeek R1 INT8 quantisation in SGLang" (Meituan team article, page 1),
section 2.3 "Quantisation method design":

* block-wise scheme: weights quantised in 128x128 tiles, activations quantised
  online per token-group, and a dequantisation inside the INT8 matmul for every
  K block (because each block carries its own scale);
* channel-wise scheme: one weight scale per output channel, activations
  quantised online per token, one dequantisation after the INT8 matmul;
* the offline conversion FP8 -> BF16 -> INT8 of the released FP8 weights.

The symmetric INT8 quantiser itself (scale = amax/127, round, clamp to +-127)
is the one written out on the page "FP8 vs INT8 quantisation for DeepSeek"
(page 4), section 3.2.1 (the int8 branch of its QAT example).

Every float step is written in numpy with an explicit precision: fp32 where the
method fixes the arithmetic (the quantisers and the bf16 rounding), and both
an fp64 path (``y64``) and an fixed-order fp32 path (``y32``) for the GEMM
outputs.  The int8 codes, the scales and the int32 partial sums are exact.

Modules:
  formats  - bf16 / fp16 / OCP FP8-E4M3FN conversions
  quant    - the quantisers (token-group, token, 128x128 tile) and the offline
             FP8 -> BF16 -> INT8 requantisation
  gemm     - block-wise, channel-wise, W8A16 group-wise and grouped MoE GEMMs
  routing  - top-k expert routing used to lay out the grouped GEMM inputs
  asym     - the asymmetric uint8 activation variant
  int4     - group-wise INT4 weights (packed two per byte) and the W4A16 GEMM
"""

from . import formats, quant, gemm, routing, int4  # noqa: F401
