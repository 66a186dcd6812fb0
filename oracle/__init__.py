"""CPU oracle for FP4 microscaling block quantization with block-scale search.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables or constants with the HIP library; each side builds its own from the
definitions.

It is deliberately plain and slow: numpy float32 arrays where the method is
defined on FP32 values (every float32 operation below is a single IEEE-754
round-to-nearest-even operation, no fused multiply-add), float64 or exact
integer arithmetic elsewhere.

Sources (web pages; cited by title and section):
  * "Resumo Técnico: ScaleSweep" -- NVFP4 two-level scaling, the global scale
    S = max|x|/(256*6), the MSE / WMSE objectives, Lemma 4.1 / Lemma 4.3 and
    the bit-pattern windows [-3,+7] (MSE) and [-8,+7] (WMSE).
  * "Bridging the Gap Between Promise and Performance for Microscaling FP4
    Quantization" (MR-GPTQ) -- MXFP4 with power-of-two E8M0 scales, block
    Hadamard micro-rotation, MSE-optimised scale grid.
  * "Resumo Técnico: TORQ" -- MXFP4 activations, the S-step that maps the
    block maximum onto the largest code.
  * "FOCUS: FP4 Optimization via Coupled-Relaxation and Dual-Granularity
    Scaling" -- block sizes 16 (NVFP4) and 32 (MXFP4); only FP4 codes plus
    the dequantization scale are stored.

Modules
  formats   E2M1 / E4M3 / E8M0 tables and round-to-nearest-even
  quant     NVFP4 ScaleSweep and MXFP4 exponent sweep, dequantization
  hadamard  block Hadamard rotation (fast transform and dense reference)
  study     float64 exhaustive-sweep tools used to pin the lemmas
  focus     FOCUS forward quantizer with coupled-relaxation coefficients
  gptq      GPTQ with sweep-chosen NVFP4 group scales
  gemm      W4A4 matrix product of MXFP4 / NVFP4 operands (float64)

Parity-unpinned items (no value printed on the pages fixes them): the FP32
evaluation order of the per-candidate loss (terms summed in element order
with one rounding each, a fused multiply-add) and the reciprocal-multiply
form y = u * fp32(1/V).  They are this oracle's canonical reading; the tests
pin everything around them (the float32 FMA emulation against exact
rational arithmetic).
"""

from . import formats, quant, hadamard, study, focus, gptq, gemm  # noqa: F401
from .quant import (  # noqa: F401
    quantize_nvfp4,
    quantize_mxfp4,
    dequantize_nvfp4,
    dequantize_mxfp4,
    NVFP4Result,
    MXFP4Result,
)
from .hadamard import block_hadamard, block_hadamard_dense64  # noqa: F401
