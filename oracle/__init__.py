"""CPU oracle for FP4 microscaling block quantization with block-scale search.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code,
tables or constants with the HIP library; each side builds its own from the
definitions.

It is deliberately plain and slow: numpy float32 arrays where the method is
defined on FP32 values (each float32 operation one IEEE-754 round-to-nearest
step; the per-block loss is an in-order chain of fused multiply-adds,
emulated exactly), float64 or exact integer arithmetic elsewhere.

Sources (web pages; cited by title and section in each module):
"Resumo Técnico: ScaleSweep", "Bridging the Gap Between Promise and
Performance for Microscaling FP4 Quantization", "Resumo Técnico: TORQ" and
"FOCUS: FP4 Optimization via Coupled-Relaxation and Dual-Granularity
Scaling".

Modules: ``formats`` (E2M1 / E4M3 / E8M0 and rounding), ``quant`` (NVFP4
ScaleSweep, MXFP4 exponent sweep, dequantization), ``hadamard`` (block
rotation), ``study`` (float64 exhaustive sweeps that pin the lemmas),
``focus`` (FOCUS forward quantizer), ``gptq`` (GPTQ with sweep-chosen group
scales), ``gemm`` (W4A4 products in float64).  Import them directly.

Parity-unpinned (no value on the pages fixes them): the FP32 evaluation
order of the per-candidate loss and the reciprocal-multiply form
y = u * fp32(1/V); the tests pin everything around them.
"""
