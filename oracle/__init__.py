"""CPU oracle for the block-quantized GEMV path (test infrastructure).

What this package is
--------------------
A plain, slow, obviously correct CPU implementation of everything the GPU path
computes, in fp64 numpy.  It exists only to check the GPU path: the test suite,
the smoke check and the CPU-baseline leg of the benchmark call it; the product
library never imports, links or runs anything in here, and nothing in here
imports the product package.  The two sides share only the seeded input
generators (``synth``), which hold none of the method's arithmetic.

What the source pages fix, and what they leave open
---------------------------------------------------
The pages (the LumenLLM README, the Lumen landing page, the bw24 README and the
memra README) describe inference engines whose decode step is a matrix-vector
product over block-quantized weights with the dequantization fused into the
weight load: NVFP4 (LumenLLM README, feature list "Quantization"; bw24 README,
feature list "NVFP4 (W4) decode path"), Q4_0 / Q8_0 (memra README, feature list
"Decode kernels"; Lumen page, "Format" section, per-tensor quantization), the
W4A8 integer dot path (bw24 README, "NVFP4 (W4) decode path": dp4a and the int8
W4A8 GEMM), expert-major MoE batching (bw24 README, feature list "MoE on 24 GB")
and a grouped-MoE prefill/verify GEMM (LumenLLM README, roadmap).  Their
principle for correctness is "every quant kernel against a CPU reference" (bw24
and memra READMEs, the kernel-check gate).

The pages give no bit layouts and no formulas.  The format definitions used
here are the public ones:

* E2M1 and E4M3 bit fields: OCP Microscaling Formats (MX) v1.0 and OCP 8-bit
  Floating Point (OFP8) v1.0 ("E4M3", the variant without infinities).
* NVFP4: 16-element blocks of E2M1 codes, one E4M3 scale per block, one fp32
  scale per tensor; value = e2m1(code) * e4m3(block scale) * tensor scale.
* Q8_0: 32-element blocks of int8 codes with one fp16 scale; value = d * q.
* Q4_0: 32-element blocks of 4-bit codes with one fp16 scale; value = d*(q-8).
* FP8: E4M3 codes with fp32 scales per tensor or per 128 x 128 tile.
* K-quants (Q4_K, Q5_K, Q6_K) and IQ4_XS: 256-element super-blocks with fp16
  scales and 6-bit or int8 sub-block scales (the GGUF definitions, stated on
  logical values in ``ops.py``).  The pages name these formats but define
  none of them; the IQ4_XS codebook values are pinned only by their own
  fixture (parity unpinned for the codebook).

Every reading taken where the pages are silent is listed in the repository's
design notes and in the docstring of the function that takes it.

Pins
----
``tests/test_oracle_*.py`` (CPU only) pin each function to something other
than itself: library decoders (torch float8_e4m3fn, numpy float16), the OCP
E2M1 value table, hand-worked one-block examples (``tests/golden/``), exact
``fractions.Fraction`` brute force on tiny shapes, closed forms and invariants.
"""

from .formats import (  # noqa: F401
    decode_bf16,
    decode_e2m1,
    decode_e4m3,
    decode_f16,
    round_to_bf16,
    bf16_ulp,
)
from .ops import (  # noqa: F401
    dequant_nvfp4,
    dequant_nvfp4_f32,
    dequant_q4_0,
    dequant_q8_0,
    gemv,
    gemv_abs,
    quantize_q8_0_act,
    gemv_q4_0_a8,
    gemv_q4_0_a8_abs,
    dequant_q4_k,
    dequant_q6_k,
    dequant_iq4_xs,
    act_q8_0_values,
    gemv_a8,
    gemv_a8_abs,
    block_isums_q4_0_a8,
    route_topk,
    group_by_expert,
    silu,
    swiglu,
    swiglu_bf16,
    moe_forward,
    prefill,
    tolerance,
)
