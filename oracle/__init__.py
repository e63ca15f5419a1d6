"""CPU oracle for the quantized linear layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct implementation of what the HIP path
computes, written from the pages in numpy (fp32 where the method rounds in
fp32, fp64 for products and statistics). It shares no code with the HIP path
and must only be imported by the tests, by the smoke check and by the CPU
baseline leg of the benchmark; the product path never calls it.

Sources (cited by page title and section):
  * "SNIP: An Adaptive Mixed Precision Framework for Subbyte LLM Training"
    -- Abstract (statistics of activations and gradients, per-layer FP8/FP4
    GEMM precision), Fig. 4 (the seven linear layers), Fig. 5 (forward and
    backward of a quantized linear layer).
  * "FP4 All the Way" summary page -- Outline (NVFP4: blocks of 16 E2M1
    values sharing one E4M3 scale; round-to-nearest in the forward pass,
    stochastic rounding in back-propagation and update; sqrt(3) threshold).
  * "Research on Mixed-Precision Training for LLMs" -- Core Techniques
    section (stochastic rounding rounds up or down by proximity and keeps the
    expected value).

Readings of points the pages leave open are listed in each module and in the
design notes of the repository. Parity status per function:
  formats.*        pinned (value tables, exhaustive nearest search, torch fp8)
  philox.*         pinned (rocRAND header engine, independent C++ build)
  quantize.*       pinned (round trips, closed-form scales, SR expectation)
  gemm.*           pinned (exact rational dot products, representable inputs)
  linear.*         pinned through quantize.* and gemm.* plus consistency tests
"""
from . import formats, philox, quantize, gemm, linear  # noqa: F401
