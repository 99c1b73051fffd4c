"""CPU oracle for the MXFP8 routed-experts SwiGLU MLP.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain, obviously-correct
reference that the HIP path is checked against. Only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. The product path (``mxfp8_mixed_precision_amd``) never imports,
links or calls anything here, and this package shares no code, tables or
constants with it.

Arithmetic is numpy in fp64 (exact for every quantity that has an exact
definition) plus integer arithmetic on bit patterns.

Sources, cited by page title and section:
  * afd-plugin PR #475 "quantize the A2E FFN transport to MXFP8" -- sections
    "Purpose" and "Implementation Notes" (E4M3 elements carrying an E8M0 block
    scale), "Test Plan" (the 32-element group), the second review (E8M0 bytes
    127/128/126 decode to 1.0/2.0/0.5) and the third review (E8M0 byte 0x00 is
    2^-127, not zero; 0xFF is NaN; an E4M3 16 under byte 0 restores to 2^-123).
  * torchtitan PR #12 "Wire the fully-fused grouped-GEMM MXFP8 plan behind
    fusion_plan" -- section "What it adds" (the four fused ops: FC1 grouped GEMM
    + SwiGLU + dual MXFP8 quantization, FC2 GEMM, fused dSwiGLU backward,
    wgrad; packed [E, 2F, D] weights in 32-block order; stock parameters;
    pad_multiple 256 per-expert alignment) and "Evidence" (zero-token experts
    get exact-zero gradients; NaN-poisoned tail negative control).
  * torchtitan PR #2 "[mxfp8 training] fused gated-activation (SwiGLU) + MXFP8
    quantization kernel override" -- sections "Summary" (w13 GEMM -> fused SwiGLU
    + dual MXFP8 quantization -> w2 GEMM; BF16 post-activation never
    materialised) and "Numerics and tests" (bitwise forward parity with
    standalone-cast quantization).
  * The quantization rule itself (scale exponent floor(log2 amax) - 8, clamped;
    E4M3 round-to-nearest-even saturating at +-448) is the OCP Microscaling
    Formats (MX) v1.0 specification's MXFP8 rule; the pages name the formats
    but do not spell the rule out.

Every function here is pinned by a ``-m "not gpu"`` test against closed forms,
worked values printed on the pages, brute force or finite differences; see
``tests/test_oracle_*.py``.
"""
