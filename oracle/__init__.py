"""CPU oracle for the sigmoid-routed MoE layer.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously correct
numpy implementation of what the layer computes. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the HIP
library and its Python binding never do, and the oracle imports nothing from
them (it shares no code with the GPU path).

Pages cited (by title):
  [TE-DSV3]   "[PyTorch] DeepSeekV3Layer: full MoE transformer layer
              (MLA + DeepSeek MoE)" — the method: sigmoid router with
              aux-loss-free bias and grouped top-k, GroupedLinear ->
              ScaledSwiGLU -> GroupedLinear experts, optional shared expert,
              expert-major permute with zero padding, MXFP8 recipe.
  [SGL-NVFP4] "Mistral Large 3 NVFP4 TRTLLM MoE support" — 4-bit W4A4 MoE,
              fc1 weight holding the w1 (gate) and w3 (up) halves.
  [AIC-DSV4]  "[Support Matrix] DeepSeek-V4 support on trtllm ..." — the two
              DeepSeek-V4 expert geometries.

Modules: routing (router GEMM, sigmoid, grouped top-k, combine weights),
permute (maps, gather, summing un-permute), mx (MX quantizer), mlp (expert
MLP, combine, layer forward), backward (routed expert backward),
router_train (router backward, sequence-wise balance loss, bias update), zipf
(the calibration that writes the skewed config's stored bias).

Parity pins: every function here is checked in tests/test_oracle_*.py
against brute force, closed forms, invariants or library routines; see those
files' docstrings. The pages print no worked numeric example, so no value is
pinned to the pages themselves.
"""
from . import mx, routing, permute, mlp, backward, router_train  # noqa: F401
