"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws random numbers and stores them in the layouts the two
sides consume (bf16 bit patterns or fp32, paper orientation).  It holds none
of the method's arithmetic: no quantisation, no masks, no projections.

Workloads follow the shapes and distributions the Prox pages describe:
  * SwiGLU FFN shapes of Qwen3-8B (d_model 4096, d_ff 12288) and Qwen3-32B
    (5120, 25600) plus a tiny fp32 layer (256, 768);
  * i.i.d. Gaussian weights (the pages use trained checkpoints, which are not
    available; Gaussian weights stand in for them);
  * Laplace(0, 1) FFN inputs, because the deep-dive blog (section on why the
    SwiGLU intermediate state is the natural signal) and the paper's Fig. 3(b)
    describe the activations as peaked and heavy-tailed, Laplace-like;
  * a small set of fixed outlier coordinates per layer, scaled up, standing in
    for the massive activations of real LLM residual streams.
"""
from .gen import (LayerConfig, Layer, CONFIGS, make_layer, make_tokens,
                  bf16_bits_from_f32, f32_from_bf16_bits, as_f64)

__all__ = ["LayerConfig", "Layer", "CONFIGS", "make_layer", "make_tokens",
           "bf16_bits_from_f32", "f32_from_bf16_bits", "as_f64"]
