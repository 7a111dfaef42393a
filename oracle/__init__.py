"""CPU oracle for the GPT-2 decoder forward pass (TEST INFRASTRUCTURE ONLY).

This package is the slow, plain reference that the HIP path is checked
against.  Only the tests, the smoke check and the CPU-baseline leg of the
benchmark may import it; the product library never calls it and has no CPU
fallback.  It shares no code with the HIP path: the only common input is the
seeded generator in ``synth``, which holds none of the model's arithmetic.

Everything is numpy in float64 (a compute-dtype switch exists for very large
shapes), one sequence at a time, with library matrix products and sorts as
single steps and no blocking or fusion beyond what the definitions state.

Sources (the pages as a reader has them):

* serving page "原生 nanoGPT 模型服务首选": section 1 (LayerNorm with optional
  bias; a None bias and a zero bias give identical forwards), section 2
  (``generate()``: crop, last-position logits divided by temperature, top-k
  filter keeping values not below the k-th largest, softmax, multinomial
  draw, append), and the section proposing the KV cache (fused c_attn split
  into q, k, v, past K/V concatenated on the time axis, causal mask only
  when there is no past, one new token per step).
* SDK guide "极速上手nanoGPT", section "模型架构解析" (GPTConfig fields and
  defaults; the manual attention path: q kᵀ scaled by 1/sqrt(head size),
  upper triangle filled with -inf, softmax, dropout, times v).
* architecture analysis "nanoGPT 架构分析", section 4.1 (pre-LN residual
  blocks, a 4x Linear-GELU-Linear MLP, weight tying of wte and lm_head,
  lm_head on the last position only at inference).
* model-building chapter "第 4 章 模型构建", sections 4.3 (parameter count
  formula), 4.5 (token + learned absolute position embeddings, the
  lower-triangular causal mask, final LayerNorm, bias-free tied lm_head) and
  4.6 (the loss: cross-entropy of every position's logits against the next
  id, the last position dropped).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, special cases, library routines, brute force, invariants).
The absolute logits of any *trained* GPT-2 are parity unpinned: the pages
print no numeric example and no trained weights are available.
"""
from .gpt import (OracleGPT, layer_norm, gelu, linear, causal_attention,
                  softmax_rows, cross_entropy_rows, round_bf16, round_fp16, count_parameters,
                  param_count_closed_form, param_count_page_estimate)
from .sampler import sample_rows, sample_row, topk_keep_set

__all__ = [
    "OracleGPT", "layer_norm", "gelu", "linear", "causal_attention",
    "softmax_rows", "cross_entropy_rows", "round_bf16", "round_fp16", "count_parameters",
    "param_count_closed_form", "param_count_page_estimate",
    "sample_rows", "sample_row", "topk_keep_set",
]
