"""Seeded synthetic inputs for the blockwise W8A8 FP8 path.

This module produces input bytes only (BF16 bit patterns, routing offsets);
it holds none of the method's arithmetic and imports neither the oracle nor
the product library, so both sides can read the same inputs from it.

The real workloads of the FP8-RL pages (Qwen3-8B-Base and Qwen3-30B-A3B-Base
rollouts on DAPO prompts) are not available; seeded Gaussian tensors with
those models' linear-layer shapes stand in for them:

* weights  W = bf16(0.02 * z),  z ~ N(0, 1)
* activations X = bf16(z * c_col): most columns c = 1, a few "outlier
  channels" (whole K columns) multiplied by a constant
* MoE routing: logits ~ N(0, 1) [tokens][experts] -> float32 softmax ->
  top-k experts per token (ties to the lower expert index) -> (expert,
  token) pairs sorted by expert then token -> ragged row offsets;
  ``moe_topk`` gives the same top-k ids per token and their probabilities
  renormalized over the k chosen experts (the combine weights).
* rollout batches for the importance weights: padded [responses][max_len]
  log-probabilities of sampled tokens under the rollout and training
  policies, a response mask and per-response advantages
  (``rollout_batch``; see its docstring for the distributions).

Host tensors use numpy's PCG64 (``default_rng([config, tensor, layer])``)
and torch's CPU BF16 conversion (round to nearest even).  Very large
tensors can be drawn directly on a GPU with torch's seeded generator
(``device_bf16_normal``); tests then copy the sampled parts they check back
to the host.
"""

from .gen import (
    LAYER_SHAPES_QWEN3_8B,
    MOE_QWEN3_30B_A3B,
    bf16_normal,
    activations,
    moe_routing,
    moe_topk,
    gather_rows,
    device_bf16_normal,
    device_activations,
    f32_to_bf16_bits,
    ROLLOUT_TRAIN_BATCH,
    rollout_batch,
)

__all__ = [
    "LAYER_SHAPES_QWEN3_8B",
    "MOE_QWEN3_30B_A3B",
    "bf16_normal",
    "activations",
    "moe_routing",
    "moe_topk",
    "gather_rows",
    "device_bf16_normal",
    "device_activations",
    "f32_to_bf16_bits",
    "ROLLOUT_TRAIN_BATCH",
    "rollout_batch",
]
