"""CPU oracle for blockwise W8A8 FP8 quantization and block-scaled GEMMs.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The product library (``fp8_blockwise_quantized_quantize_amd``)
never imports it and has no CPU fallback.

The oracle is a plain, slow, obviously-correct restatement of what the method
computes, written from these pages:

* "FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
  Learning" (paper-graph-ui summary page; cited below as [FP8-RL summary]):
  §3.4.1 "Blockwise FP8 Quantization for Linear Layers" (E4M3 format, the
  128x128 weight blocks, the quantization formula W^ = round(W / scale), the
  scale chosen so the block maximum maps to the FP8 maximum 448, the 1x128
  activation tiles, "Static vs. Dynamic Quantization") and §3.4.2 "Dynamic
  Weight Synchronization Pipeline" (Phase 2 step 2: block amax -> scale ->
  divide -> round to nearest E4M3; Phase 3: FP32 accumulation, then a
  conversion back to BF16).
* "How FP8 Reinforcement Learning Accelerates LLMs Without Crashing"
  (in5seconds news page), section "End-to-End Precision Recipes Across
  Generation and Training Engines": [128, 128] and [1, 128] block scaling.
* The E4M3 bit layout is the one of "FP8 Formats for Deep Learning", the
  format reference the FP8-RL pages build on (1 sign, 4 exponent bits with
  bias 7, 3 mantissa bits; no infinities; S.1111.111 is NaN; max 448).

Modules
-------
``e4m3``   encode/decode of the E4M3 ("e4m3fn") code points.
``bf16``   BF16 bit patterns <-> float, and round-to-nearest-even into BF16.
``quant``  per-tile amax -> scale -> divide -> round; 128x128 weight blocks
           and 1x128 per-token activation groups.
``gemm``   block-scaled GEMM (dequantize, exact product, one BF16 rounding),
           its FP32-accumulated form and its ragged grouped (MoE) form.
``moe``    MoE expert-FFN glue: pairs sorted by expert, gathered FP8 rows,
           SiLU(gate) * up -> BF16 -> 1x128 groups, the weighted combine.
``kv``     FP8 KV cache: per-step K/V scale calibration, quantizing cache
           write into token slots ([FP8-RL summary] §3.4.4).
``train``  FP8 training operands: W and W^T in 128x128 blocks, x in groups
           along K and x^T in groups along the tokens ([FP8-RL summary]
           §3.4.5).
``tis``    token-level importance weights of the rollout correction
           ([FP8-RL summary] §3.4.3): TIS clipping and MIS masking.

Precision readings (the pages leave these open; each is pinned by a test in
``tests/test_oracle_*.py``):

* scale ``s = fl32(amax / 448)`` (IEEE float32 division), stored as float32;
* quotient ``fl32(x / s)`` (IEEE float32 division, denormals kept), then one
  round-to-nearest-even into E4M3 with saturation at +-448;
* an all-zero tile has ``s = 0`` and every code is the sign of its zero;
* the GEMM output is the exact dot product of the dequantized operands
  (evaluated in float64) rounded once to BF16.

Every function here is pinned by tests against hand-computed values, brute
force, closed forms and invariants; none is marked "parity unpinned".
"""

from .e4m3 import E4M3_MAX, decode_e4m3, encode_e4m3, e4m3_finite_magnitudes
from .bf16 import bf16_bits_to_f32, round_to_bf16_bits, bf16_bits_to_f64
from .quant import (
    BLOCK,
    quantize_tiles,
    quant_weight_blockwise,
    quant_weight_block,
    quant_act_per_token_group,
    act_fragment_order,
)
from .gemm import (
    dequant_act,
    dequant_weight,
    gemm_ref,
    gemm_ref_bf16,
    gemm_ref_fp32,
    grouped_gemm_ref,
)
from .tis import importance_weights
from .train import quant_weight_blockwise_dual, quant_act_dual
from .kv import kv_calibrate, kv_quantize, kv_cache_write
from .moe import sort_by_expert, gather_quantize_act, silu_mul_bf16, silu_mul_quantize, combine

__all__ = [
    "E4M3_MAX",
    "decode_e4m3",
    "encode_e4m3",
    "e4m3_finite_magnitudes",
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "round_to_bf16_bits",
    "BLOCK",
    "quantize_tiles",
    "quant_weight_blockwise",
    "quant_weight_block",
    "quant_act_per_token_group",
    "dequant_act",
    "dequant_weight",
    "gemm_ref",
    "gemm_ref_bf16",
    "gemm_ref_fp32",
    "grouped_gemm_ref",
    "importance_weights",
    "sort_by_expert",
    "gather_quantize_act",
    "silu_mul_bf16",
    "silu_mul_quantize",
    "combine",
    "kv_calibrate",
    "kv_quantize",
    "kv_cache_write",
    "quant_weight_blockwise_dual",
    "quant_act_dual",
]
