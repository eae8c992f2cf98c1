"""Quantization for FP8 training (forward, dgrad and wgrad operands).

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ([FP8-RL summary] §3.4.5 "End-to-End FP8 RL (Training +
Rollout)": the trainer also runs its forward and backward GEMMs in FP8,
with the blockwise recipe of §3.4.1):

* forward  y  = x W^T       x in 1x128 groups along K, W in 128x128 blocks;
* dgrad    dx = dy W        dy in 1x128 groups along N, W^T ([K][N]) in
                            128x128 blocks;
* wgrad    dW = dy^T x      dy^T ([N][M]) and x^T ([K][M]) in 1x128 groups
                            along the token axis M.

Readings of what the pages leave open (they give no backward recipe):

* Every operand is quantized with the rule of §3.4.1 in the layout its GEMM
  reduces over: a [rows][cols] matrix in 1x128 groups along cols, or in
  128x128 blocks.  The transposed operands are therefore the plain
  definitions applied to the transposed BF16 matrix.
* W^T's 128x128 blocks are W's blocks transposed, so its codes and scales
  are W's, transposed (pinned in ``tests/test_oracle_train.py``).
"""

import numpy as np

from .quant import quant_act_per_token_group, quant_weight_blockwise


def quant_weight_blockwise_dual(w_bits):
    """W [N][K] (or [B][N][K]) -> ((codes, scales) of W, (codes, scales) of W^T)."""
    w = np.asarray(w_bits, dtype=np.uint16)
    wt = np.ascontiguousarray(np.swapaxes(w, -1, -2))
    return quant_weight_blockwise(w), quant_weight_blockwise(wt)


def quant_act_dual(x_bits):
    """x [M][K] -> ((codes [M][K], scales [M][ceil(K/128)]) in groups along K,
    (codes [K][M], scales [K][ceil(M/128)]) of x^T in groups along M)."""
    x = np.asarray(x_bits, dtype=np.uint16)
    return quant_act_per_token_group(x), quant_act_per_token_group(np.ascontiguousarray(x.T))
