"""Blockwise / groupwise FP8 quantization: amax -> scale -> divide -> round.

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ([FP8-RL summary] §3.4.1, the formula for W^, and §3.4.2
Phase 2 step 2):

    for every tile T (a 128x128 weight block, or a 1x128 activation group):
        amax_T = max |x| over the in-bounds elements of T
        s_T    = fl32(amax_T / 448)          (largest |x| maps to the E4M3 max)
        q[i]   = E4M3_RNE_sat( fl32(x[i] / s_T) )

Readings of what the pages leave open:

* the scale is stored in float32 (the pages say "FP8 scales" in one place;
  an FP8 scale could not hold amax/448 for small blocks, and the task
  statement fixes one FP32 scale per block);
* the divisor is exactly 448.0, no epsilon and no power-of-two rounding;
* the quotient is the IEEE float32 quotient (numpy's float32 division is
  correctly rounded and keeps denormals), then one rounding into E4M3;
* amax == 0 (all-zero tile): s = 0 and each code is the sign of its zero
  (0x00 for +0, 0x80 for -0), which is what x / s gives for any s > 0;
* tiles are aligned at (0, 0); edge tiles of a dimension that is not a
  multiple of 128 are partial and their amax covers the in-bounds
  elements only;
* weights are laid out [N][K] (out x in), activations [M][K]; activation
  groups are 128 consecutive K elements of one token (the "1 x 128 tiles"
  of §3.4.1); activation scales are [M][ceil(K/128)], weight scales
  [ceil(N/128)][ceil(K/128)].
* inputs must be finite.
"""

import numpy as np

from .bf16 import bf16_bits_to_f32
from .e4m3 import E4M3_MAX, encode_e4m3

BLOCK = 128


def quantize_tiles(tiles):
    """Quantize each row of a 2-D float32 array as one tile.

    Returns ``(codes uint8 [T][L], scales float32 [T])``.  This single
    function is the definition shared by the weight and activation paths.
    """
    x = np.asarray(tiles, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("quantize_tiles expects [tiles][elements]")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the contract")
    t, n = x.shape
    if n == 0:
        return np.zeros((t, 0), np.uint8), np.zeros((t,), np.float32)
    amax = np.max(np.abs(x), axis=1)  # exact
    scale = amax / np.float32(E4M3_MAX)  # float32 / float32 -> IEEE float32
    assert scale.dtype == np.float32
    codes = np.empty(x.shape, np.uint8)
    zero = amax == 0
    if np.any(zero):
        codes[zero] = np.where(np.signbit(x[zero]), 0x80, 0x00).astype(np.uint8)
    nz = ~zero
    if np.any(nz):
        with np.errstate(over="raise", invalid="raise", divide="raise"):
            q = x[nz] / scale[nz][:, None]  # IEEE float32 quotient
        assert q.dtype == np.float32
        codes[nz] = encode_e4m3(q)
    return codes, scale


def quant_weight_block(block_bits):
    """Quantize one (possibly partial) weight block given as BF16 bits [r][c]."""
    x = bf16_bits_to_f32(block_bits)
    r, c = x.shape
    codes, scale = quantize_tiles(x.reshape(1, r * c))
    return codes.reshape(r, c), scale[0]


def quant_weight_blockwise(w_bits):
    """128x128 blockwise quantization of BF16 weights.

    ``w_bits``: uint16 BF16 bit patterns, shape [N][K] or [B][N][K].
    Returns ``(codes uint8, same shape; scales float32 [..][ceil(N/128)][ceil(K/128)])``.
    """
    w = np.asarray(w_bits, dtype=np.uint16)
    squeeze = w.ndim == 2
    if squeeze:
        w = w[None]
    if w.ndim != 3:
        raise ValueError("weights must be [N][K] or [B][N][K]")
    b, n, k = w.shape
    nb, kb = -(-n // BLOCK), -(-k // BLOCK)
    if n % BLOCK == 0 and k % BLOCK == 0:
        # All blocks are full: gather each block's 16384 elements into one row
        # and hand all blocks to the tile definition at once (same result as
        # the block loop below, which handles partial edge blocks).
        x = bf16_bits_to_f32(w).reshape(b, nb, BLOCK, kb, BLOCK).transpose(0, 1, 3, 2, 4)
        q, s = quantize_tiles(x.reshape(b * nb * kb, BLOCK * BLOCK))
        codes = q.reshape(b, nb, kb, BLOCK, BLOCK).transpose(0, 1, 3, 2, 4).reshape(b, n, k)
        scales = s.reshape(b, nb, kb)
        return (codes[0], scales[0]) if squeeze else (np.ascontiguousarray(codes), scales)
    codes = np.empty(w.shape, np.uint8)
    scales = np.zeros((b, nb, kb), np.float32)
    for l in range(b):
        for i in range(nb):
            rows = slice(i * BLOCK, min(n, (i + 1) * BLOCK))
            for j in range(kb):
                cols = slice(j * BLOCK, min(k, (j + 1) * BLOCK))
                q, s = quant_weight_block(w[l, rows, cols])
                codes[l, rows, cols] = q
                scales[l, i, j] = s
    if squeeze:
        return codes[0], scales[0]
    return codes, scales


def quant_act_per_token_group(x_bits):
    """Per-token 1x128 group quantization of BF16 activations [M][K].

    Returns ``(codes uint8 [M][K], scales float32 [M][ceil(K/128)])``.
    Each (token, group) pair is one tile; the tiles of one group column are
    handed to ``quantize_tiles`` together (one tile per row).
    """
    x = bf16_bits_to_f32(np.asarray(x_bits, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("activations must be [M][K]")
    m, k = x.shape
    g = -(-k // BLOCK)
    codes = np.empty((m, k), np.uint8)
    scales = np.zeros((m, g), np.float32)
    for j in range(g):
        cols = slice(j * BLOCK, min(k, (j + 1) * BLOCK))
        q, s = quantize_tiles(x[:, cols])
        codes[:, cols] = q
        scales[:, j] = s
    return codes, scales


def act_fragment_order(codes):
    """Byte order of codes [R][K] (R % 16 == 0, K % 128 == 0) as the
    16x16x128 FP8 MFMA reads an operand: per 16-row group and 128-wide
    K-block one 2 KB block; in it, lane l = 16 c + r (r = row within the
    group, c = 0..3) holds bytes 16 c .. 16 c + 15 of its row's K-block at
    l * 16 and bytes 64 + 16 c .. 79 + 16 c at 1024 + l * 16.  The same order
    serves activations [M][K] and weights [N][K] (both operands are read in
    this form).  A pure permutation of the row-major codes (what the
    block-scaled GEMM computes is unchanged; the pages leave the byte layout
    of the quantized operands open).
    """
    q = np.asarray(codes, np.uint8)
    m, k = q.shape
    if m % 16 or k % BLOCK:
        raise ValueError("fragment order needs M % 16 == 0 and K % 128 == 0")
    # axes: row group, row in group, K-block, half, 16-byte chunk c, byte
    t = q.reshape(m // 16, 16, k // BLOCK, 2, 4, 16)
    return np.ascontiguousarray(t.transpose(0, 2, 3, 4, 1, 5)).reshape(m, k)
