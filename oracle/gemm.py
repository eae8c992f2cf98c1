"""Block-scaled W8A8 GEMM and its ragged grouped (MoE expert) form.

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ([FP8-RL summary] §3.4.1 "Static vs. Dynamic
Quantization" and §3.4.2 Phase 3): the FP8 weights and the dynamically
quantized FP8 activations are multiplied, the products are accumulated in
FP32 and the result is converted back to BF16.  Mathematically the layer
output is the product of the two dequantized operands:

    A~[m,k] = dec(qa[m,k]) * sa[m, k//128]            (1x128 groups)
    W~[n,k] = dec(qw[n,k]) * sw[n//128, k//128]       (128x128 blocks)
    y[m,n]  = sum_k A~[m,k] * W~[n,k]                 (y = A~ W~^T)
    out     = BF16_RNE(y)

The oracle evaluates this definition directly in float64 (the dequantized
operands are exact in float64: a float32 scale times a 4-bit significand)
with one library matmul, and rounds once into BF16.  The summation order of
a real kernel is free, so GPU results are compared with a tolerance.

``gemm_ref_fp32`` is the same product evaluated with FP32 accumulation, as
§3.4.2 Phase 3 describes the arithmetic: per 128-wide K-block the float32
product of the decoded codes, times the two block scales, added into a
float32 accumulator.  It is the fast form used for CPU timing; its distance
from the exact value is bounded by float32 rounding (pinned in the tests).

MoE expert layers (fc1/fc2, §3.4.1 "Quantization Scope") use the same
scheme per expert: expert e owns rows [off[e], off[e+1]) of the stacked
activations and its own weight and scale grid.
"""

import numpy as np

from .bf16 import round_to_bf16_bits
from .e4m3 import decode_e4m3
from .quant import BLOCK


def _check_k(k):
    if k % BLOCK:
        raise ValueError("GEMM K must be a multiple of 128")


def dequant_act(codes, scales):
    """A~ = dec(q) * s_a[m, k//128] in float64, [M][K]."""
    q = np.asarray(codes, np.uint8)
    s = np.asarray(scales, np.float32).astype(np.float64)
    m, k = q.shape
    if s.shape != (m, -(-k // BLOCK)):
        raise ValueError("activation scales must be [M][ceil(K/128)]")
    group = np.arange(k) // BLOCK
    return decode_e4m3(q) * s[:, group]


def dequant_weight(codes, scales, rows=None):
    """W~ = dec(q) * s_w[n//128, k//128] in float64, [N][K] (or the given rows)."""
    q = np.asarray(codes, np.uint8)
    s = np.asarray(scales, np.float32).astype(np.float64)
    n, k = q.shape
    if s.shape != (-(-n // BLOCK), -(-k // BLOCK)):
        raise ValueError("weight scales must be [ceil(N/128)][ceil(K/128)]")
    r = np.arange(n) if rows is None else np.asarray(rows)
    group = np.arange(k) // BLOCK
    return decode_e4m3(q[r]) * s[(r // BLOCK)[:, None], group[None, :]]


def gemm_ref(a_codes, a_scales, w_codes, w_scales, rows=None, cols=None):
    """y = A~ W~^T in float64 (before the BF16 rounding).

    ``rows`` / ``cols`` restrict the computation to a sub-grid of outputs
    (used to check full-size problems on sampled entries).
    """
    qa = np.asarray(a_codes, np.uint8)
    _check_k(qa.shape[1])
    r = np.arange(qa.shape[0]) if rows is None else np.asarray(rows)
    a = dequant_act(qa[r], np.asarray(a_scales)[r])
    w = dequant_weight(w_codes, w_scales, rows=cols)
    return a @ w.T


def gemm_ref_bf16(a_codes, a_scales, w_codes, w_scales, rows=None, cols=None):
    """BF16 bit patterns of the GEMM output (one RNE rounding of the float64 result)."""
    return round_to_bf16_bits(gemm_ref(a_codes, a_scales, w_codes, w_scales, rows, cols))


def gemm_ref_fp32(a_codes, a_scales, w_codes, w_scales, rows=None):
    """y = sum_kb (s_a[m,kb] * s_w[n//128,kb]) * P_kb[m,n] with float32 arithmetic.

    P_kb is the float32 product of the decoded (unscaled) codes of K-block kb
    (one library matmul per K-block; the decoded codes are exact in float32),
    the scale product is a float32 multiply, and the K-blocks are summed in a
    float32 accumulator in K order.  ``rows`` restricts the output to those
    activation rows.  Returns float32 [M][N] (before the BF16 rounding).
    """
    qa = np.asarray(a_codes, np.uint8)
    qw = np.asarray(w_codes, np.uint8)
    m_all, k = qa.shape
    n = qw.shape[0]
    _check_k(k)
    r = np.arange(m_all) if rows is None else np.asarray(rows)
    sa = np.asarray(a_scales, np.float32)[r]
    sw = np.asarray(w_scales, np.float32)
    if sa.shape != (len(r), k // BLOCK) or sw.shape != (-(-n // BLOCK), k // BLOCK):
        raise ValueError("scales must be [M][K/128] and [ceil(N/128)][K/128]")
    da = decode_e4m3(qa[r]).astype(np.float32)
    dw = decode_e4m3(qw).astype(np.float32)
    block_of_n = np.arange(n) // BLOCK
    y = np.zeros((len(r), n), np.float32)
    for kb in range(k // BLOCK):
        cols = slice(kb * BLOCK, (kb + 1) * BLOCK)
        p = da[:, cols] @ dw[:, cols].T
        c = sa[:, kb][:, None] * sw[block_of_n, kb][None, :]
        y += p * c
    return y


def grouped_gemm_ref(a_codes, a_scales, w_codes, w_scales, offsets):
    """Ragged grouped GEMM: rows [off[e], off[e+1]) use expert e's weights.

    ``w_codes`` [G][N][K], ``w_scales`` [G][ceil(N/128)][K/128], ``offsets``
    [G+1] non-decreasing with offsets[0] == 0 and offsets[G] == M.
    Returns float64 [M][N].
    """
    qa = np.asarray(a_codes, np.uint8)
    sa = np.asarray(a_scales)
    qw = np.asarray(w_codes, np.uint8)
    sw = np.asarray(w_scales)
    off = np.asarray(offsets, np.int64)
    g, n, k = qw.shape
    m = qa.shape[0]
    _check_k(k)
    if off.shape != (g + 1,) or off[0] != 0 or off[-1] != m or np.any(np.diff(off) < 0):
        raise ValueError("offsets must be [G+1], non-decreasing, 0 .. M")
    y = np.zeros((m, n), np.float64)
    for e in range(g):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            y[lo:hi] = gemm_ref(qa[lo:hi], sa[lo:hi], qw[e], sw[e])
    return y
