"""Pins of the oracle's block-scaled GEMM and grouped GEMM (CPU only).

Pins: an exact-rational triple loop on tiny shapes (every product and sum in
Fractions, one rounding to BF16 by exhaustive search), the FP32-accumulated
form against that exact sum within its float32 error bound, one-hot and all-ones
activation rows that reproduce dequantized weight rows and row sums, exact
doubling under a power-of-two activation scale, and the grouped form against
per-expert dense calls (G = 1, empty experts, a single hot expert).
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import (
    decode_e4m3,
    dequant_weight,
    gemm_ref,
    gemm_ref_bf16,
    gemm_ref_fp32,
    grouped_gemm_ref,
    quant_act_per_token_group,
    quant_weight_blockwise,
)
from synthetic import activations, bf16_normal


def _codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    return c


def _nearest_bf16(fr):
    """Exhaustive nearest BF16 (ties to even) of an exact rational."""
    c = np.float32(float(fr))
    b = int(c.view(np.uint32)) >> 16
    best = None
    for bb in range(b - 2, b + 3):
        bb &= 0xFFFF
        if (bb & 0x7F80) == 0x7F80:
            continue
        v = Fraction(float((np.uint32(bb) << np.uint32(16)).view(np.float32)))
        key = (abs(v - fr), bb & 1)
        if best is None or key < best[0]:
            best = (key, bb)
    return best[1]


@pytest.mark.parametrize("seed", range(3))
def test_tiny_gemm_against_exact_rational_triple_loop(seed):
    rng = np.random.default_rng(seed)
    m, n, k = 3, 5 + 128 * (seed == 2), 256
    qa, qw = _codes(rng, (m, k)), _codes(rng, (n, k))
    sa = rng.uniform(0.001, 2.0, (m, k // 128)).astype(np.float32)
    sw = rng.uniform(0.001, 2.0, (-(-n // 128), k // 128)).astype(np.float32)
    y = gemm_ref(qa, sa, qw, sw)
    yb = gemm_ref_bf16(qa, sa, qw, sw)
    da, dw = decode_e4m3(qa), decode_e4m3(qw)
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                acc += (Fraction(float(da[i, t])) * Fraction(float(sa[i, t // 128]))
                        * Fraction(float(dw[j, t])) * Fraction(float(sw[j // 128, t // 128])))
            assert abs(Fraction(float(y[i, j])) - acc) <= abs(acc) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 200)
            assert yb[i, j] == _nearest_bf16(acc)


def test_one_hot_rows_reproduce_weight_rows():
    rng = np.random.default_rng(4)
    n, k = 256, 384
    qw = _codes(rng, (n, k))
    sw = rng.uniform(0.01, 1.0, (2, 3)).astype(np.float32)
    cols = np.array([0, 127, 128, 300, 383])
    qa = np.zeros((len(cols), k), np.uint8)
    qa[np.arange(len(cols)), cols] = 0x38  # E4M3 1.0
    sa = np.ones((len(cols), 3), np.float32)
    y = gemm_ref(qa, sa, qw, sw)
    w = dequant_weight(qw, sw)
    assert np.array_equal(y, w[:, cols].T)
    # all-ones activations give the weight row sums
    y1 = gemm_ref(np.full((1, k), 0x38, np.uint8), np.ones((1, 3), np.float32), qw, sw)
    assert np.allclose(y1[0], w.sum(axis=1), rtol=1e-12, atol=0)


def test_power_of_two_activation_scale_doubles_output():
    rng = np.random.default_rng(5)
    qa, qw = _codes(rng, (7, 256)), _codes(rng, (130, 256))
    sa = rng.uniform(0.1, 1, (7, 2)).astype(np.float32)
    sw = rng.uniform(0.1, 1, (2, 2)).astype(np.float32)
    y = gemm_ref(qa, sa, qw, sw)
    y2 = gemm_ref(qa, sa * np.float32(2), qw, sw)
    assert np.array_equal(y2, 2 * y)


def test_sampled_entries_equal_full():
    x, _ = activations(64, 512, (20, 0), n_outliers=4, outlier_mult=50.0)
    w = bf16_normal((384, 512), 0.02, (20, 1))
    qa, sa = quant_act_per_token_group(x)
    qw, sw = quant_weight_blockwise(w)
    full = gemm_ref(qa, sa, qw, sw)
    rows, cols = np.array([0, 5, 63]), np.array([1, 200, 383])
    # BLAS may sum in another order for a sub-grid: equal to float64 rounding
    assert np.allclose(gemm_ref(qa, sa, qw, sw, rows, cols), full[np.ix_(rows, cols)], rtol=1e-12, atol=1e-14)


def test_quantized_gemm_close_to_bf16_gemm():
    """End-to-end sanity: W8A8 output is within FP8 quantization noise of the BF16 product."""
    x, _ = activations(32, 512, (21, 0), n_outliers=4, outlier_mult=50.0)
    w = bf16_normal((384, 512), 0.02, (21, 1))
    qa, sa = quant_act_per_token_group(x)
    qw, sw = quant_weight_blockwise(w)
    y = gemm_ref(qa, sa, qw, sw)
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = xf @ wf.T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.06  # two E4M3 roundings, each <= 2^-4 relative


def test_grouped_equals_per_expert_dense():
    rng = np.random.default_rng(6)
    g, n, k = 5, 256, 256
    counts = np.array([3, 0, 17, 1, 0])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    m = int(off[-1])
    qa, sa = _codes(rng, (m, k)), rng.uniform(0.1, 1, (m, 2)).astype(np.float32)
    qw = _codes(rng, (g, n, k))
    sw = rng.uniform(0.1, 1, (g, 2, 2)).astype(np.float32)
    y = grouped_gemm_ref(qa, sa, qw, sw, off)
    for e in range(g):
        lo, hi = off[e], off[e + 1]
        if hi > lo:
            assert np.array_equal(y[lo:hi], gemm_ref(qa[lo:hi], sa[lo:hi], qw[e], sw[e]))
    # G == 1 is the dense GEMM
    y1 = grouped_gemm_ref(qa, sa, qw[:1], sw[:1], np.array([0, m], np.int32))
    assert np.array_equal(y1, gemm_ref(qa, sa, qw[0], sw[0]))


def test_grouped_rejects_bad_offsets():
    qa = np.zeros((4, 128), np.uint8)
    sa = np.ones((4, 1), np.float32)
    qw = np.zeros((2, 128, 128), np.uint8)
    sw = np.ones((2, 1, 1), np.float32)
    with pytest.raises(ValueError):
        grouped_gemm_ref(qa, sa, qw, sw, np.array([0, 3, 2], np.int32))
    with pytest.raises(ValueError):
        grouped_gemm_ref(qa, sa, qw, sw, np.array([0, 2, 5], np.int32))
    with pytest.raises(ValueError):
        gemm_ref(np.zeros((1, 100), np.uint8), np.ones((1, 1), np.float32), np.zeros((1, 100), np.uint8),
                 np.ones((1, 1), np.float32))


def test_planted_mistake_is_caught():
    """Using the wrong weight-scale row (n % nb instead of n // 128) changes outputs."""
    rng = np.random.default_rng(7)
    qa, qw = _codes(rng, (4, 128)), _codes(rng, (256, 128))
    sa = np.ones((4, 1), np.float32)
    sw = np.array([[1.0], [3.0]], np.float32)
    y = gemm_ref(qa, sa, qw, sw)
    wrong_w = decode_e4m3(qw) * sw[np.arange(256) % 2]
    wrong = decode_e4m3(qa) @ wrong_w.T
    assert not np.allclose(wrong, y)


def _exact_sum(da, sa, dw, sw, i, j):
    acc, mag = Fraction(0), Fraction(0)
    for t in range(da.shape[1]):
        term = (Fraction(float(da[i, t])) * Fraction(float(sa[i, t // 128]))
                * Fraction(float(dw[j, t])) * Fraction(float(sw[j // 128, t // 128])))
        acc += term
        mag += abs(term)
    return acc, mag


@pytest.mark.parametrize("seed", range(3))
def test_fp32_accumulated_form_within_float32_bound_of_exact_sum(seed):
    """gemm_ref_fp32 vs the exact rational sum: each K-block's float32 product
    (<= 128 roundings in any order), the scale product and its multiply (2),
    and KB accumulator additions give |y - exact| <= (128 + KB + 2) u sum|terms|
    (u = 2^-24, first order; the factor is generous)."""
    rng = np.random.default_rng(40 + seed)
    m, n, k = 3, 5 + 128 * (seed == 1), 128 * (2 + seed)
    qa, qw = _codes(rng, (m, k)), _codes(rng, (n, k))
    sa = rng.uniform(0.001, 2.0, (m, k // 128)).astype(np.float32)
    sw = rng.uniform(0.001, 2.0, (-(-n // 128), k // 128)).astype(np.float32)
    y = gemm_ref_fp32(qa, sa, qw, sw)
    assert y.dtype == np.float32 and y.shape == (m, n)
    da, dw = decode_e4m3(qa), decode_e4m3(qw)
    kb = k // 128
    for i in range(m):
        for j in range(n):
            acc, mag = _exact_sum(da, sa, dw, sw, i, j)
            bound = mag * Fraction(128 + kb + 3, 2 ** 24)
            assert abs(Fraction(float(y[i, j])) - acc) <= bound, (i, j)
    # the sampled-rows form computes the same rows
    rows = np.array([2, 0])
    assert np.array_equal(gemm_ref_fp32(qa, sa, qw, sw, rows=rows), y[rows])


def test_fp32_accumulated_form_exact_on_one_hot_rows():
    """One non-zero product per output: the product of the codes and the scale
    product are exact, so y is the exact dequantized weight rounded once to
    float32."""
    rng = np.random.default_rng(44)
    n, k = 256, 384
    qw = _codes(rng, (n, k))
    sw = rng.uniform(0.01, 1.0, (2, 3)).astype(np.float32)
    cols = np.array([0, 127, 128, 300, 383])
    qa = np.zeros((len(cols), k), np.uint8)
    qa[np.arange(len(cols)), cols] = 0x38  # E4M3 1.0
    sa = np.ones((len(cols), 3), np.float32)
    y = gemm_ref_fp32(qa, sa, qw, sw)
    w = dequant_weight(qw, sw)
    assert np.array_equal(y, w[:, cols].T.astype(np.float32))


def test_fp32_accumulated_form_catches_a_transposed_scale_grid():
    """A planted mistake in the fp32 form's recipe (weight scales indexed
    [kb][n//128]) moves the result far outside the float32 bound."""
    rng = np.random.default_rng(45)
    qa, qw = _codes(rng, (4, 256)), _codes(rng, (256, 256))
    sa = rng.uniform(0.5, 1, (4, 2)).astype(np.float32)
    sw = np.array([[1.0, 4.0], [0.25, 2.0]], np.float32)
    y = gemm_ref_fp32(qa, sa, qw, sw)
    wrong = gemm_ref_fp32(qa, sa, qw, np.ascontiguousarray(sw.T))
    exact = gemm_ref(qa, sa, qw, sw)
    assert np.max(np.abs(y - exact)) < 1e-4 * np.max(np.abs(exact))
    assert np.max(np.abs(wrong - exact)) > 0.1 * np.max(np.abs(exact))
