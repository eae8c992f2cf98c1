"""Pins of the oracle's block / group quantizers (CPU only).

Pins used (none re-types the oracle's own formula):
* an exact-rational brute force on tiny tiles: the scale and every quotient
  are rounded to float32 by exhaustive comparison of Fractions, and the code
  is the nearest E4M3 magnitude found by search;
* closed forms: a block whose amax is 448 * 2^j has scale exactly 2^j and
  its codes are the hand-table encodings of x / 2^j;
* invariants: the amax element of every non-zero block encodes to +-448,
  |dec(q) * s - x| <= half an E4M3 ulp of x/s (times s) plus the float32
  rounding of the quotient, all-zero blocks, single-element and constant
  blocks;
* metamorphic relations: negation, scaling by 2^k, permutation within a
  block, stacking layers, row permutation of activations.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import (
    BLOCK,
    act_fragment_order,
    decode_e4m3,
    e4m3_finite_magnitudes,
    quant_act_per_token_group,
    quant_weight_block,
    quant_weight_blockwise,
)
from synthetic import activations, bf16_normal, f32_to_bf16_bits

MAGS = [Fraction(float(m)) for m in e4m3_finite_magnitudes()]


def _rn32(fr):
    """Round an exact rational to the nearest float32 (ties to even) by search."""
    c = np.float32(float(fr))
    u = int(np.abs(c).view(np.uint32))
    sign = -1 if fr < 0 else 1
    best = None
    for uu in (u - 2, u - 1, u, u + 1, u + 2):
        if uu < 0 or uu >= 0x7F800000:
            continue
        v = Fraction(float(np.uint32(uu).view(np.float32))) * sign
        key = (abs(v - fr), uu & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def _nearest_code(fr):
    a = abs(fr)
    d = [abs(a - m) for m in MAGS]
    lo = min(d)
    idx = [i for i, x in enumerate(d) if x == lo]
    i = idx[0] if len(idx) == 1 else [j for j in idx if j % 2 == 0][0]
    return i


def brute_quant_tile(x_f32):
    """Exact-rational restatement of one tile: returns (codes, scale)."""
    vals = [Fraction(float(v)) for v in x_f32.reshape(-1)]
    amax = max(abs(v) for v in vals)
    s = _rn32(amax / 448)
    codes = []
    for v, raw in zip(vals, x_f32.reshape(-1)):
        neg = bool(np.signbit(raw))
        if s == 0:
            codes.append(0x80 if neg else 0x00)
            continue
        q = _rn32(v / s)
        codes.append(_nearest_code(q) | (0x80 if neg else 0))
    return np.array(codes, np.uint8).reshape(x_f32.shape), np.float32(float(s))


def _f32(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@pytest.mark.parametrize("seed", range(6))
def test_tiny_blocks_against_exact_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    r, c = int(rng.integers(1, 40)), int(rng.integers(1, 40))
    std = float(np.exp2(rng.integers(-20, 20)))
    bits = bf16_normal((r, c), std, (99, seed))
    q, s = quant_weight_block(bits)
    bq, bs = brute_quant_tile(_f32(bits))
    assert s.view(np.uint32) == bs.view(np.uint32)
    assert np.array_equal(q, bq)


def test_tiny_activation_groups_against_brute_force():
    bits, _ = activations(5, 300, (98, 0), n_outliers=3, outlier_mult=50.0)
    q, s = quant_act_per_token_group(bits)
    x = _f32(bits)
    assert s.shape == (5, 3)
    for m in range(5):
        for g in range(3):
            cols = slice(g * BLOCK, min(300, (g + 1) * BLOCK))
            bq, bs = brute_quant_tile(x[m:m + 1, cols])
            assert s[m, g].view(np.uint32) == bs.view(np.uint32)
            assert np.array_equal(q[m:m + 1, cols], bq)


def test_subnormal_scale_block_against_brute_force():
    # amax so small that amax/448 is a float32 denormal
    bits = np.array([[0x0001, 0x8003, 0x0002], [0x0000, 0x8000, 0x0005]], np.uint16)  # bf16 denormals
    q, s = quant_weight_block(bits)
    bq, bs = brute_quant_tile(_f32(bits))
    assert s.view(np.uint32) == bs.view(np.uint32)
    assert s < np.float32(1.1754944e-38)
    assert np.array_equal(q, bq)


@pytest.mark.parametrize("j", [-12, -3, 0, 5])
def test_power_of_two_scale_closed_form(j):
    # values chosen from the hand table, times 2^j; amax = 448 * 2^j -> s = 2^j
    base = np.array([448.0, -1.0, 0.5, 3.0, -240.0, 2.0 ** -6, 2.0 ** -9, 1.0625, 1.1875, 400.0, -0.0, 0.0],
                    np.float64)
    want = np.array([0x7E, 0xB8, 0x30, 0x44, 0xF7, 0x08, 0x01, 0x38, 0x3A, 0x7C, 0x80, 0x00], np.uint8)
    x = (base * 2.0 ** j).astype(np.float32)
    bits = f32_to_bf16_bits(x).reshape(3, 4)
    assert np.array_equal(_f32(bits).reshape(-1), x)  # exactly representable in bf16
    q, s = quant_weight_block(bits)
    assert s == np.float32(2.0 ** j)
    assert np.array_equal(q.reshape(-1), want)


def test_invariants_on_random_blocks():
    w = bf16_normal((512, 640), 0.02, (1, 2, 3))
    q, s = quant_weight_blockwise(w)
    x = _f32(w).astype(np.float64)
    assert s.shape == (4, 5)
    dec = decode_e4m3(q)
    for i in range(4):
        for j in range(5):
            blk = (slice(i * 128, (i + 1) * 128), slice(j * 128, (j + 1) * 128))
            xb, qb, db, sb = x[blk], q[blk], dec[blk], float(s[i, j])
            amax = np.abs(xb).max()
            # the amax element maps to the largest code
            k = np.unravel_index(np.argmax(np.abs(xb)), xb.shape)
            assert qb[k] & 0x7F == 0x7E
            # scale is within half a float32 ulp of amax / 448
            assert abs(sb - amax / 448) <= 2.0 ** -24 * amax / 448
            # per-element error bound
            t = np.abs(xb) / sb
            e = np.floor(np.log2(np.maximum(t, 2.0 ** -6)))
            ulp8 = np.exp2(e - 3)  # E4M3 spacing in t's binade (2^-9 below 2^-6)
            bound = (0.5 * ulp8 + t * 2.0 ** -23) * sb
            assert np.all(np.abs(db * sb - xb) <= bound)
            assert np.all(np.abs(db) <= 448)


def test_all_zero_single_and_constant_blocks():
    z = np.zeros((128, 128), np.uint16)
    z[3, 4] = 0x8000  # a negative zero
    q, s = quant_weight_block(z)
    assert s == 0 and q[3, 4] == 0x80 and (q.sum() == 0x80)
    one = np.zeros((128, 128), np.uint16)
    one[5, 6] = f32_to_bf16_bits(np.float32([-0.37]))[0]
    q, s = quant_weight_block(one)
    assert q[5, 6] == 0xFE and np.count_nonzero(q) == 1
    assert s == np.float32(_f32(one[5:6, 6:7])[0, 0] * -1) / np.float32(448)
    const = np.full((128, 128), f32_to_bf16_bits(np.float32([1.7]))[0], np.uint16)
    q, s = quant_weight_block(const)
    assert np.all(q == 0x7E)


def test_metamorphic_negation_and_permutation():
    w = bf16_normal((128, 128), 0.02, (5, 0))
    q, s = quant_weight_block(w)
    qn, sn = quant_weight_block(w ^ np.uint16(0x8000))
    assert sn == s and np.array_equal(qn, q ^ np.uint8(0x80))
    rng = np.random.default_rng(0)
    perm = rng.permutation(128 * 128)
    qp, sp = quant_weight_block(w.reshape(-1)[perm].reshape(128, 128))
    assert sp == s and np.array_equal(qp.reshape(-1), q.reshape(-1)[perm])


@pytest.mark.parametrize("k", [-20, -1, 3, 40])
def test_metamorphic_power_of_two_scaling(k):
    w = bf16_normal((128, 256), 1.0, (6, k + 100))
    x = _f32(w)
    y = (x.astype(np.float64) * 2.0 ** k).astype(np.float32)
    assert np.array_equal(y.astype(np.float64) / 2.0 ** k, x.astype(np.float64))  # exact
    wy = f32_to_bf16_bits(y)
    q, s = quant_weight_blockwise(w)
    qy, sy = quant_weight_blockwise(wy)
    assert np.array_equal(q, qy)
    assert np.array_equal(sy.astype(np.float64), s.astype(np.float64) * 2.0 ** k)


def test_stacked_layers_equal_separate():
    a = bf16_normal((256, 384), 0.02, (7, 0))
    b = bf16_normal((128, 384), 0.02, (7, 1))
    qs, ss = quant_weight_blockwise(np.concatenate([a, b], axis=0))
    qa, sa = quant_weight_blockwise(a)
    qb, sb = quant_weight_blockwise(b)
    assert np.array_equal(qs, np.concatenate([qa, qb]))
    assert np.array_equal(ss, np.concatenate([sa, sb]))
    # the batch form equals per-matrix calls
    c = bf16_normal((2, 256, 384), 0.02, (7, 2))
    qc, sc = quant_weight_blockwise(c)
    for l in range(2):
        ql, sl = quant_weight_blockwise(c[l])
        assert np.array_equal(qc[l], ql) and np.array_equal(sc[l], sl)


def test_ragged_edges():
    w = bf16_normal((200, 300), 0.02, (8, 0))
    q, s = quant_weight_blockwise(w)
    assert s.shape == (2, 3)
    q2, s2 = quant_weight_block(w[128:200, 256:300])
    assert np.array_equal(q[128:, 256:], q2) and s[1, 2] == s2
    # padding with zeros does not change codes or scales of in-bounds elements
    pad = np.zeros((256, 384), np.uint16)
    pad[:200, :300] = w
    qp, sp = quant_weight_blockwise(pad)
    assert np.array_equal(qp[:200, :300], q) and np.array_equal(sp, s)


def test_activation_rows_commute_with_gather():
    x, _ = activations(64, 512, (9, 0), n_outliers=4, outlier_mult=50.0)
    q, s = quant_act_per_token_group(x)
    idx = np.random.default_rng(1).integers(0, 64, 200)
    qg, sg = quant_act_per_token_group(x[idx])
    assert np.array_equal(qg, q[idx]) and np.array_equal(sg, s[idx])


def test_activation_group_equals_weight_tile_definition():
    # a 1x128 group and a 1x128 "block" are the same tile
    x, _ = activations(1, 256, (10, 0))
    q, s = quant_act_per_token_group(x)
    for g in range(2):
        qb, sb = quant_weight_block(x[:, g * 128:(g + 1) * 128])
        assert np.array_equal(q[:, g * 128:(g + 1) * 128], qb) and s[0, g] == sb


def test_outlier_columns_change_only_their_groups():
    x, cols = activations(16, 512, (11, 0), n_outliers=4, outlier_mult=50.0)
    x0, _ = activations(16, 512, (11, 0))
    q, s = quant_act_per_token_group(x)
    q0, s0 = quant_act_per_token_group(x0)
    hit = np.unique(cols // 128)
    for g in range(4):
        same = np.array_equal(s[:, g], s0[:, g])
        assert same == (g not in hit)


def test_planted_mistake_is_caught():
    """Multiplying by the float32 reciprocal instead of dividing changes bytes."""
    w = bf16_normal((512, 512), 0.02, (12, 0))
    q, s = quant_weight_blockwise(w)
    x = _f32(w)
    from oracle import encode_e4m3
    wrong = np.empty_like(q)
    for i in range(4):
        for j in range(4):
            blk = (slice(i * 128, (i + 1) * 128), slice(j * 128, (j + 1) * 128))
            r = np.float32(1) / s[i, j]
            wrong[blk] = encode_e4m3(x[blk] * r)
    assert not np.array_equal(wrong, q)


def test_act_fragment_order_element_mapping():
    """Every code lands where the MFMA operand layout puts it: checked one
    element at a time against the offset formula written out in scalars, and
    the permutation is a bijection (every byte moved exactly once)."""
    rng = np.random.default_rng(123)
    m, k = 32, 384
    codes = rng.integers(0, 256, (m, k)).astype(np.uint8)
    frag = act_fragment_order(codes).reshape(-1)
    kb = k // 128
    seen = np.zeros(m * k, bool)
    for r in range(m):
        for c in range(k):
            off = ((r // 16 * kb + c // 128) * 2 + (c % 128) // 64) * 1024 + (((c % 64) // 16) * 16 + r % 16) * 16 + c % 16
            assert frag[off] == codes[r, c]
            seen[off] = True
    assert seen.all()
    with pytest.raises(ValueError):
        act_fragment_order(codes[:24])
