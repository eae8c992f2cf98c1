"""Pins of the MoE glue oracle (oracle/moe.py): brute force on tiny inputs,
an independent sorting of the synthetic router, textbook SiLU values and the
logistic function of scipy, and a matrix form of the combine."""

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

from oracle import quant_act_per_token_group, round_to_bf16_bits
from oracle.bf16 import bf16_bits_to_f64
from oracle.moe import combine, gather_quantize_act, silu_mul_bf16, silu_mul_f64, silu_mul_quantize, sort_by_expert
from synthetic import f32_to_bf16_bits, moe_routing, moe_topk


def brute_sort(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    rows, offsets = [], [0]
    for e in range(E):
        for p, v in enumerate(flat):
            if v == e:
                rows.append(p)
        offsets.append(len(rows))
    pair_row = [-1] * len(flat)
    for r, p in enumerate(rows):
        pair_row[p] = r
    return offsets, rows, pair_row


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (5, 2, 3, 1), (17, 4, 9, 2), (40, 8, 16, 3), (0, 8, 4, 4)])
def test_sort_brute_force(T, k, E, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, E + 2, size=(T, k)).astype(np.int32)   # duplicates and invalid ids included
    off, rows, pr = sort_by_expert(ids, E)
    boff, brows, bpr = brute_sort(ids, E)
    assert list(off) == boff and list(rows) == brows and list(pr) == bpr


def test_sort_matches_router_order_and_invariants():
    T, E, k = 512, 128, 8
    ids, _ = moe_topk(T, E, k, (70, 0))
    off, rows, pr = sort_by_expert(ids, E)
    tok, exp, roff = moe_routing(T, E, k, (70, 0))
    assert np.array_equal(off, roff)
    assert np.array_equal(rows // k, tok)
    assert np.array_equal(ids.reshape(-1)[rows], exp)
    assert np.array_equal(pr[rows], np.arange(T * k))
    for e in range(E):
        seg = rows[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_gather_quantize_is_quantize_then_gather():
    rng = np.random.default_rng(5)
    T, K, k = 9, 384, 3
    x = f32_to_bf16_bits(rng.normal(0, 1, (T, K)).astype(np.float32) * np.float32(3.0))
    ids = np.stack([rng.permutation(6)[:k] for _ in range(T)]).astype(np.int32)
    _, rows, _ = sort_by_expert(ids, 6)
    q, s = gather_quantize_act(x, rows, k)
    q0, s0 = quant_act_per_token_group(x)
    assert np.array_equal(q, q0[rows // k]) and np.array_equal(s, s0[rows // k])


def bf16(v):
    return f32_to_bf16_bits(np.asarray(v, np.float32))


def test_silu_textbook_values():
    # SiLU(1) = 1 / (1 + 1/e), SiLU(-1) = -1 / (1 + e), SiLU(0) = 0
    g = np.array([1.0, -1.0, 0.0, 2.0], np.float32)
    u = np.array([1.0, 1.0, 5.0, -0.5], np.float32)
    y = np.concatenate([bf16(g), bf16(u)])[None, :]
    h = silu_mul_f64(y, 4)[0]
    assert abs(h[0] - 0.7310585786300049) < 1e-15
    assert abs(h[1] + 0.2689414213699951) < 1e-15
    assert h[2] == 0.0
    assert abs(h[3] - (-0.5 * 1.7615941559557649)) < 1e-15
    bits = silu_mul_bf16(y, 4)[0]
    assert list(bits) == list(round_to_bf16_bits(np.array([0.7310585786300049, -0.2689414213699951, 0.0,
                                                           -0.8807970779778824])))


def test_silu_against_scipy_logistic_and_identities():
    rng = np.random.default_rng(6)
    M, F = 64, 256
    y = bf16(rng.normal(0, 2.5, (M, 2 * F)).astype(np.float32))
    g = bf16_bits_to_f64(y[:, :F])
    u = bf16_bits_to_f64(y[:, F:])
    h = silu_mul_f64(y, F)
    ref = g * expit(g) * u
    assert np.all(np.abs(h - ref) <= 1e-15 * np.abs(ref) + 1e-300)   # a few float64 roundings apart
    assert np.array_equal(silu_mul_bf16(y, F), round_to_bf16_bits(ref))
    # SiLU(g) - SiLU(-g) = g (u = 1)
    ones = np.ones_like(y[:, F:])
    hp = silu_mul_f64(np.concatenate([y[:, :F], ones * 0 + bf16(1.0)], axis=1), F)
    yn = y[:, :F] ^ np.uint16(0x8000)
    hn = silu_mul_f64(np.concatenate([yn, ones * 0 + bf16(1.0)], axis=1), F)
    assert np.all(np.abs(hp - hn - g) <= 1e-14 * (np.abs(g) + 1))


def decimal_silu_bf16(g, u, prec=60):
    """BF16 bits nearest to SiLU(g) * u evaluated with `prec` significant digits
    (an independent high-precision evaluation; ties cannot occur for g != 0)."""
    with localcontext() as ctx:
        ctx.prec = prec
        G, U = Decimal(float(g)), Decimal(float(u))
        h = G / (1 + (-G).exp()) * U
        hf = float(h)
        if hf == 0.0:
            return round_to_bf16_bits(np.array([hf]))[0]
        _, ex = np.frexp(hf)
        q = 2.0 ** (max(ex - 1, -126) - 7)
        lo = np.floor(hf / q) * q
        cands = [lo - q, lo, lo + q, lo + 2 * q]
        best = min(cands, key=lambda c: abs(Decimal(c) - h))
        if best == 0.0:
            best = np.copysign(0.0, hf)  # a tiny value rounds to the zero of its sign
        return round_to_bf16_bits(np.array([best]))[0]


def test_silu_layout_gate_first():
    # up = 0 gives h = 0 whatever the gate; a large gate g gives h ~ g * up
    F = 128
    g = bf16(np.full(F, 40.0))
    u = bf16(np.linspace(-3, 3, F))
    h = silu_mul_bf16(np.concatenate([g, u])[None, :], F)[0]
    uv = bf16_bits_to_f64(u)
    assert [int(b) for b in h] == [int(decimal_silu_bf16(40.0, v)) for v in uv]
    h0 = silu_mul_bf16(np.concatenate([u, bf16(np.zeros(F))])[None, :], F)[0]
    assert np.all((h0 & 0x7FFF) == 0)


def test_silu_quantize_is_quant_of_bf16_h():
    rng = np.random.default_rng(7)
    y = bf16(rng.normal(0, 1, (8, 2 * 384)).astype(np.float32))
    q, s = silu_mul_quantize(y, 384)
    q0, s0 = quant_act_per_token_group(silu_mul_bf16(y, 384))
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
    assert q.shape == (8, 384) and s.shape == (8, 3)


def test_combine_brute_force_exact():
    rng = np.random.default_rng(8)
    T, k, H, M = 6, 3, 5, 20
    y = bf16(rng.normal(0, 1, (M, H)).astype(np.float32))
    w = rng.random((T, k)).astype(np.float32)
    pr = rng.integers(-1, M, size=T * k).astype(np.int32)
    out, mag, bits = combine(y, pr, w)
    yv = bf16_bits_to_f64(y)
    for t in range(T):
        for h in range(H):
            exact = Fraction(0)
            for j in range(k):
                r = pr[t * k + j]
                if r >= 0:
                    exact += Fraction(float(w[t, j])) * Fraction(float(yv[r, h]))
            assert abs(Fraction(out[t, h]) - exact) <= Fraction(2.0 ** -50) * (abs(exact) + 1)
    assert np.array_equal(bits, round_to_bf16_bits(out))


def test_combine_matrix_form_and_special_weights():
    rng = np.random.default_rng(9)
    T, k, H, E = 32, 4, 64, 8
    ids, w = moe_topk(T, E, k, (71, 0))
    _, rows, pr = sort_by_expert(ids, E)
    y = bf16(rng.normal(0, 1, (T * k, H)).astype(np.float32))
    out, _, _ = combine(y, pr, w)
    S = np.zeros((T, T * k))
    for t in range(T):
        for j in range(k):
            S[t, pr[t * k + j]] += float(w[t, j])
    assert np.allclose(out, S @ bf16_bits_to_f64(y), rtol=1e-13, atol=1e-13)
    # one-hot weights copy the chosen row
    onehot = np.zeros((T, k), np.float32)
    onehot[:, 1] = 1.0
    _, _, bits = combine(y, pr, onehot)
    assert np.array_equal(bits, y[pr.reshape(T, k)[:, 1]])


def test_silu_rounding_matches_high_precision():
    # random gates over a wide range against a 60-digit evaluation
    rng = np.random.default_rng(10)
    g = np.concatenate([rng.normal(0, 3, 300), rng.uniform(-100, 100, 100), rng.normal(0, 1e-6, 50)])
    u = rng.normal(0, 2, g.size)
    y = bf16(np.concatenate([g, u]))[None, :]
    gv, uv = bf16_bits_to_f64(y[0, :g.size]), bf16_bits_to_f64(y[0, g.size:])
    h = silu_mul_bf16(y, g.size)[0]
    assert [int(b) for b in h] == [int(decimal_silu_bf16(a, b)) for a, b in zip(gv, uv)]


def test_silu_structural_near_ties():
    # tiny gate: g u / 2 exactly a BF16 midpoint; the exact h lies beyond it
    # in magnitude for g > 0 (sigma(g) > 1/2) and short of it for g < 0
    g = 0.75 * 2.0 ** -52
    u = -0.7109375
    assert (Fraction(g) * Fraction(u) / 2) == Fraction(-273, 4) * Fraction(2) ** -60
    for gs, expect_up in ((g, True), (-g, False)):
        y = bf16(np.array([gs, u]))[None, :]
        h = silu_mul_bf16(y, 1)[0, 0]
        mid = gs * u / 2
        hv = float(bf16_bits_to_f64(np.array([h]))[0])
        assert (abs(hv) > abs(mid)) == expect_up
        assert h == decimal_silu_bf16(gs, u, prec=80)
    # g = -2^-133 (smallest BF16 denormal), u = 1: h is just short of half the
    # smallest denormal in magnitude, so it rounds to -0
    y = np.array([[0x8001, bf16([1.0])[0]]], np.uint16)
    assert silu_mul_bf16(y, 1)[0, 0] == 0x8000
    assert silu_mul_bf16(np.array([[0x0001, bf16([1.0])[0]]], np.uint16), 1)[0, 0] == 0x0001
    # large gate: g u exactly a midpoint; sigma(g) < 1 puts h short of it
    found = 0
    for ub in range(0x3f80, 0x4000):
        uv = float(bf16_bits_to_f64(np.array([ub], np.uint16))[0])
        p = 40.0 * uv
        _, ex = np.frexp(p)
        q = 2.0 ** (ex - 1 - 7)
        if (p / q) % 1 == 0.5:
            y = np.array([[bf16([40.0])[0], ub]], np.uint16)
            hv = float(bf16_bits_to_f64(silu_mul_bf16(y, 1))[0, 0])
            assert abs(hv) < abs(p)
            found += 1
    assert found > 0
