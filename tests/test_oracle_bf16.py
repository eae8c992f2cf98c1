"""Pins of the oracle's BF16 helpers (CPU only)."""

from fractions import Fraction

import numpy as np
import torch

from oracle import bf16_bits_to_f32, round_to_bf16_bits


def test_widening_known_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4040, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    f = bf16_bits_to_f32(bits)
    assert f[0] == 1.0 and f[1] == -1.0 and f[2] == 3.0
    assert f[3] == 0.0 and np.signbit(f[4])
    assert f[5] == np.float32(3.3895314e38)
    assert f[6] == np.float32(2.0 ** -133)


def test_rounding_matches_torch_cast_on_float32():
    """torch's CPU float32 -> bfloat16 cast is round-to-nearest-even."""
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 500_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.38e38)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(round_to_bf16_bits(f.astype(np.float64)), want)


def _nearest_bf16_exact(x):
    """Brute force: exact comparison of |x - b| over the two BF16 neighbours."""
    fx = Fraction(x)
    c = np.float32(x)  # within a float32 ulp of x
    b = int(c.view(np.uint32)) >> 16
    cands = []
    for bb in (b - 1, b, b + 1, b + 2):
        if 0 <= (bb & 0x7FFF) <= 0x7F7F:
            v = (np.uint32(bb & 0xFFFF) << np.uint32(16)).view(np.float32)
            cands.append((abs(Fraction(float(v)) - fx), bb & 1, bb & 0xFFFF))
    cands.sort()
    best = [c for c in cands if c[0] == cands[0][0]]
    if len(best) > 1:
        best = [c for c in best if c[1] == 0]
    return best[0][2]


def test_rounding_of_float64_by_exact_search():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))
    # exact ties and near-ties that a float32 intermediate would double-round
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -40, -(1 + 2.0 ** -8 + 2.0 ** -30)])
    x = np.concatenate([x, ties])
    got = round_to_bf16_bits(x)
    want = np.array([_nearest_bf16_exact(v) for v in x], np.uint16)
    assert np.array_equal(got, want)
    assert got[-4] == 0x3F80 and got[-3] == 0x3F82  # ties to even
    assert got[-2] == 0x3F81  # just above the tie: up (no double rounding)
