"""Pins of the oracle's E4M3 codec (CPU only).

The codec is pinned three independent ways: a hand-computed table
(tests/golden/e4m3_hand_table.txt), a brute-force nearest-code search over
the 127 finite magnitudes (which saturates by construction and breaks ties
to the even code), and closed-form facts of the format (448 max, 2^-6
smallest normal, 2^-9 smallest subnormal, 254 finite codes).
"""

import os

import numpy as np
import pytest

from oracle import decode_e4m3, encode_e4m3, e4m3_finite_magnitudes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand_table.txt")


def _parse_value(tok):
    if tok == "-0.0":
        return -0.0
    return float(eval(tok, {"__builtins__": {}}, {}))  # "2**-6", "7.5*2**-9" ...


def load_hand_table():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            rows.append((_parse_value(parts[0]), int(parts[1], 16)))
    return rows


def brute_force_encode(values):
    """Nearest finite E4M3 magnitude by exhaustive search; ties -> even code.

    Distances are exact in float64 only while |v| and the code magnitudes are
    within ~2^29 of each other, so the search is limited to |v| < 2^24;
    larger inputs are covered by ``test_saturation_closed_form``.
    """
    v = np.asarray(values, np.float32).astype(np.float64)
    assert np.all(np.abs(v) < 2.0 ** 24)
    mags = e4m3_finite_magnitudes()  # index == code 0..126
    d = np.abs(np.abs(v)[:, None] - mags[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among the (at most two) nearest codes pick the even one
    even = cand & (np.arange(127)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return (pick | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def test_hand_table_encode():
    rows = load_hand_table()
    assert len(rows) >= 30
    vals = np.array([r[0] for r in rows], np.float64).astype(np.float32)
    want = np.array([r[1] for r in rows], np.uint8)
    got = encode_e4m3(vals)
    bad = [(rows[i][0], hex(want[i]), hex(got[i])) for i in np.nonzero(got != want)[0]]
    assert not bad, bad


def test_hand_table_decode_exact_rows():
    # rows whose value is exactly representable decode back to that value
    for val, code in load_hand_table():
        dec = decode_e4m3(np.uint8(code))
        if abs(val) <= 448 and np.float64(dec) == val:
            assert np.signbit(dec) == np.signbit(val) or val != 0


def test_format_closed_forms():
    mags = e4m3_finite_magnitudes()
    assert mags.shape == (127,)
    assert mags[0x7E] == 448.0
    assert mags[0x08] == 2.0 ** -6
    assert mags[0x01] == 2.0 ** -9
    assert mags[0x07] == 7 * 2.0 ** -9
    assert np.all(np.diff(mags) > 0)  # strictly increasing with the code
    assert np.isnan(decode_e4m3(np.uint8(0x7F))) and np.isnan(decode_e4m3(np.uint8(0xFF)))
    # negative codes mirror positive ones
    pos = decode_e4m3(np.arange(0, 127))
    neg = decode_e4m3(np.arange(128, 255))
    assert np.array_equal(-pos, neg)
    # 254 finite codes, 253 distinct finite values (+0 and -0 compare equal)
    fin = decode_e4m3(np.arange(256))
    assert np.isfinite(fin).sum() == 254
    assert len(np.unique(fin[np.isfinite(fin)])) == 253


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    assert np.array_equal(encode_e4m3(decode_e4m3(codes)), codes)


def test_all_bf16_patterns_against_brute_force():
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 2.0 ** 24)]
    assert np.array_equal(encode_e4m3(f), brute_force_encode(f))


def test_saturation_closed_form():
    """Every finite float32 at or above 448 in magnitude encodes to +-448."""
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) >= 448)]
    big = np.concatenate([f, np.float32([3.4028235e38, -3.4028235e38, 448.00003, 463.99997])])
    want = np.where(np.signbit(big), 0xFE, 0x7E).astype(np.uint8)
    assert np.array_equal(encode_e4m3(big), want)


@pytest.mark.parametrize("scale", [0.7071067, 1.3333334, 3.1415927, 1e-3, 37.5, 2.0 ** -7])
def test_scaled_bf16_patterns_against_brute_force(scale):
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 1e30)]
    v = (f * np.float32(scale)).astype(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 2.0 ** 24)]
    assert np.array_equal(encode_e4m3(v), brute_force_encode(v))


def test_neighbourhood_of_every_midpoint_and_code():
    """Every float32 within 4 ulps of each code value and each midpoint."""
    mags = e4m3_finite_magnitudes()
    mids = (mags[:-1] + mags[1:]) / 2
    pts = np.concatenate([mags, mids, [464.0, 480.0, 512.0]]).astype(np.float32)
    u = pts.view(np.int32)
    offs = np.arange(-4, 5, dtype=np.int32)
    nb = (u[:, None] + offs[None, :]).reshape(-1)
    nb = nb[nb >= 0].view(np.float32)
    v = np.concatenate([nb, -nb])
    assert np.array_equal(encode_e4m3(v), brute_force_encode(v))


def test_random_float32_against_brute_force():
    rng = np.random.default_rng(1234)
    lin = rng.uniform(-520, 520, 200_000).astype(np.float32)
    log = (np.exp2(rng.uniform(-40, 10, 200_000)) * rng.choice([-1, 1], 200_000)).astype(np.float32)
    bits = rng.integers(0, 0x44000000, 200_000, dtype=np.int64).astype(np.uint32).view(np.float32)
    v = np.concatenate([lin, log, bits])
    assert np.array_equal(encode_e4m3(v), brute_force_encode(v))


def test_float32_denormals_and_tiny():
    v = np.array([1e-45, -1e-45, 1e-40, -1e-40, 1.1754942e-38, 2.0 ** -11, -(2.0 ** -11)], np.float32)
    got = encode_e4m3(v)
    assert list(got) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x00, 0x80]


def test_non_finite_rejected():
    with pytest.raises(ValueError):
        encode_e4m3(np.array([np.inf], np.float32))
    with pytest.raises(ValueError):
        encode_e4m3(np.array([np.nan], np.float32))


def test_planted_mistake_is_caught():
    """A plausible encoder bug (ties away from zero) fails the brute force."""
    v = np.float32(np.array([1.0625, 7.5 * 2 ** -9, 400.0]))
    wrong = np.array([0x39, 0x08, 0x7D], np.uint8)  # round-half-up answers
    assert not np.array_equal(wrong, brute_force_encode(v))
    assert np.array_equal(encode_e4m3(v), brute_force_encode(v))
