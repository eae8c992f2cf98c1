"""The GPU encoder test expands the oracle's encoder over every float32 bit
pattern through its step-function form (helpers.e4m3_transition_table).
This CPU test checks that expansion against the oracle's encoder itself."""

import numpy as np

from helpers import e4m3_transition_table
from oracle import encode_e4m3


def _expand(table, bits):
    bits = np.asarray(bits, np.uint32)
    mag = (bits & np.uint32(0x7FFFFFFF)).astype(np.int64)
    code = np.searchsorted(table, mag, side="right").astype(np.uint8)
    return code | ((bits >> np.uint32(24)).astype(np.uint8) & np.uint8(0x80))


def test_table_matches_oracle_everywhere_it_changes():
    t = e4m3_transition_table()
    assert t.shape == (126,) and np.all(np.diff(t) > 0)
    # every transition point and its neighbours, both signs
    pts = np.concatenate([t - 1, t, t + 1]).astype(np.uint32)
    pts = np.concatenate([pts, pts | np.uint32(0x80000000)])
    assert np.array_equal(_expand(t, pts), encode_e4m3(pts.view(np.float32)))


def test_table_matches_oracle_on_random_patterns():
    t = e4m3_transition_table()
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    bits = bits[np.isfinite(f)]
    assert np.array_equal(_expand(t, bits), encode_e4m3(bits.view(np.float32)))
