"""Pins of the FP8 KV-cache oracle (oracle/kv.py): the calibration scale is
the per-head / per-layer tile scale, calibration tokens encode exactly as
their tile does, values beyond the calibrated range saturate, the per-layer
scale is the largest per-head one, and the cache write is a slot scatter."""

import numpy as np
import pytest

from oracle import decode_e4m3, quantize_tiles
from oracle.bf16 import bf16_bits_to_f32
from oracle.kv import kv_cache_write, kv_calibrate, kv_quantize
from synthetic import f32_to_bf16_bits


def kv(T, H, D, seed, std=1.0):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, std, (T, H, D)).astype(np.float32)
    x *= rng.uniform(0.1, 4.0, (1, H, 1)).astype(np.float32)   # heads of different ranges
    return f32_to_bf16_bits(x)


def test_calibration_scale_closed_form():
    x = kv(5, 3, 16, 1)
    xf = bf16_bits_to_f32(x)
    s_h = kv_calibrate(x, per_head=True)
    s_l = kv_calibrate(x, per_head=False)
    amax_h = np.abs(xf).max(axis=(0, 2))
    assert np.array_equal(s_h, (amax_h / np.float32(448)).astype(np.float32))
    assert s_l.shape == (1,) and s_l[0] == np.float32(np.abs(xf).max() / np.float32(448))
    assert s_l[0] == s_h.max()   # fl32(a / 448) is monotone in a


def test_calibration_tokens_encode_as_their_tile():
    x = kv(7, 4, 32, 2)
    for per_head in (True, False):
        s = kv_calibrate(x, per_head)
        q = kv_quantize(x, s, per_head)
        T, H, D = x.shape
        tiles = x.transpose(1, 0, 2).reshape(H, T * D) if per_head else x.reshape(1, -1)
        qt, st = quantize_tiles(bf16_bits_to_f32(tiles))
        ref = qt.reshape(H, T, D).transpose(1, 0, 2) if per_head else qt.reshape(T, H, D)
        assert np.array_equal(q, ref) and np.array_equal(s, st)
        # the largest magnitude of each tile encodes to +-448
        assert np.any((q & 0x7F) == 0x7E)


def test_saturation_beyond_calibrated_range():
    x = kv(4, 2, 8, 3)
    s = kv_calibrate(x, True)
    xf = bf16_bits_to_f32(x)
    big = f32_to_bf16_bits(np.float32(3.0) * xf)           # a later step's larger values
    q = kv_quantize(big, s, True)
    dec = decode_e4m3(q)
    assert np.all(np.abs(dec) <= 448)
    over = np.abs(bf16_bits_to_f32(big)) / s[None, :, None] >= 464
    assert np.any(over) and np.all((q[over] & 0x7F) == 0x7E)
    assert np.array_equal(np.signbit(dec[over]), np.signbit(bf16_bits_to_f32(big)[over]))
    # a value just below the rounding boundary to 448 stays below it
    h = np.array([[[np.float32(447.0)]]], np.float32)
    assert decode_e4m3(kv_quantize(f32_to_bf16_bits(h), np.ones(1, np.float32), True))[0, 0, 0] == 448.0


def test_zero_scale_and_zero_values():
    x = np.zeros((2, 1, 8), np.uint16)
    x[0, 0, 1] = 0x8000                                      # -0
    s = kv_calibrate(x, True)
    assert s[0] == 0
    y = f32_to_bf16_bits(np.array([[[0.0, -0.0, 1.0, -2.0, 0.0, 0.0, 0.0, 0.0]]], np.float32))
    q = kv_quantize(y, s, True)
    assert list(q[0, 0, :4]) == [0x00, 0x80, 0x7E, 0xFE]


def test_cache_write_scatter():
    T, H, D, S = 9, 2, 16, 20
    x = kv(T, H, D, 4)
    s = kv_calibrate(x, False)
    cache = np.full((S, H, D), 0xAB, np.uint8)
    slots = np.array([3, 0, -1, 19, 7, 20, 11, 2, 5], np.int64)    # -1 and 20: padding
    out = kv_cache_write(cache, x, s, False, slots)
    q = kv_quantize(x, s, False)
    for t, sl in enumerate(slots):
        if 0 <= sl < S:
            assert np.array_equal(out[sl], q[t])
    untouched = np.setdiff1d(np.arange(S), slots[(slots >= 0) & (slots < S)])
    assert np.all(out[untouched] == 0xAB)
    assert np.all(cache == 0xAB)                              # the input is not modified


def test_dequantized_error_bound():
    # |dec(q) s - x| <= (half an E4M3 ulp + a float32 ulp) * s inside the range
    x = kv(16, 4, 64, 5)
    s = kv_calibrate(x, True)
    q = kv_quantize(x, s, True)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    sv = s[None, :, None].astype(np.float64)
    err = np.abs(decode_e4m3(q) * sv - xf)
    a = np.abs(xf / sv)
    ulp = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(err <= (0.5 * ulp + 2.0 ** -23 * a) * sv + 1e-30)


def test_kv_layout_checks():
    # per-head scales must match the head count
    with pytest.raises(ValueError):
        kv_quantize(np.zeros((2, 3, 4), np.uint16), np.ones(2, np.float32), True)
