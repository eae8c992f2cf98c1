"""E4M3 ("e4m3fn") code points: decode and round-to-nearest-even encode.

Test infrastructure only (see ``oracle/__init__.py``).

Format ([FP8-RL summary] §3.4.1 "Quantization Format and Granularity", which
takes the layout from "FP8 Formats for Deep Learning"): one sign bit, four
exponent bits with bias 7, three mantissa bits.

* exponent field 0: subnormal, value = m * 2^-9 (m = 0..7);
* exponent field 1..15: normal, value = (1 + m/8) * 2^(e-7);
* the pattern S.1111.111 (0x7F / 0xFF) is NaN; there is no infinity, so the
  largest finite magnitude is 1.75 * 2^8 = 448 (the FP8 maximum that §3.4.1
  maps each block maximum to) and the smallest normal is 2^-6.

Encoding rounds to the nearest representable value (§3.4.2 Phase 2 step 2
rounds each quotient to the nearest E4M3 value), ties to the even code (the IEEE
default; the pages give no tie rule), and saturates to +-448 instead of
producing NaN (the format has no infinity and the pages give no overflow
rule; the scale rule of §3.4.1 keeps in-range inputs at |v| <= 448 anyway).
The sign is kept, so negative values that round to zero give 0x80.
"""

import numpy as np

E4M3_MAX = 448.0
_NAN_MAG = 0x7F
_MAX_CODE = 0x7E


def decode_e4m3(codes):
    """Decode uint8 E4M3 codes to float64 (exact).  0x7F/0xFF decode to NaN."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes are bytes")
    sign = c >> 7
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    sub = man * 2.0 ** -9
    nrm = (1.0 + man / 8.0) * np.exp2((exp - 7).astype(np.float64))
    mag = np.where(exp == 0, sub, nrm)
    mag = np.where((c & 0x7F) == _NAN_MAG, np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def e4m3_finite_magnitudes():
    """The 127 non-negative finite E4M3 magnitudes, indexed by code 0x00..0x7E."""
    return decode_e4m3(np.arange(0, _MAX_CODE + 1))


def encode_e4m3(values):
    """Encode float32 values to E4M3 codes (uint8), round-to-nearest-even, saturating.

    ``values`` is converted to float32 first: the quantizer always hands the
    encoder a float32 quotient.  All arithmetic below is exact in float64
    (a float32 has 24 significant bits; the scalings are powers of two).
    Non-finite inputs are outside the contract and raise ``ValueError``.
    """
    v = np.asarray(values, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("encode_e4m3: non-finite input is outside the contract")
    neg = np.signbit(v)
    a = np.abs(v.astype(np.float64))
    code = np.zeros(a.shape, dtype=np.int64)

    # Subnormal range |v| < 2^-6: the grid is the multiples of 2^-9.
    # rint() rounds half to even; m == 8 is the smallest normal, whose code is 0x08.
    sub = a < 2.0 ** -6
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)

    # Normal range: a = (1 + f/8) * 2^e with e = floor(log2 a).
    nrm = ~sub
    frac, ex = np.frexp(a[nrm])  # a = frac * 2^ex, frac in [0.5, 1)
    e = ex.astype(np.int64) - 1
    f = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)  # 0..8, ties to even
    carry = f == 8  # rounding up into the next binade
    e = e + carry
    f = np.where(carry, 0, f)
    c_n = ((e + 7) << 3) | f
    code[nrm] = np.minimum(c_n, _MAX_CODE)  # saturate at 448 (code 0x7E)

    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)
