"""BF16 bit patterns: exact widening and round-to-nearest-even narrowing.

Test infrastructure only (see ``oracle/__init__.py``).

BF16 is the upper half of an IEEE binary32: 1 sign, 8 exponent, 7 mantissa
bits.  The pages use it for the trainer's master weights and for the
activations and outputs around the FP8 linear layers ([FP8-RL summary]
§3.4.1 and §3.4.2 Phase 3: results are "accumulated in FP32 ... and then
converted back to BF16/FP16").
"""

import numpy as np

_BF16_MAX = float(np.uint32(0x7F7F0000).view(np.float32))  # 3.3895e38


def bf16_bits_to_f32(bits):
    """uint16 BF16 bit patterns -> float32 (exact: append 16 zero bits)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def round_to_bf16_bits(values):
    """Round float64 (or float32) values once, to nearest-even, into BF16 bits.

    The rounding is done directly from the input precision (no intermediate
    float32 step, so no double rounding).  BF16 keeps 8 significant bits and
    float32's exponent range; below 2^-126 the grid is the multiples of
    2^-133.  Magnitudes that round above the largest finite BF16 become
    infinity, as IEEE round-to-nearest does.
    """
    x = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("round_to_bf16_bits: non-finite input")
    _, ex = np.frexp(x)  # |x| = frac * 2^ex, frac in [0.5, 1)
    e = ex.astype(np.int64) - 1  # |x| in [2^e, 2^(e+1))
    e = np.maximum(e, -126)  # subnormal grid below 2^-126
    quantum = np.exp2((e - 7).astype(np.float64))
    r = np.rint(x / quantum) * quantum  # exact in float64; rint = half-even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    f = r.astype(np.float32)  # exact: r has <= 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
