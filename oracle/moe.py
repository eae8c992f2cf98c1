"""MoE expert-FFN glue around the grouped block-scaled GEMMs.

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ([FP8-RL summary] §3.4.1 "Quantization Scope": the MoE
expert layers fc1 / fc2 are FP8 W8A8 linears like the dense ones; the gated
MLP's gate and up projections produce activations that are multiplied
element-wise before the down projection; §3.4.1 "Static vs. Dynamic
Quantization": activations are quantized on the fly in 1x128 tiles and the
surrounding nonlinearities stay in higher precision):

1. ``sort_by_expert``: the (token, slot) pairs of top-k routing, grouped by
   expert so each expert's rows are contiguous for the grouped GEMM.
2. ``gather_quantize_act``: the FP8 activation rows of the sorted pairs
   (1x128 per-token groups of the token's BF16 hidden state).
3. ``silu_mul_bf16`` / ``silu_mul_quantize``: h = SiLU(gate) * up from the
   fc1 output, rounded to BF16, then quantized in 1x128 groups for fc2.
4. ``combine``: each token's output is the routing-weighted sum of its k
   expert outputs, rounded to BF16.

Readings of what the pages leave open:

* Routing ids are int32 [T][k]; pair p = t * k + j.  Pairs are ordered by
  expert, then by p (for distinct ids per token: by token).  Ids outside
  [0, E) take no row (pair_row = -1) and are left out of the offsets.
* fc1's output row is [gate | up]: columns [0, F) are the gate projection,
  [F, 2F) the up projection (one fused fc1 GEMM of width 2F).
* The gated activation is SiLU(g) = g / (1 + exp(-g)) (Qwen3's MLP, the
  model family of the pages' experiments).  h = SiLU(g) * u of the BF16
  inputs is rounded once, to nearest even, to BF16 (the precision in which
  the nonlinearity stays), then quantized like any activation.  The
  rounding is that of the exact real value: float64 decides it except near
  a BF16 midpoint, where an exact comparison does.
* The combine weights are float32 [T][k]; the sum is formed in float64 and
  rounded once to BF16.  Pairs without a row contribute nothing.

Pinned in ``tests/test_oracle_moe.py``.
"""

from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

from .bf16 import bf16_bits_to_f64, round_to_bf16_bits
from .quant import quant_act_per_token_group


def sort_by_expert(topk_ids, E):
    """Group routing pairs by expert.

    Returns ``(offsets int32 [E+1], sorted_pair int32 [n_valid], pair_row int32
    [T*k])``: expert e owns sorted rows [offsets[e], offsets[e+1]); row r holds
    pair sorted_pair[r]; pair p sits in row pair_row[p] (-1 if its id is not
    an expert).
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    P = ids.size
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E) if P else np.zeros(E, np.int64)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    pairs = np.nonzero(valid)[0]
    order = pairs[np.argsort(ids[pairs], kind="stable")]     # by expert, then pair index
    pair_row = np.full(P, -1, np.int64)
    pair_row[order] = np.arange(order.size)
    return offsets.astype(np.int32), order.astype(np.int32), pair_row.astype(np.int32)


def gather_quantize_act(x_bits, sorted_pair, k):
    """FP8 codes and scales of rows x[sorted_pair // k] (1x128 groups)."""
    x = np.asarray(x_bits, dtype=np.uint16)
    tok = np.asarray(sorted_pair, dtype=np.int64) // int(k)
    return quant_act_per_token_group(x[tok])


def silu_mul_f64(y_bits, F):
    """Exact-as-float64 h = SiLU(gate) * up of fc1 output rows [M][2F] (BF16 bits)."""
    y = bf16_bits_to_f64(np.asarray(y_bits, dtype=np.uint16))
    g, u = y[:, :F], y[:, F:2 * F]
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def _exceeds_midpoint(g, u, mid):
    """|SiLU(g) * u| > |mid| for a BF16 midpoint mid of the same sign, decided exactly.

    With P = g * u (exact) and r = mid / P > 0 (rationals):
        |h| > |mid|  <=>  sigma(g) > r,  sigma(g) = 1 / (1 + e^-g),
    which is false for r >= 1 (sigma < 1) and otherwise, with s = 1/r - 1 > 0,
        <=>  e^-g < s  <=>  g > -ln(s).
    ln(s) of the rational s is taken to 100 significant digits; g is a BF16
    value and -ln(s) is transcendental unless s = 1 (then the test is g > 0).
    """
    P = Fraction(g) * Fraction(u)
    r = mid / P
    if r >= 1:
        return False
    s = 1 / r - 1
    if s == 1:
        return g > 0
    with localcontext() as ctx:
        ctx.prec = 100
        ln_s = (Decimal(s.numerator) / Decimal(s.denominator)).ln()
        return Decimal(g) > -ln_s


def silu_mul_bf16(y_bits, F):
    """h = SiLU(gate) * up correctly rounded (nearest even) to BF16 (bits, [M][F]).

    The float64 value decides the rounding unless it lies within 2^-40
    (relative) of a BF16 midpoint; there the side of the midpoint is decided
    exactly (``_exceeds_midpoint``).  Such near-ties are structural: for a
    tiny gate SiLU(g) * u = g u / 2 + O(g^2), and for a large gate
    SiLU(g) * u = g u (1 - e^-g + ...), where g u / 2 or g u (16-bit
    products of two BF16 values) can be exactly a midpoint.
    """
    y = np.asarray(y_bits, dtype=np.uint16)
    h = silu_mul_f64(y, F)
    bits = round_to_bf16_bits(h)
    _, ex = np.frexp(h)
    q = np.exp2((np.maximum(ex.astype(np.int64) - 1, -126) - 7).astype(np.float64))   # BF16 spacing at h
    m = h / q                                   # exact: the BF16 grid becomes the integers
    fl = np.floor(m)
    near = (h != 0) & (np.abs(m - fl - 0.5) <= np.abs(m) * 2.0 ** -40)
    g_all = bf16_bits_to_f64(y[:, :F])
    u_all = bf16_bits_to_f64(y[:, F:2 * F])
    for i, j in zip(*np.nonzero(near)):
        mid = (Fraction(float(fl[i, j])) + Fraction(1, 2)) * Fraction(float(q[i, j]))
        up = _exceeds_midpoint(float(g_all[i, j]), float(u_all[i, j]), mid)
        lo, hi = float(fl[i, j]) * q[i, j], (float(fl[i, j]) + 1.0) * q[i, j]
        val = (hi if up else lo) if m[i, j] > 0 else (lo if up else hi)
        val = np.copysign(val, h[i, j]) if val == 0 else val        # rounding to zero keeps the sign
        bits[i, j] = round_to_bf16_bits(np.array([val]))[0]     # exact: val is on the BF16 grid
    return bits


def silu_mul_quantize(y_bits, F):
    """(codes [M][F], scales [M][ceil(F/128)]) of the BF16 h, in 1x128 groups."""
    return quant_act_per_token_group(silu_mul_bf16(y_bits, F))


def combine(y_bits, pair_row, weights):
    """out[t] = sum_j weights[t][j] * y[pair_row[t*k+j]] in float64.

    Returns ``(out_f64 [T][H], abs_terms [T][H], out_bf16_bits)``, where
    ``abs_terms`` is sum_j |w * y| (the scale of the rounding error of any
    float32 evaluation of the sum).
    """
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    T, k = w.shape
    y = bf16_bits_to_f64(np.asarray(y_bits, dtype=np.uint16))
    H = y.shape[1]
    rows = np.asarray(pair_row, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, H))
    mag = np.zeros((T, H))
    for j in range(k):
        r = rows[:, j]
        ok = (r >= 0) & (r < y.shape[0])
        term = np.zeros((T, H))
        term[ok] = w[ok, j][:, None] * y[r[ok]]
        out += term
        mag += np.abs(term)
    return out, mag, round_to_bf16_bits(out)
