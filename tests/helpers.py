"""Shared test helpers (test infrastructure; imports the oracle, never the reverse)."""

import os
import sys

import numpy as np

from oracle import encode_e4m3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def announce(*parts):
    """Name the case before a GPU step, so a failing step can be identified."""
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def gemm_tolerance_report(y_bits, y_ref):
    """Compare BF16 GPU output bits with the float64 oracle value.

    Acceptance (the task's 1e-2 relative-error bar, made precise): both the
    relative Frobenius error and the worst element error, measured against
    max(|y_ref|, rms(y_ref)), must be <= 1e-2.  Also reports the fraction of
    outputs equal to the oracle's own BF16 rounding.
    """
    y = (np.asarray(y_bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = np.asarray(y_ref, np.float64)
    if ref.size == 0:
        return {"rel_fro": 0.0, "rel_max": 0.0, "exact_bf16_frac": 1.0}
    diff = y - ref
    nref = np.linalg.norm(ref)
    rel_fro = float(np.linalg.norm(diff) / nref) if nref > 0 else float(np.linalg.norm(diff))
    rms = float(np.sqrt(np.mean(ref ** 2)))
    denom = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    rel_max = float(np.max(np.abs(diff) / denom))
    from oracle import round_to_bf16_bits

    exact = float(np.mean(round_to_bf16_bits(ref) == np.asarray(y_bits, np.uint16)))
    return {"rel_fro": rel_fro, "rel_max": rel_max, "exact_bf16_frac": exact}


def assert_gemm_close(y_bits, y_ref, tol=1e-2, min_exact=0.9):
    rep = gemm_tolerance_report(y_bits, y_ref)
    assert rep["rel_fro"] <= tol and rep["rel_max"] <= tol, rep
    assert rep["exact_bf16_frac"] >= min_exact, rep
    return rep


def e4m3_transition_table():
    """Oracle's E4M3 encoder as a step function of the float32 bit pattern.

    For non-negative float32 values the oracle's code is non-decreasing in the
    bit pattern u (0 .. 0x7F7FFFFF).  T[c-1] is the smallest u whose code is
    >= c (c = 1 .. 126), found by binary search with the oracle's own
    encoder, so code(u) == searchsorted(T, u, side='right').  Negative values
    take the same code with the sign bit set.
    """
    table = []
    hi_all = 0x7F7FFFFF
    for c in range(1, 127):
        lo, hi = 0, hi_all
        while lo < hi:
            mid = (lo + hi) // 2
            code = int(encode_e4m3(np.array([mid], np.uint32).view(np.float32))[0])
            if code >= c:
                hi = mid
            else:
                lo = mid + 1
        table.append(lo)
    return np.array(table, np.int64)


def bf16_bits_to_device(bits, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def device_to_bits(t):
    """bfloat16 / int16 device tensor -> uint16 numpy bit patterns."""
    import torch

    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def sampled_gemm_ref(x_rows_bits, w_bits, cols):
    """Oracle W8A8 output at (rows of x_rows_bits) x (cols) from BF16 inputs.

    Quantizes the given activation rows (1x128 groups are row-local) and only
    the 128-row weight blocks that hold the sampled output columns, then
    multiplies the dequantized operands.  Every step is the oracle's.
    """
    from oracle import dequant_act, dequant_weight, quant_act_per_token_group, quant_weight_blockwise

    qa, sa = quant_act_per_token_group(x_rows_bits)
    a = dequant_act(qa, sa)
    cols = np.asarray(cols)
    wrows = np.empty((len(cols), w_bits.shape[1]), np.float64)
    for rb in np.unique(cols // 128):
        sel = np.nonzero(cols // 128 == rb)[0]
        lo, hi = rb * 128, min(w_bits.shape[0], (rb + 1) * 128)
        qw, sw = quant_weight_blockwise(w_bits[lo:hi])
        wrows[sel] = dequant_weight(qw, sw)[cols[sel] - lo]
    return a @ wrows.T


def sample_cols(rng, n, blocks=4, per_block=16):
    """Output columns drawn from a few 128-row weight blocks (cheap for the oracle)."""
    nb = -(-n // 128)
    chosen = rng.choice(nb, size=min(blocks, nb), replace=False)
    cols = []
    for rb in chosen:
        lo, hi = rb * 128, min(n, rb * 128 + 128)
        cols.extend(rng.choice(np.arange(lo, hi), size=min(per_block, hi - lo), replace=False))
    return np.sort(np.array(cols, np.int64))
