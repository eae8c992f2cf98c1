"""Token-level importance weights for FP8 rollouts (TIS and MIS).

Test infrastructure only (see ``oracle/__init__.py``).

What is computed ([FP8-RL summary] §3.4.3 "Train-Inference Mismatch and
Importance-Sampling Correction"):

* "The Importance Weight Formula": for each generated token a the weight is
  the ratio of the full-precision training policy's probability of a to the
  FP8 rollout policy's probability of it, w = pi_theta(a|s) / pi_theta^FP8(a|s).
  Both policies hand over log-probabilities, so
      w = exp(logp_train - logp_rollout).
* "Truncated Importance Sampling (TIS)": w_TIS = clip(w, C), i.e. w limited
  to the interval [1/C, C]; the experiments use C = 2 (also §3.4.6, the
  importance-sampling entry of the configuration list).
* The weight multiplies the token's advantage in the policy loss (end of
  "The Importance Weight Formula"), so ``advantages`` optionally yields
  w * A as well.

Readings of what the pages leave open:

* §3.4.5's architecture list says the clip range is [-C, C]; the formula
  paragraph of §3.4.3 and its worked description (below 1/2 -> 1/2, above
  2 -> 2 for C = 2) say [1/C, C].  The latter is taken.
* MIS (masked importance sampling) is only named at the end of §3.4.3 as
  the stronger alternative.  Reading: a token whose weight lies outside
  [1/C, C] gets weight 0 (it is masked out of the loss) instead of being
  clipped; tokens inside keep w.  The in/out decision is taken in the
  log domain in float32: d32 = fl32(logp_train - logp_rollout) is kept iff
  |d32| <= fl32(ln C).  Any implementation that takes the same float32
  decision agrees with this one exactly.
* Log-probabilities and C are float32 values.  The weight is exp of the
  difference of the two inputs, evaluated, clipped and multiplied in
  float64 and rounded once to float32.
* A response mask (padding positions, mask == 0) forces w = 0 and
  w * A = 0 there.
* C must be >= 1 (for C < 1 the interval [1/C, C] is empty); C = inf
  gives the untruncated weights.
* w * A is +0 wherever w is 0 (masked or MIS-rejected tokens), whatever A.
* A NaN difference (NaN input, or -inf - -inf) gives NaN under TIS and 0
  under MIS; logp_train = -inf (probability 0) gives 1/C under TIS.

The ratio-of-probabilities definition, the clip range, the page's worked
numbers and the unbiasedness of untruncated weights are pinned in
``tests/test_oracle_tis.py``.
"""

import math

import numpy as np

TIS = 0
MIS = 1


def log_threshold_f32(C):
    """fl32(ln C): the MIS band edge in float32 (|d32| <= this keeps a token)."""
    return np.float32(math.log(float(C)))


def importance_weights(logp_train, logp_rollout, C=2.0, mode=TIS, mask=None, advantages=None):
    """Per-token TIS / MIS weights.

    logp_train, logp_rollout: float32 arrays of one shape (log pi_theta(a|s),
    log pi_theta^FP8(a|s) of the sampled tokens).  Returns ``w`` (float32),
    or ``(w, w * advantages)`` when ``advantages`` is given.
    """
    lt = np.asarray(logp_train, dtype=np.float32)
    lr = np.asarray(logp_rollout, dtype=np.float32)
    if lt.shape != lr.shape:
        raise ValueError("log-prob arrays differ in shape")
    C = float(np.float32(C))
    if not C >= 1.0:
        raise ValueError("C must be >= 1 (C = inf gives the untruncated weights)")
    if mode not in (TIS, MIS):
        raise ValueError("mode must be TIS or MIS")

    with np.errstate(invalid="ignore", over="ignore"):
        d = lt.astype(np.float64) - lr.astype(np.float64)   # difference in float64
        ratio = np.exp(d)                                    # pi_theta / pi_theta^FP8
        w = np.clip(ratio, 1.0 / C, C)                       # [1/C, C]; NaN stays NaN
        if mode == MIS:
            d32 = lt - lr                                    # float32 IEEE subtraction
            keep = np.abs(d32) <= log_threshold_f32(C)       # NaN -> False
            w = np.where(keep, w, 0.0)
    if mask is not None:
        m = np.asarray(mask)
        if m.shape != lt.shape:
            raise ValueError("mask differs in shape")
        w = np.where(m != 0, w, 0.0)
    with np.errstate(over="ignore"):
        w32 = w.astype(np.float32)                           # beyond the float32 range: inf
    if advantages is None:
        return w32
    a = np.asarray(advantages, dtype=np.float32)
    if a.shape != lt.shape:
        raise ValueError("advantages differ in shape")
    with np.errstate(invalid="ignore", over="ignore"):
        wa = np.where(w == 0.0, 0.0, w * a.astype(np.float64)).astype(np.float32)
    return w32, wa
