"""Pins of the importance-weight oracle (oracle/tis.py) to what the FP8-RL
summary page, section 3.4.3, fixes: the weight is a ratio of the two
policies' probabilities, TIS limits it to [1/C, C], the page's worked
numbers, and the unbiasedness of the untruncated weights."""

import math
import os

import numpy as np
import pytest

from oracle.tis import MIS, TIS, importance_weights, log_threshold_f32

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tis_page_examples.txt")


def f32log(p):
    return np.float32(np.log(np.asarray(p, dtype=np.float64)))


def ulp32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)


def load_golden():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([float(v) for v in line.split()])
    return np.array(rows)


def test_page_examples():
    g = load_golden()
    assert len(g) >= 5
    pt, pr, C, raw, tis, kept = g.T
    lt, lr = f32log(pt), f32log(pr)
    for i in range(len(g)):
        w_raw = importance_weights(lt[i:i + 1], lr[i:i + 1], C=math.inf)[0]
        # the float32 log-probs carry ~1e-7 relative error into the ratio
        assert abs(w_raw - raw[i]) <= 2e-6 * raw[i], (i, w_raw, raw[i])
        w_tis = importance_weights(lt[i:i + 1], lr[i:i + 1], C=C[i], mode=TIS)[0]
        if tis[i] in (C[i], 1.0 / C[i]):
            assert w_tis == np.float32(tis[i])        # clipped: the bound itself, exactly
        else:
            assert abs(w_tis - tis[i]) <= 2e-6 * tis[i]
        w_mis = importance_weights(lt[i:i + 1], lr[i:i + 1], C=C[i], mode=MIS)[0]
        assert (w_mis != 0) == bool(kept[i])
        if kept[i]:
            assert w_mis == w_tis


def test_weight_is_ratio_of_probabilities():
    # w = p_train / p_rollout computed as a quotient of probabilities, not via
    # the log difference: catches a swapped operand or a wrong sign.
    rng = np.random.default_rng(1)
    lt = np.float32(-rng.exponential(3.0, 4000))
    lr = np.float32(lt + rng.normal(0.0, 0.5, 4000))
    lr = np.minimum(lr, np.float32(0.0))
    quotient = np.exp(lt.astype(np.float64)) / np.exp(lr.astype(np.float64))
    w = importance_weights(lt, lr, C=math.inf)
    assert np.all(np.abs(w - quotient) <= ulp32(quotient))
    # and the TIS weight is that quotient limited to [1/2, 2]
    w2 = importance_weights(lt, lr, C=2.0)
    ref = np.minimum(np.maximum(quotient, 0.5), 2.0)
    assert np.all(np.abs(w2 - ref) <= ulp32(ref))
    assert np.any(w2 == 2.0) and np.any(w2 == 0.5) and np.any((w2 > 0.5) & (w2 < 2.0))


def test_untruncated_weights_are_unbiased():
    # Section 3.4.3 "Why this form": E_{a~q}[w(a) f(a)] = E_{a~p}[f(a)] when q
    # covers the support of p.  Exact expectation over a small vocabulary.
    rng = np.random.default_rng(2)
    rev_err = []
    for trial in range(20):
        V = 16
        p = rng.dirichlet(np.ones(V))
        q = 0.7 * p + 0.3 * rng.dirichlet(np.ones(V))   # rollout policy close to p
        f = rng.normal(size=V)
        w = importance_weights(f32log(p), f32log(q), C=math.inf).astype(np.float64)
        lhs = float(np.sum(q * w * f))
        rhs = float(np.sum(p * f))
        assert abs(lhs - rhs) <= 1e-5 * (np.sum(np.abs(p * f)) + 1e-30), trial
        # the reversed ratio would estimate a different expectation
        w_rev = importance_weights(f32log(q), f32log(p), C=math.inf).astype(np.float64)
        rev_err.append(abs(float(np.sum(q * w_rev * f)) - rhs))
    assert np.median(rev_err) > 1e-2


def test_swap_gives_reciprocal_and_monotone():
    rng = np.random.default_rng(3)
    lt = np.float32(-rng.exponential(2.0, 3000))
    lr = np.float32(-rng.exponential(2.0, 3000))
    a = importance_weights(lt, lr, C=2.0).astype(np.float64)
    b = importance_weights(lr, lt, C=2.0).astype(np.float64)
    assert np.all(np.abs(a * b - 1.0) <= 3 * 2.0 ** -24)
    # non-decreasing in logp_train, non-increasing in logp_rollout
    xs = np.float32(np.sort(rng.uniform(-5, 1, 2000)))
    zero = np.zeros_like(xs)
    wt = importance_weights(xs, zero, C=3.0)
    assert np.all(np.diff(wt) >= 0)
    wr = importance_weights(zero, xs, C=3.0)
    assert np.all(np.diff(wr) <= 0)


def test_clip_bounds_exact_and_c_one():
    lt = np.float32([50.0, -50.0, 0.0, 1e-3, -1e-3])
    lr = np.zeros(5, np.float32)
    w = importance_weights(lt, lr, C=2.0)
    assert w[0] == 2.0 and w[1] == 0.5 and w[2] == 1.0
    w1 = importance_weights(lt, lr, C=1.0)
    assert np.all(w1 == 1.0)
    m1 = importance_weights(lt, lr, C=1.0, mode=MIS)
    assert list(m1) == [0.0, 0.0, 1.0, 0.0, 0.0]


def test_mis_band_edge_in_float32():
    t = log_threshold_f32(2.0)
    assert t == np.float32(0.6931472)
    up = np.nextafter(t, np.float32(1.0))
    lt = np.array([t, -t, up, -up, 0.0], np.float32)
    lr = np.zeros(5, np.float32)
    w = importance_weights(lt, lr, C=2.0, mode=MIS)
    assert w[0] > 0 and w[1] > 0 and w[2] == 0 and w[3] == 0 and w[4] == 1.0
    # kept tokens carry exactly the TIS weight
    assert w[0] == importance_weights(lt[:1], lr[:1], C=2.0)[0]
    # the decision uses the float32 difference: both inputs away from zero
    lr2 = np.full(5, np.float32(-3.0))
    lt2 = (lr2 + lt).astype(np.float32)
    d32 = lt2 - lr2
    w2 = importance_weights(lt2, lr2, C=2.0, mode=MIS)
    assert np.array_equal(w2 != 0, np.abs(d32) <= t)


def test_mask_and_weighted_advantage():
    rng = np.random.default_rng(4)
    n = 1000
    lt = np.float32(-rng.exponential(1.0, n))
    lr = np.float32(lt + rng.normal(0, 0.6, n))
    adv = np.float32(rng.normal(0, 1, n))
    mask = (rng.random(n) < 0.8).astype(np.uint8)
    for mode in (TIS, MIS):
        w, wa = importance_weights(lt, lr, C=2.0, mode=mode, mask=mask, advantages=adv)
        w_nomask = importance_weights(lt, lr, C=2.0, mode=mode)
        assert np.all(w[mask == 0] == 0) and np.all(wa[mask == 0] == 0)
        assert np.array_equal(w[mask == 1], w_nomask[mask == 1])
        prod = w.astype(np.float64) * adv.astype(np.float64)
        assert np.all(np.abs(wa - prod) <= 2 * ulp32(prod))   # w rounded once more here
        assert not np.any(np.signbit(wa[w == 0]))


def test_special_values_and_errors():
    lt = np.array([-np.inf, np.nan, -np.inf, 0.0], np.float32)
    lr = np.array([-1.0, -1.0, -np.inf, np.nan], np.float32)
    w = importance_weights(lt, lr, C=2.0)
    assert w[0] == 0.5 and np.isnan(w[1]) and np.isnan(w[2]) and np.isnan(w[3])
    m = importance_weights(lt, lr, C=2.0, mode=MIS)
    assert list(m) == [0.0, 0.0, 0.0, 0.0]
    with pytest.raises(ValueError):
        importance_weights(lt, lr, C=0.5)
    with pytest.raises(ValueError):
        importance_weights(lt, lr, C=float("nan"))
    with pytest.raises(ValueError):
        importance_weights(lt, lr, mode=7)
