"""GPU parity of token_importance_weights against the oracle (oracle/tis.py).

Bar: the weight within 2 ulp of the oracle's correctly rounded value (one
float32 exp of at most 1 ulp, the final fma rounding, the oracle's own
rounding); w * A within 6 ulp (that error, one more rounding on each side);
every zero (padding, MIS rejection), every NaN and every clipped bound
identical.  The MIS in/out decision is exact on both sides (float32
difference against fl32(ln C))."""

import math

import numpy as np
import pytest

from helpers import announce
from oracle.tis import MIS, TIS, importance_weights, log_threshold_f32

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MODES = {"tis": TIS, "mis": MIS}


def fb():
    import fp8_blockwise_quantized_quantize_amd as m

    return m


def ulp32(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def run_gpu(lt, lr, C, mode, mask=None, adv=None):
    d = "cuda:0"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    res = fb().token_importance_weights(t(lt), t(lr), C=C, mode=mode,
                                        mask=None if mask is None else t(mask),
                                        advantages=None if adv is None else t(adv))
    torch.cuda.synchronize()
    if adv is None:
        return res.cpu().numpy(), None
    return res[0].cpu().numpy(), res[1].cpu().numpy()


def compare(w, ref, tol_ulp, what):
    w = np.asarray(w, np.float32)
    ref = np.asarray(ref, np.float32)
    assert w.shape == ref.shape
    nan_g, nan_r = np.isnan(w), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{what}: NaN positions differ"
    ok = ~nan_r
    assert np.array_equal(w[ok] == 0, ref[ok] == 0), f"{what}: zero positions differ"
    inf_r = np.isinf(ref) & ok
    assert np.array_equal(w[inf_r], ref[inf_r]), f"{what}: infinities differ"
    fin = ok & ~inf_r
    err = np.abs(w[fin].astype(np.float64) - ref[fin].astype(np.float64)) / np.maximum(ulp32(ref[fin]), 2.0 ** -149)
    worst = float(err.max()) if err.size else 0.0
    print(f"{what}: max error {worst:.2f} ulp over {fin.sum()} values", flush=True)
    assert worst <= tol_ulp, (what, worst)


def check(lt, lr, C, mode, mask=None, adv=None, label=""):
    announce("importance", label, lt.shape, C, mode, mask is not None, adv is not None)
    w, wa = run_gpu(lt, lr, C, mode, mask, adv)
    ref = importance_weights(lt, lr, C=C, mode=MODES[mode], mask=mask, advantages=adv)
    if adv is None:
        compare(w, ref, 2.0, f"w[{label}]")
    else:
        compare(w, ref[0], 2.0, f"w[{label}]")
        compare(wa, ref[1], 6.0, f"wA[{label}]")
        assert not np.any(np.signbit(wa[w == 0]))
    # clipped values are the bounds themselves
    if np.isfinite(C):
        ref_w = ref if adv is None else ref[0]
        at_hi = ref_w == np.float32(C)
        assert np.all(w[at_hi & (np.abs(lt - lr) > 1.0 + math.log(C))] == np.float32(C))
    return w


def random_logprobs(n, seed, spread=1.0):
    rng = np.random.default_rng([77, seed])
    lr = (-rng.exponential(1.0, n)).astype(np.float32)
    lt = (lr + rng.normal(0.0, spread, n)).astype(np.float32)
    return lt, lr


@pytest.mark.parametrize("n", [1, 3, 4, 5, 255, 1023, 1024, 4099, 3 * 1024 + 7, 70001])
@pytest.mark.parametrize("mode", ["tis", "mis"])
def test_sizes_and_ragged_tails(n, mode):
    lt, lr = random_logprobs(n, n)
    rng = np.random.default_rng([78, n])
    mask = (rng.random(n) < 0.7).astype(np.uint8)
    adv = rng.normal(0, 1, n).astype(np.float32)
    check(lt, lr, 2.0, mode, label=f"n={n}")
    check(lt, lr, 2.0, mode, mask=mask, adv=adv, label=f"n={n} mask adv")
    check(lt, lr, 2.0, mode, adv=adv, label=f"n={n} adv")
    check(lt, lr, 2.0, mode, mask=mask, label=f"n={n} mask")


@pytest.mark.parametrize("C", [1.0, 1.25, 2.0, 4.5, 1e4, math.inf])
@pytest.mark.parametrize("mode", ["tis", "mis"])
def test_thresholds(C, mode):
    lt, lr = random_logprobs(50000, 5, spread=3.0)
    check(lt, lr, C, mode, label=f"C={C}")


def test_wide_range_untruncated():
    # |d| up to 80: the rounding of the float32 difference would cost up to
    # ~2^5 ulp in exp; the exact two-term difference keeps the weight within 2.
    rng = np.random.default_rng(11)
    lr = (-rng.uniform(0, 80, 100000)).astype(np.float32)
    lt = (-rng.uniform(0, 80, 100000)).astype(np.float32)
    check(lt, lr, math.inf, "tis", label="wide")
    # tiny differences of large log-probs
    lt2 = (lr + rng.normal(0, 1e-4, lr.size)).astype(np.float32)
    check(lt2, lr, 2.0, "tis", label="tiny d")


def test_special_values():
    lt = np.array([-np.inf, np.nan, -np.inf, 0.0, 200.0, -200.0, 100.0, -120.0, 0.0], np.float32)
    lr = np.array([-1.0, -1.0, -np.inf, np.nan, 0.0, 0.0, 0.0, 0.0, -np.inf], np.float32)
    for C in (2.0, math.inf):
        for mode in ("tis", "mis"):
            check(lt, lr, C, mode, label=f"specials C={C}")
    w, _ = run_gpu(lt, lr, 2.0, "tis")
    assert w[0] == 0.5 and w[4] == 2.0 and w[5] == 0.5 and w[8] == 2.0
    w, _ = run_gpu(lt, lr, math.inf, "tis")
    assert w[6] == np.inf and w[7] == 0.0 and w[8] == np.inf


def test_mis_band_edges_exact():
    edges = []
    for C in (2.0, 1.5, 3.0, 10.0):
        t = log_threshold_f32(C)
        for v in (t, -t, np.nextafter(t, np.float32(9)), -np.nextafter(t, np.float32(9)),
                  np.nextafter(t, np.float32(0)), -np.nextafter(t, np.float32(0))):
            edges.append(v)
    d = np.array(edges, np.float32)
    for base in (0.0, -0.75, -3.0, -17.5):
        lr = np.full(d.shape, np.float32(base))
        lt = (lr + d).astype(np.float32)
        for C in (2.0, 1.5, 3.0, 10.0):
            w = check(lt, lr, C, "mis", label=f"edges C={C} base={base}")
            keep = np.abs(lt - lr) <= log_threshold_f32(C)
            assert np.array_equal(w != 0, keep)


def test_padding_is_never_read_into_the_result():
    rng = np.random.default_rng(12)
    n = 4096 + 5
    lt, lr = random_logprobs(n, 12)
    adv = rng.normal(0, 1, n).astype(np.float32)
    mask = np.ones(n, np.uint8)
    mask[1000:3000] = 0
    mask[-3:] = 0
    lt[mask == 0] = np.nan
    lr[mask == 0] = np.inf
    adv[mask == 0] = np.nan
    w = check(lt, lr, 2.0, "tis", mask=mask, adv=adv, label="nan padding")
    assert np.all(w[mask == 0] == 0)


def test_outputs_stay_in_bounds():
    # outputs are views into larger buffers whose guard region must survive
    d = "cuda:0"
    for n in (1, 6, 1029):
        lt, lr = random_logprobs(n, 100 + n)
        big_w = torch.full((n + 64,), 7.0, device=d)
        big_a = torch.full((n + 64,), 7.0, device=d)
        ltd, lrd = torch.from_numpy(lt).to(d), torch.from_numpy(lr).to(d)
        adv = torch.ones(n, device=d)
        announce("importance guard", n)
        fb().token_importance_weights(ltd, lrd, C=2.0, mode="tis", advantages=adv,
                                      out=big_w[:n], out_adv=big_a[:n])
        torch.cuda.synchronize()
        assert torch.all(big_w[n:] == 7.0) and torch.all(big_a[n:] == 7.0)
        ref = importance_weights(lt, lr, C=2.0)
        compare(big_w[:n].cpu().numpy(), ref, 2.0, f"guard n={n}")


def test_training_batch_full_size():
    # one training batch of the FP8-RL experiments: 32 prompts x 16 responses,
    # padded to 20,000 tokens; every token compared with the oracle
    from synthetic import ROLLOUT_TRAIN_BATCH, rollout_batch

    b = rollout_batch(ROLLOUT_TRAIN_BATCH["responses"], ROLLOUT_TRAIN_BATCH["max_len"], (31, 1))
    for mode in ("tis", "mis"):
        check(b["logp_train"], b["logp_rollout"], 2.0, mode, mask=b["mask"], adv=b["advantages"],
              label=f"train batch {mode}")


def test_binding_rejects_bad_arguments():
    d = "cuda:0"
    x = torch.zeros(8, device=d)
    with pytest.raises(fb().FP8BQError):
        fb().token_importance_weights(x, x, C=0.5)
    with pytest.raises(ValueError):
        fb().token_importance_weights(x, x, mode="other")
    with pytest.raises(TypeError):
        fb().token_importance_weights(x.double(), x.double())
    w = fb().token_importance_weights(torch.zeros(0, device=d), torch.zeros(0, device=d))
    assert w.numel() == 0
