"""Pins for the oracle's calibrated-threshold lowering and log-space calibration fit (CPU only).

Model-Optimizer "Skip-Softmax Sparse Attention for Diffusion Models", "Threshold Modes" table and
the exported config example: threshold_scale_factor = a * exp(b * target_sparsity) with the
prefill coefficients a = 1443.49, b = 4.30 (tests/golden/page_constants.json); the backend divides
by seq_k and the kernel uses log2 of the result.  The values are checked against Python's
``decimal`` module at 50 significant digits (an independent exp/ln), and against the model's
structural invariants.  The fit is checked by recovering the page's (a, b) from exact trials, against
numpy.polyfit on noisy trials, and by dropping trials that carry no information.
"""
import decimal
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _consts():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        return json.load(f)


def _decimal_threshold(a, b, s, seq_k):
    ctx = decimal.Context(prec=50)
    D = decimal.Decimal
    sf = ctx.multiply(D(repr(a)), ctx.exp(ctx.multiply(D(repr(b)), D(repr(s)))))
    lam = ctx.divide(sf, D(seq_k))
    l2 = ctx.divide(ctx.ln(lam), ctx.ln(D(2)))
    return float(sf), float(lam), float(l2)


@pytest.mark.parametrize("s", [0.0, 0.3, 0.5, 0.613, 0.7, 0.9, 0.999])
@pytest.mark.parametrize("seq_k", [1, 256, 4096, 8192, 16257, 32760])
def test_matches_decimal(s, seq_k):
    c = _consts()["calibration_prefill"]
    got = oracle.threshold(c["a"], c["b"], s, seq_k)
    exp = _decimal_threshold(c["a"], c["b"], s, seq_k)
    for g, e in zip(got, exp):
        assert abs(g - e) <= 4e-16 * max(1.0, abs(e))


def test_structure():
    c = _consts()["calibration_prefill"]
    a, b = c["a"], c["b"]
    assert oracle.threshold(a, b, 0.0, 1)[0] == a
    s1, s2 = 0.2, 0.65
    sf1, sf2 = oracle.threshold(a, b, s1, 1)[0], oracle.threshold(a, b, s2, 1)[0]
    assert abs(math.log(sf2) - math.log(sf1) - b * (s2 - s1)) < 1e-13
    for seq_k in (1, 777, 32760):
        sf, lam, l2 = oracle.threshold(a, b, 0.5, seq_k)
        assert abs(lam * seq_k - sf) < 1e-12 * sf
        assert abs(2.0 ** l2 - lam) < 1e-14 * lam


def test_page_fixed_example_is_a_plain_lambda():
    # The fixed-threshold example passes lambda directly; the kernel only takes log2 of it.
    lam = _consts()["fixed_threshold_example"]["lambda"]
    assert abs(math.log2(lam) - (-0.700005)) < 1e-6


@pytest.mark.parametrize("args", [(0.0, 4.3, 0.5, 10), (-1.0, 4.3, 0.5, 10),
                                  (1443.49, float("inf"), 0.5, 10), (1443.49, 4.3, 1.0, 10),
                                  (1443.49, 4.3, -0.1, 10), (1443.49, 4.3, 0.5, 0)])
def test_rejects(args):
    with pytest.raises(ValueError):
        oracle.threshold(*args)


# ---- log-space calibration fit --------------------------------------------------------------------
# Model-Optimizer "Skip-Softmax Sparse Attention for Diffusion Models", introduction: the
# exponential model is calibrated once from trial thresholds, log-space fitting recommended.

def test_fit_recovers_page_coefficients_from_exact_trials():
    c = _consts()["calibration_prefill"]
    seq_k = 32760
    s = np.array([0.31, 0.42, 0.5, 0.58, 0.66, 0.81])
    lam = c["a"] * np.exp(c["b"] * s) / seq_k
    a, b, lo, hi = oracle.fit_threshold(lam, s, seq_k)
    assert abs(a - c["a"]) < 1e-10 * c["a"] and abs(b - c["b"]) < 1e-12
    assert (lo, hi) == (0.31, 0.81)
    for si, li in zip(s, lam):   # the fitted model lowers each target back to its trial
        assert abs(oracle.threshold(a, b, si, seq_k)[1] - li) < 1e-12 * li


def test_fit_matches_numpy_polyfit_on_noisy_trials():
    rng = np.random.default_rng(7)
    s = np.sort(rng.uniform(0.2, 0.9, 12))
    seq_k = 8192
    lam = 900.0 * np.exp(5.1 * s + rng.normal(0, 0.3, s.size)) / seq_k
    a, b, _, _ = oracle.fit_threshold(lam, s, seq_k)
    slope, icept = np.polyfit(s, np.log(lam * seq_k), 1)
    assert abs(b - slope) < 1e-10 and abs(math.log(a) - icept) < 1e-10


def test_fit_ignores_trials_without_information():
    seq_k = 4096
    s = np.array([0.35, 0.5, 0.7])
    lam = 1443.49 * np.exp(4.3 * s) / seq_k
    base = oracle.fit_threshold(lam, s, seq_k)
    # no tile skipped, every tile skipped, lambda = 0: all dropped
    lam2 = np.concatenate([lam, [1e-4, 50.0, 0.0]])
    s2 = np.concatenate([s, [0.0, 1.0, 0.4]])
    assert oracle.fit_threshold(lam2, s2, seq_k) == base
    with pytest.raises(ValueError):
        oracle.fit_threshold(lam2[3:], s2[3:], seq_k)
    with pytest.raises(ValueError):
        oracle.fit_threshold([0.1, 0.2], [0.5, 0.5], seq_k)


def test_workload_constants_are_the_pages():
    import workloads as W
    c = _consts()
    assert (W.CALIB_A, W.CALIB_B) == (c["calibration_prefill"]["a"], c["calibration_prefill"]["b"])
    assert W.THRESHOLD_TRIALS == c["threshold_trials"]["values"]
