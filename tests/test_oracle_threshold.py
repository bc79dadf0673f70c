"""Pins for the oracle's calibrated-threshold lowering (CPU only).

Model-Optimizer "Skip-Softmax Sparse Attention for Diffusion Models", "Threshold Modes" table and
the exported config example: threshold_scale_factor = a * exp(b * target_sparsity) with the
prefill coefficients a = 1443.49, b = 4.30 (tests/golden/page_constants.json); the backend divides
by seq_k and the kernel uses log2 of the result.  The values are checked against Python's
``decimal`` module at 50 significant digits (an independent exp/ln), and against the model's
structural invariants.
"""
import decimal
import json
import math
import os

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
