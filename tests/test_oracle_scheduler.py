"""Pins of the confidence-head / prefix-survival / scheduler oracle: the
pages' worked example, closed forms and the early-stop behaviour."""

import os

import numpy as np

from oracle import scheduler as S

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    vals = {}
    with open(os.path.join(HERE, "golden", "scheduler_worked_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, *nums = line.split()
                vals[key] = [float(x) for x in nums]
    return vals


def test_worked_example():
    g = _golden()
    for c3 in (0.0, 0.3, 0.99):  # the page's third confidence is cut off; the choice must not depend on it
        a = S.prefix_survival(g["confidence"] + [c3])
        th = S.thetas(a, g["sps"])
        np.testing.assert_array_equal(np.round(th[:3], 2), g["theta"])
        assert S.verify_length(a, g["sps"]) == int(g["chosen_length"][0])


def test_early_stop_is_causal():
    """Theta dips at l = 1 and would peak later: the causal search stops at 0
    and never looks past the first drop."""
    a = np.array([0.9, 0.9, 0.9])
    sps = np.array([1.0, 0.4, 0.4, 0.4])
    th = S.thetas(a, sps)
    assert th[1] < th[0] and th[3] > th[0]
    assert S.verify_length(a, sps) == 0


def test_flat_profile_takes_every_draft_and_zero_confidence_none():
    a = S.prefix_survival([0.6, 0.5, 0.9, 0.2])
    assert S.verify_length(a, np.ones(5)) == 4
    assert S.verify_length(np.zeros(4), np.array([1.0, 0.99, 0.98, 0.97, 0.96])) == 0


def test_prefix_survival_is_running_product():
    c = np.array([[0.5, 0.5, 0.5], [1.0, 0.2, 0.0]])
    np.testing.assert_array_equal(S.prefix_survival(c), [[0.5, 0.25, 0.125], [1.0, 0.2, 0.0]])


def test_confidence_closed_forms():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 12))
    assert np.allclose(S.confidence(h, np.zeros(12), 0.3), 1.0 / (1.0 + np.exp(-0.3)))
    w = np.zeros(12); w[4] = 2.0
    np.testing.assert_allclose(S.confidence(h, w, -1.0), 1.0 / (1.0 + np.exp(-(2.0 * h[:, 4] - 1.0))), rtol=1e-15)
    # Markov input: W1 = I (V = r = 6), weight_e one-hot at j -> adds 3 exactly when prev == j
    w1 = np.eye(6)
    we = np.zeros(6); we[2] = 3.0
    prev = np.array([2, 0, 2, 5, 1])
    got = S.confidence(h, np.zeros(12), 0.0, w1, prev, we)
    np.testing.assert_allclose(got, np.where(prev == 2, 1.0 / (1.0 + np.exp(-3.0)), 0.5), rtol=1e-15)
