"""Pins of the closed forms against the values the pages print."""
import json
import os

import numpy as np

from oracle import closed_form as cf

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_form.json")))


def rounds_to(x, printed, digits):
    return abs(x - printed) <= 0.5 * 10 ** (-digits) + 1e-12


def test_expected_emitted_printed_value():
    for e in GOLDEN["expected_emitted"]:
        assert rounds_to(cf.expected_emitted(e["alpha"], e["gamma"]), e["value"], e["printed_digits"])


def test_expected_emitted_equals_termwise_sum():
    for a in (0.1, 0.5, 0.62, 0.8, 0.95):
        for g in range(1, 11):
            assert np.isclose(cf.expected_emitted(a, g), sum(a ** k for k in range(g + 1)), rtol=1e-14)
    assert cf.expected_emitted(1.0, 4) == 5.0


def test_emitted_law():
    for a in (0.3, 0.8):
        law = cf.emitted_law(a, 4)
        assert np.isclose(law.sum(), 1.0)
        assert np.isclose((np.arange(1, 6) * law).sum(), cf.expected_emitted(a, 4))
        # P(N >= k+1) = a^k
        for k in range(5):
            assert np.isclose(law[k:].sum(), a ** k)
    per = cf.emitted_law_per_slot([0.8] * 4)
    assert np.allclose(per, cf.emitted_law(0.8, 4))
    assert np.isclose(cf.expected_emitted_per_slot([0.8] * 4), 3.3616)


def test_speedup_printed_values():
    cfac = GOLDEN["cost_factor"]
    assert np.isclose(1 + cfac["gamma"] * cfac["c"], cfac["value"])
    for s in GOLDEN["speedup"]:
        assert rounds_to(cf.speedup(s["alpha"], s["gamma"], s["c"]), s["value"], s["printed_digits"])
    inc = GOLDEN["speedup_increment_0p8_to_0p9"]
    d = cf.speedup(0.9, inc["gamma"], inc["c"]) - cf.speedup(0.8, inc["gamma"], inc["c"])
    assert rounds_to(d, inc["value"], inc["printed_digits"])


def test_layer_skip_claims():
    ls = GOLDEN["layer_skip"]
    c = ls["c"]
    s = [cf.speedup_layer_skip(ls["decreasing_in_gamma_at_alpha"], g, c) for g in range(1, 11)]
    assert all(x > y for x, y in zip(s, s[1:]))
    s9 = [cf.speedup_layer_skip(0.9, g, c) for g in range(1, 16)]
    best = 1 + int(np.argmax(s9))
    lo, hi = ls["best_gamma_range_at_alpha_0p9"]
    assert lo <= best <= hi


def test_monte_carlo_emitted_count():
    rng = np.random.default_rng(0)
    a, g, N = 0.8, 4, 400000
    acc = rng.random((N, g)) < a
    first_rej = np.where(acc.all(1), g, np.argmin(acc, axis=1))
    emitted = first_rej + 1
    assert abs(emitted.mean() - cf.expected_emitted(a, g)) < 5 * np.sqrt(2.57 / N)
