"""Pins of the oracle's aligned top-k / top-p verification (CPU only).

[MTP-drafters] 3.1 (top-k and nucleus sampling), [MTP-drafters] 5.2 and [Infra-ch8] "why
the output does not change" (the drafter and the verifier must filter alike),
[MTP-deep-dive] 5.1 (deployed with top_k 64, top_p 0.95).  Pinned by a hand-derived
fixture with a tie at the top-k cut, the unfiltered limit (top_k = V, top_p = 1 is
the plain rule bit for bit), structural properties of the kept set, and a chi-square
test that emitted tokens follow the filtered distribution.
"""
import json
import os

import numpy as np
from scipy import stats

from oracle import rules

HERE = os.path.dirname(os.path.abspath(__file__))


def test_fixture():
    g = json.load(open(os.path.join(HERE, "golden", "filtered_probs.json")))
    l = np.array([g["logits"]], dtype=np.float32)
    for c in g["cases"]:
        p, kept, _ = rules.filtered_probs(l, g["temperature"], c["top_k"], c["top_p"])
        assert np.nonzero(kept[0])[0].tolist() == c["kept"], c
        for k, v in c["p"].items():
            assert abs(float(p[0, int(k)]) - v) < 1e-7, (c, k)
        assert abs(float(p[0].astype(np.float64).sum()) - 1.0) < 1e-6


def test_unfiltered_limit_is_the_plain_rule():
    rng = np.random.default_rng(11)
    B, gamma, V = 64, 3, 12
    l = (rng.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    p_plain = rules.target_probs(l, 0.7)
    p_filt, kept, flags = rules.filtered_probs(l, 0.7, V, 1.0)
    np.testing.assert_array_equal(p_filt, p_plain)
    assert kept.all() and not flags.any()
    q = rng.dirichlet(np.ones(V), size=(B, gamma))
    draft = rng.integers(0, V, size=(B, gamma))
    a = rules.sample_rule(l, draft, q, 0.7, 99, np.arange(B))
    b = rules.sample_rule_filtered(l, draft, q, 0.7, V, 1.0, 99, np.arange(B))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_kept_set_properties():
    rng = np.random.default_rng(12)
    for trial in range(200):
        V = int(rng.integers(1, 30))
        l = (rng.integers(-3, 4, size=(1, V)) * 0.5).astype(np.float32)     # ties happen
        T = float(rng.choice([0.5, 1.0, 2.0]))
        k = int(rng.integers(1, V + 3))
        tp = float(rng.choice([0.3, 0.8, 0.95, 1.0]))
        p, kept, _ = rules.filtered_probs(l, T, k, tp)
        order = sorted(range(V), key=lambda v: (-float(l[0, v]), v))
        n = int(kept.sum())
        assert 1 <= n <= min(k, V)
        assert set(np.nonzero(kept[0])[0].tolist()) == set(order[:n])          # a prefix of the order
        assert np.all(p[0][~kept[0]] == 0) and np.all(p[0][kept[0]] > 0)
        # top-p: renormalised top-k probabilities, cumulative before the last kept < top_p,
        # and the kept mass reaches top_p unless every top-k token is kept
        topk = order[:min(k, V)]
        x = l[0, topk].astype(np.float64)
        pk = np.exp((x - x[0]) / T)
        pk /= pk.sum()
        cum = np.cumsum(pk)
        assert n == 1 or cum[n - 2] < tp
        assert n == len(topk) or cum[n - 1] >= tp
        np.testing.assert_allclose(p[0, topk[:n]], pk[:n] / pk[:n].sum(), rtol=1e-6)


def test_emitted_tokens_follow_the_filtered_distribution():
    """gamma = 1: the first emitted token (the accepted draft, else the correction) has the
    law of the filtered slot-0 distribution; q is the drafter's own filtered distribution."""
    rng = np.random.default_rng(13)
    V, B, T, k, tp = 10, 40000, 1.0, 5, 0.9
    lt = (rng.standard_normal(V) * 1.5).astype(np.float32)
    ld = (lt + rng.standard_normal(V).astype(np.float32))
    l = np.broadcast_to(lt, (B, 2, V)).copy()
    qd, _, _ = rules.filtered_probs(ld[None], T, k, tp)
    q = np.broadcast_to(qd.astype(np.float64), (B, 1, V)).copy()
    draft = rng.choice(V, size=(B, 1), p=qd[0] / qd[0].sum())
    n, tok, _ = rules.sample_rule_filtered(l, draft, q, T, k, tp, 2024, np.arange(B) * 3)
    pt, kept, _ = rules.filtered_probs(lt[None], T, k, tp)
    counts = np.bincount(tok[:, 0], minlength=V)
    assert np.all(counts[~kept[0]] == 0)                  # never outside the filtered support
    exp = pt[0][kept[0]].astype(np.float64) * B
    chi2 = ((counts[kept[0]] - exp) ** 2 / exp).sum()
    assert stats.chi2.sf(chi2, int(kept.sum()) - 1) > 1e-3, chi2
