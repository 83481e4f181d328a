"""Closed forms of the verify step's statistics (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Model: every draft is accepted independently with probability alpha (the
simplifying assumption of [Self-spec] section 4.1).  At least k drafts are
accepted with probability alpha^k, so the emitted count N (accepted drafts plus
the one correction/bonus token) has

    P(N = k)       = alpha^(k-1) (1 - alpha),   k = 1..gamma
    P(N = gamma+1) = alpha^gamma
    E[N]           = 1 + sum_{k=1..gamma} alpha^k = (1 - alpha^(gamma+1)) / (1 - alpha)

([Infra-ch8] "how the benefit is computed", [Self-spec] section 4.1; 3.36 at
alpha = 0.8, gamma = 4).  With a per-slot acceptance rate alpha_i the same
argument gives E[N] = 1 + sum_k prod_{i<k} alpha_i.

Speedup: a round costs gamma draft steps of relative cost c plus one target
pass, S = E[N] / (1 + gamma c) ([Infra-ch8] "how the benefit is computed");
the layer-skip variant whose verify reuses the draft's shallow layers costs
1 - c + gamma c ([Self-spec] section 4.2).

Pinned by: the pages' printed values 3.36 (alpha .8, gamma 4) and the
speedups 1.79 / 3.11 and "about 0.7 more at alpha .9" at gamma 4, c = 0.02
(tests/golden/closed_form.json); Monte Carlo of the emitted count.
"""
import numpy as np


def expected_emitted(alpha, gamma):
    """E[N] for a constant acceptance rate alpha (alpha == 1 gives gamma + 1)."""
    a = float(alpha)
    if a == 1.0:
        return float(gamma + 1)
    return (1.0 - a ** (gamma + 1)) / (1.0 - a)


def expected_emitted_per_slot(alphas):
    """E[N] = 1 + sum_{k=1..gamma} prod_{i<k} alpha_i for per-slot rates."""
    e, run = 1.0, 1.0
    for a in alphas:
        run *= float(a)
        e += run
    return e


def emitted_law(alpha, gamma):
    """P(N = k) for k = 1..gamma+1 as a float64 array of length gamma + 1."""
    a = float(alpha)
    law = np.array([a ** (k - 1) * (1.0 - a) for k in range(1, gamma + 1)] + [a ** gamma])
    return law


def emitted_law_per_slot(alphas):
    """P(N = k), k = 1..gamma+1, for per-slot acceptance rates."""
    alphas = [float(a) for a in alphas]
    law, run = [], 1.0
    for a in alphas:
        law.append(run * (1.0 - a))
        run *= a
    law.append(run)
    return np.array(law)


def speedup(alpha, gamma, c):
    """S = E[N] / (1 + gamma c): draft cost c per step, one target pass."""
    return expected_emitted(alpha, gamma) / (1.0 + gamma * c)


def speedup_layer_skip(alpha, gamma, c):
    """S = E[N] / (1 - c + gamma c): verify reuses the draft's first layers."""
    return expected_emitted(alpha, gamma) / (1.0 - c + gamma * c)
