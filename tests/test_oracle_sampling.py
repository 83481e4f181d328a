"""Pins of the oracle's sampling rule: exact output law, closed form, chi-square.

The exact enumeration runs the oracle's own acceptance test (on its 24-bit
uniform grid), its first-rejection logic and its choice of the resampling
row, with every random source enumerated exactly.  Target and draft
probabilities are dyadic rationals whose draft values are powers of two, so
the 24-bit acceptance probability equals min(1, p/q) exactly and float32
holds every value; the resulting law of emitted tokens must then equal the
target's, position by position ([MTP-deep-dive] section 2.2: the output
marginal equals p; [Infra-ch8] "why the output does not change";
[Self-spec] section 3.2).
"""
import itertools
from fractions import Fraction as F

import numpy as np
import pytest

from oracle import closed_form, philox, rules

GRID = 1 << 24


def accept_count(px, qx):
    """Number of 24-bit grid points u with the oracle's accepts(u, q, p) true
    (monotone in u, found by bisection on the oracle's own predicate)."""
    lo, hi = 0, GRID          # accepts at k/GRID for k < answer
    if not rules.accepts(0.0, qx, px):
        return 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if rules.accepts(mid / GRID, qx, px):
            lo = mid
        else:
            hi = mid
    return lo + 1


def exact_law(p, q):
    """Exact law of one verify round built from the oracle's pieces.

    ``p``: [gamma+1][V] Fractions, ``q``: [gamma][V] Fractions.  Returns a dict
    mapping emitted token tuples to probabilities.
    """
    gamma, V = len(q), len(p[0])
    p32 = np.array([[float(x) for x in row] for row in p], dtype=np.float32)[None]
    q64 = np.array([[float(x) for x in row] for row in q])[None]
    for i in range(gamma + 1):   # exactness of the float32 representation
        assert all(F(float(p32[0, i, v])) == p[i][v] for v in range(V))
    law = {}
    for xs in itertools.product(range(V), repeat=gamma):
        px_draft = F(1)
        for i, x in enumerate(xs):
            px_draft *= q[i][x]
        if px_draft == 0:
            continue
        # per-slot acceptance probability on the 24-bit grid, and a representative
        # u of each outcome
        acc, u_acc, u_rej = [], [], []
        for i, x in enumerate(xs):
            c = accept_count(float(p32[0, i, x]), float(q64[0, i, x]))
            acc.append(F(c, GRID))
            u_acc.append((c - 1) / GRID if c > 0 else None)
            u_rej.append(c / GRID if c < GRID else None)
        for outcome in itertools.product((True, False), repeat=gamma):
            pr = px_draft
            u = []
            for i, o in enumerate(outcome):
                pr *= acc[i] if o else 1 - acc[i]
                u.append(u_acc[i] if o else u_rej[i])
            if pr == 0:
                continue
            n, _ = rules.accept_slots(p32, q64, np.array([xs]), np.array([u], dtype=np.float64))
            k = int(n[0])
            r = rules.resample_rows(p32, q64, n)[0]
            rf = [F(float(v)) for v in r]
            z = sum(rf)
            for y in range(V):
                if rf[y] == 0:
                    continue
                key = tuple(xs[:k]) + (y,)
                law[key] = law.get(key, F(0)) + pr * rf[y] / z
    return law


def check_law_is_target(law, p):
    gamma = len(p) - 1
    V = len(p[0])
    assert sum(law.values()) == 1
    # P(prefix accepted and next token y) = P(prefix accepted) * p_k(y)
    for k in range(gamma + 1):
        for prefix in itertools.product(range(V), repeat=k):
            reach = sum(pr for t, pr in law.items() if len(t) > k and t[:k] == prefix)
            for y in range(V):
                got = sum(pr for t, pr in law.items() if len(t) > k and t[:k] == prefix and t[k] == y)
                assert got == reach * p[k][y], (k, prefix, y)
        # first token overall
    for y in range(V):
        assert sum(pr for t, pr in law.items() if t[0] == y) == p[0][y]


def dyadic_case(rng, V, gamma, zero_q=False, zero_p=False):
    qs_base = {4: [F(1, 2), F(1, 4), F(1, 8), F(1, 8)],
               8: [F(1, 4), F(1, 4), F(1, 8), F(1, 8), F(1, 16), F(1, 16), F(1, 16), F(1, 16)],
               3: [F(1, 2), F(1, 4), F(1, 4)]}[V]
    p = []
    for _ in range(gamma + 1):
        a = rng.integers(0 if zero_p else 1, 9, V)
        if a.sum() == 0:
            a[0] = 1
        s = int(a.sum())
        # make the denominator a power of two: scale to 64ths by adjusting the last entry
        num = [int(x) * 64 // s for x in a]
        num[int(np.argmax(a))] += 64 - sum(num)
        p.append([F(x, 64) for x in num])
    q = []
    for _ in range(gamma):
        perm = rng.permutation(V)
        row = [qs_base[j] for j in perm]
        if zero_q:   # merge two equal smallest entries: still powers of two
            mn = min(row)
            j, k = [i for i in range(V) if row[i] == mn][:2]
            row[k] += row[j]
            row[j] = F(0)
        q.append(row)
    return p, q


@pytest.mark.parametrize("V,gamma,zero_q,zero_p,seed", [
    (3, 1, False, False, 0), (3, 2, False, False, 1), (4, 2, False, False, 2),
    (4, 2, True, False, 3), (4, 2, False, True, 4), (8, 1, False, False, 5),
    (8, 2, True, True, 6),
])
def test_exact_output_law_equals_target(V, gamma, zero_q, zero_p, seed):
    rng = np.random.default_rng(seed)
    p, q = dyadic_case(rng, V, gamma, zero_q, zero_p)
    law = exact_law(p, q)
    check_law_is_target(law, p)
    # P(at least k accepted) = prod_{i<k} alpha_i
    for k in range(gamma + 1):
        reach = sum(pr for t, pr in law.items() if len(t) > k)
        expect = F(1)
        for i in range(k):
            expect *= sum(min(p[i][v], q[i][v]) for v in range(V))
        assert reach == expect


def test_exact_law_detects_planted_mistakes(monkeypatch):
    """A wrong acceptance direction, a wrong residual sign, or the lossy
    shortcuts of [Self-spec] section 3.1/3.2 break the exact law."""
    rng = np.random.default_rng(11)
    p, q = dyadic_case(rng, 4, 2)

    def law_fails():
        try:
            check_law_is_target(exact_law(p, q), p)
        except AssertionError:
            return True
        return False

    assert not law_fails()
    with monkeypatch.context() as m:   # accept with probability min(1, q/p)
        m.setattr(rules, "accepts", lambda u, qx, px: np.asarray(u) * px < qx)
        assert law_fails()
    orig = rules.residual_rows
    with monkeypatch.context() as m:   # residual max(0, q - p)
        m.setattr(rules, "residual_rows", lambda pr, qr: orig(np.asarray(qr, np.float32), pr))
        assert law_fails()
    with monkeypatch.context() as m:   # accept every draft without correction
        m.setattr(rules, "accepts", lambda u, qx, px: np.ones(np.shape(u), bool) | (np.asarray(px) >= 0))
        assert law_fails()
    with monkeypatch.context() as m:   # resample from p instead of the residual
        m.setattr(rules, "residual_rows", lambda pr, qr: np.asarray(pr, np.float32))
        assert law_fails()


def run_stats(case_rounds, gamma=4, V=32, alpha=0.8, seed_key=123, chunk=100000):
    """Vectorised config-2-style run through the full oracle rule with Philox."""
    rng = np.random.default_rng(seed_key)
    p = rng.dirichlet(np.full(V, 0.5), size=gamma + 1)
    q = np.empty((gamma, V))
    for j in range(gamma):
        while True:
            r = rng.dirichlet(np.full(V, 0.5))
            tv = 0.5 * np.abs(p[j] - r).sum()
            if tv >= 1 - alpha:
                break
        lam = (1 - alpha) / tv
        q[j] = (1 - lam) * p[j] + lam * r
    q32 = q.astype(np.float32)
    l = np.log(p).astype(np.float32)
    ns, toks = [], []
    for c0 in range(0, case_rounds, chunk):
        B = min(chunk, case_rounds - c0)
        d = np.empty((B, gamma), np.int64)
        for j in range(gamma):
            cdf = np.cumsum(q32[j].astype(np.float64))
            d[:, j] = np.minimum(np.searchsorted(cdf, rng.random(B) * cdf[-1], side="right"), V - 1)
        n, tok, _ = rules.sample_rule(np.broadcast_to(l, (B, gamma + 1, V)), d,
                                      np.broadcast_to(q32, (B, gamma, V)), 1.0, 0xABC, np.zeros(B, np.int64), seq0=c0)
        ns.append(n)
        toks.append(tok)
    p32 = rules.target_probs(l, 1.0).astype(np.float64)
    return p32, q32, np.concatenate(ns), np.concatenate(toks)


def test_statistics_match_closed_form_and_target():
    rounds = 200000
    gamma = 4
    p32, q32, n, tok = run_stats(rounds)
    alphas = rules.acceptance_rate(p32[:gamma], q32)
    assert np.allclose(alphas, 0.8, atol=1e-5)
    emitted = n + 1
    law = closed_form.emitted_law_per_slot(alphas)
    mean = closed_form.expected_emitted_per_slot(alphas)
    var = float(((np.arange(1, gamma + 2) - mean) ** 2 * law).sum())
    se = np.sqrt(var / rounds)
    assert abs(emitted.mean() - mean) < 5 * se
    # law of N: chi-square with gamma dof
    cnt = np.bincount(emitted, minlength=gamma + 2)[1:]
    exp = law * rounds
    chi2 = ((cnt - exp) ** 2 / exp).sum()
    assert chi2 < 25  # 4 dof, p ~ 5e-5
    # emitted token at position k ~ p_k among rounds reaching slot k
    for k in range(gamma + 1):
        sel = n >= k
        counts = np.bincount(tok[sel, k], minlength=32).astype(float)
        e = p32[k] * sel.sum()
        keep = e >= 5
        chi = ((counts[keep] - e[keep]) ** 2 / e[keep]).sum() + \
            (counts[~keep].sum() - e[~keep].sum()) ** 2 / max(e[~keep].sum(), 1e-9)
        dof = keep.sum()
        assert chi < dof + 6 * np.sqrt(2 * dof) + 10, (k, chi, dof)


def test_closed_form_mean_at_alpha_08():
    assert abs(closed_form.expected_emitted(0.8, 4) - 3.3616) < 1e-12


def test_q_equals_p_accepts_everything():
    rng = np.random.default_rng(5)
    B, g, V = 400, 4, 20
    l = rng.standard_normal((B, g + 1, V)).astype(np.float32)
    p32 = rules.target_probs(l, 1.0)
    q = p32[:, :g].astype(np.float64)
    d = np.array([[rng.choice(V, p=q[b, i] / q[b, i].sum()) for i in range(g)] for b in range(B)])
    n, tok, _ = rules.sample_rule(l, d, q, 1.0, 7, np.zeros(B, np.int64))
    assert np.all(n == g)
    assert np.array_equal(tok[:, :g], d)


def test_disjoint_supports_reject_first_slot():
    B, g, V = 100, 3, 10
    l = np.full((B, g + 1, V), -1e4, np.float32)
    l[:, :, :5] = 0.0                       # p supported on 0..4
    q = np.zeros((B, g, V))
    q[:, :, 5:] = 0.2                       # q supported on 5..9
    rng = np.random.default_rng(6)
    d = rng.integers(5, 10, (B, g))
    n, tok, _ = rules.sample_rule(l, d, q, 1.0, 8, np.zeros(B, np.int64))
    assert np.all(n == 0)
    assert np.all((tok[:, 0] >= 0) & (tok[:, 0] < 5))
    assert np.all(tok[:, 1:] == -1)


def test_gumbel_sampler_chi_square():
    """Gumbel-max with the Philox uniforms samples r / sum(r)."""
    V = 32
    rng = np.random.default_rng(7)
    r = rng.dirichlet(np.full(V, 0.7)).astype(np.float32)
    r[3] = 0.0
    N = 100000
    s = rules.gumbel_scores(np.broadcast_to(r, (N, V)), 42, np.arange(N), np.full(N, 9))
    y = np.argmax(s, axis=-1)
    assert not np.any(y == 3)
    counts = np.bincount(y, minlength=V).astype(float)
    e = r.astype(np.float64) / r.sum() * N
    keep = e >= 5
    chi = ((counts[keep] - e[keep]) ** 2 / e[keep]).sum()
    dof = keep.sum() - 1
    assert chi < dof + 6 * np.sqrt(2 * dof)


def test_independent_streams_per_position_and_sequence():
    """Different sequences and positions draw different uniforms
    ([Self-spec] section 3.3)."""
    u = philox.accept_uniform(5, np.arange(64)[:, None], np.arange(64)[None, :])
    assert len(np.unique(u)) > 4090
