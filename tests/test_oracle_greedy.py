"""Pins of the oracle's greedy rule: the pages' worked example and brute force."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import rules

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def logits_with_argmax(targets, V, rng, ties):
    """float32 logits [B, G1, V] whose lowest-index argmax per slot is ``targets``.

    With ``ties`` some entries after the target copy its value, so only the
    lowest-index rule picks the target.
    """
    B, G1 = targets.shape
    l = rng.uniform(-1, 0.5, (B, G1, V)).astype(np.float32)
    for b in range(B):
        for i in range(G1):
            t = targets[b, i]
            l[b, i, t] = 1.0
            if ties:
                for j in range(t + 1, V):
                    if rng.random() < 0.5:
                        l[b, i, j] = 1.0
    return l


def test_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    vocab = g["vocab"]
    idx = {t: i for i, t in enumerate(vocab)}
    V = len(vocab)
    targets = np.array([[idx[t] for t in g["target_choice_per_slot"]]])
    rng = np.random.default_rng(0)
    l32 = logits_with_argmax(targets, V, rng, ties=False)
    for case in g["cases"]:
        draft = np.array([[idx[t] for t in case["draft"]]])
        n, tokens, flagged = rules.greedy_rule(l32, draft)
        assert int(n[0]) == case["accepted"]
        emitted = [vocab[t] for t in tokens[0] if t >= 0]
        assert emitted == case["emitted"]
        assert not flagged[0]


def check_greedy_properties(argmaxes, draft, n, tokens):
    """The properties that determine the greedy output uniquely."""
    gamma = draft.shape[0]
    k = int(n)
    assert 0 <= k <= gamma
    for j in range(k):                       # accepted drafts equal the target's choice
        assert draft[j] == argmaxes[j] and tokens[j] == draft[j]
    assert tokens[k] == argmaxes[k]          # then the target's own token
    assert k == gamma or draft[k] != argmaxes[k]   # stop at the first disagreement
    assert all(t == -1 for t in tokens[k + 1:])


def test_brute_force_all_tuples():
    """V = 8, gamma = 2: every argmax tuple x every draft tuple (32768 cases),
    half of them with ties resolved to the lowest index."""
    V, gamma = 8, 2
    arg = np.array(list(itertools.product(range(V), repeat=gamma + 1)))
    drafts = np.array(list(itertools.product(range(V), repeat=gamma)))
    A = np.repeat(arg, len(drafts), axis=0)
    D = np.tile(drafts, (len(arg), 1))
    rng = np.random.default_rng(1)
    l32 = logits_with_argmax(A, V, rng, ties=False)
    # ties on a random half
    half = rng.random(len(A)) < 0.5
    for b in np.nonzero(half)[0][:4000]:
        for i in range(gamma + 1):
            for j in range(A[b, i] + 1, V):
                if rng.random() < 0.5:
                    l32[b, i, j] = 1.0
    n, tokens, _ = rules.greedy_rule(l32, D)
    for b in range(len(A)):
        check_greedy_properties(A[b], D[b], n[b], tokens[b])


def test_brute_force_gamma3_small_vocab():
    V, gamma = 3, 3
    arg = np.array(list(itertools.product(range(V), repeat=gamma + 1)))
    drafts = np.array(list(itertools.product(range(V), repeat=gamma)))
    A = np.repeat(arg, len(drafts), axis=0)
    D = np.tile(drafts, (len(arg), 1))
    l32 = logits_with_argmax(A, V, np.random.default_rng(2), ties=True)
    n, tokens, _ = rules.greedy_rule(l32, D)
    for b in range(len(A)):
        check_greedy_properties(A[b], D[b], n[b], tokens[b])


def test_out_of_range_draft_is_rejected():
    l32 = np.zeros((2, 3, 5), np.float32)
    l32[:, :, 2] = 1
    n, tokens, _ = rules.greedy_rule(l32, np.array([[2, -1], [2, 5]]))
    assert n.tolist() == [1, 1]
    assert tokens.tolist() == [[2, 2, -1], [2, 2, -1]]


def test_greedy_flags_near_ties():
    l32 = np.zeros((1, 2, 4), np.float32)
    l32[0, 0, 1] = 1.0
    l32[0, 0, 2] = 1.0 - 5e-4
    l32[0, 1, 3] = 1.0
    _, _, flagged = rules.greedy_rule(l32, np.array([[1]]))
    assert flagged[0]
    l32[0, 0, 2] = 0.5
    _, _, flagged = rules.greedy_rule(l32, np.array([[1]]))
    assert not flagged[0]


def test_sampling_at_zero_temperature_is_greedy():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 5, 40))
    d = np.argmax(l[:, :4] + 0.3 * rng.standard_normal((50, 4, 40)), axis=-1)
    q = rng.dirichlet(np.ones(40), size=(50, 4))
    a = rules.verify_sample(l, d, q, 0.0, 1, np.zeros(50, int))
    b = rules.verify_greedy(l, d)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # and a very low temperature agrees with greedy on every unflagged round
    n, tok, fl = rules.verify_sample(l, d, q, 1e-4, 1, np.zeros(50, int))
    n0, tok0, _ = b
    ok = ~fl
    assert np.array_equal(n[ok], n0[ok]) and np.array_equal(tok[ok], tok0[ok])


def test_diag_hand_example():
    """Greedy margins by hand: slot 0 logits (0, 1, 3) -> gap 2; slot 1 (2, 2, 1) -> a tie,
    gap 0; slot 2 (5, 1, 0) -> gap 4.  Drafts (2, 1): slot 0 accepts, slot 1 rejects
    (its argmax is 0, the lower index of the tie), so slot 2 is not decided.  Drafts
    (2, 0): every slot is decided."""
    logits = np.array([[[0.0, 1.0, 3.0], [2.0, 2.0, 1.0], [5.0, 1.0, 0.0]]])
    n, tok, fl = rules.verify_greedy(logits, np.array([[2, 1]]))
    assert n.tolist() == [1] and tok.tolist() == [[2, 0, -1]]        # draft 1 != argmax 0 at slot 1
    d = rules.verify_diag(logits, np.array([[2, 1]]), None, 0.0, 0, np.zeros(1), n)
    assert d[0, :2].tolist() == [2.0, 0.0] and np.isnan(d[0, 2])
    assert fl.tolist() == [True]                                      # the tie is a flagged decision
    d = rules.verify_diag(logits, np.array([[2, 0]]), None, 0.0, 0, np.zeros(1), np.array([2]))
    assert d[0].tolist() == [2.0, 0.0, 4.0]
    assert np.isnan(rules.verify_diag(logits, np.array([[2, 0]]), None, 0.0, 0, np.zeros(1), np.array([-1]))).all()


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_diag_agrees_with_flags(T):
    """A sequence is flagged exactly when one of its defined margins is below the flag
    margin (random steps with small gaps, so both outcomes occur)."""
    rng = np.random.default_rng(5)
    B, gamma, V = 400, 3, 6
    logits = np.round(rng.standard_normal((B, gamma + 1, V)) * 3, 2)     # ties and near ties
    q = rng.dirichlet(np.ones(V), size=(B, gamma))
    draft = np.array([[rng.choice(V, p=q[b, i]) for i in range(gamma)] for b in range(B)])
    if T == 0.0:
        draft = np.where(rng.random((B, gamma)) < 0.7, np.argmax(logits[:, :gamma], -1), draft)
    n, tok, fl = rules.verify_sample(logits, draft, q, T, 11, np.arange(B) * 7)
    d = rules.verify_diag(logits, draft, q, T, 11, np.arange(B) * 7, n)
    below = np.any(np.nan_to_num(d, nan=np.inf) < rules.FLAG_MARGIN, axis=1)
    assert np.array_equal(below, fl)
    assert fl.any() and (~fl).any()
