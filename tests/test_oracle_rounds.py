"""Pins of the round policies (oracle/rounds.py): padding equals per-sequence
verification, the heuristic schedule on a hand-written run, the confidence cut on
hand-made rows, candidate selection by brute force, and multi-candidate greedy rounds
reproducing greedy autoregressive decoding on a tiny decoder."""
import copy

import numpy as np
import pytest

from oracle import decoder as dec
from oracle import rounds, rules
from tests.test_oracle_decoder import tiny_model


def test_padded_batch_equals_per_sequence_verification():
    rng = np.random.default_rng(3)
    B, G, V = 12, 5, 37
    logits = rng.standard_normal((B, G + 1, V)) * 2
    gamma_b = rng.integers(1, G + 1, B)
    l32 = rules.f32_logits(logits)
    # greedy: drafts agree with the argmax for a random prefix
    arg = np.argmax(l32, axis=-1)
    draft = np.where(rng.random((B, G)) < 0.7, arg[:, :G], (arg[:, :G] + 1) % V)
    pd, _ = rounds.pad_drafts(draft, None, gamma_b)
    n, tok, _ = rules.verify_greedy(logits, pd)
    for b in range(B):
        g = int(gamma_b[b])
        n1, t1, _ = rules.verify_greedy(logits[b:b + 1, :g + 1], draft[b:b + 1, :g])
        assert n[b] == n1[0] and tok[b, :g + 1].tolist() == t1[0].tolist() and np.all(tok[b, g + 1:] == -1)
    # sampling, q near p so that drafts are often accepted
    T, seed = 0.9, 77
    p = rules.target_probs(l32[:, :G], T).astype(np.float64)
    q = p * np.exp(0.3 * rng.standard_normal(p.shape))
    q /= q.sum(-1, keepdims=True)
    draft = np.array([[rng.choice(V, p=q[b, i]) for i in range(G)] for b in range(B)])
    pos0 = rng.integers(0, 500, B)
    pd, pq = rounds.pad_drafts(draft, q, gamma_b)
    n, tok, _ = rules.verify_sample(logits, pd, pq, T, seed, pos0)
    seen = set()
    for b in range(B):
        g = int(gamma_b[b])
        n1, t1, _ = rules.verify_sample(logits[b:b + 1, :g + 1], draft[b:b + 1, :g], q[b:b + 1, :g], T, seed,
                                        pos0[b:b + 1], seq0=b)
        assert n[b] == n1[0] and tok[b, :g + 1].tolist() == t1[0].tolist() and np.all(tok[b, g + 1:] == -1)
        seen.add((int(n[b]) == g))
    assert seen == {True, False}          # both the all-accepted bonus and a rejection occur


def test_heuristic_schedule_hand_run():
    g, seq = 4, []
    for n in [4, 6, 2, 0, 0, 0, 0, 1, -1, 1, 2]:
        g = int(rounds.heuristic_gamma([n], [g], 1, 7)[0])
        seq.append(g)
    assert seq == [6, 7, 6, 5, 4, 3, 2, 1, 1, 3, 2]
    assert rounds.heuristic_gamma([3, 0, 5], [3, 1, 5], 1, 5).tolist() == [5, 1, 5]


def test_confidence_cut():
    V = 5
    q = np.zeros((3, 4, V))
    for b, peaks in enumerate([[0.9, 0.8, 0.3, 0.9], [0.2, 0.9, 0.9, 0.9], [0.6, 0.6, 0.6, 0.6]]):
        for k, pk in enumerate(peaks):
            q[b, k, 0] = pk
            q[b, k, 1:] = (1 - pk) / (V - 1)
    assert rounds.confidence_gamma(q, [4, 4, 3], 0.5).tolist() == [2, 1, 3]
    assert rounds.confidence_gamma(q, [1, 4, 4], 0.95).tolist() == [1, 1, 1]


def test_candidate_selection_brute_force():
    rng = np.random.default_rng(9)
    n = rng.integers(-1, 5, (200, 4))
    tok = rng.integers(0, 50, (200, 4, 5))
    idx, nb, tb = rounds.select_candidates(n, tok)
    assert idx.tolist() == np.argmax(n, axis=1).tolist()      # first maximal index
    assert nb.tolist() == n.max(axis=1).tolist()
    assert np.array_equal(tb, tok[np.arange(200), idx])


@pytest.mark.parametrize("C,corrupt", [(3, 0.4), (2, 0.7)])
def test_greedy_candidates_reproduce_autoregressive_decoding(C, corrupt):
    """Each round verifies C corrupted copies of the true continuation, keeps the longest
    accepted; the emitted stream equals plain greedy decoding token for token."""
    gamma, steps = 4, 24
    wts, kv0 = tiny_model(seed=21 + C, B=1, max_len=256)
    first = np.array([5])
    ar = dec.greedy_autoregressive(wts, first, copy.deepcopy(kv0), steps + gamma + 2)[0]
    rng = np.random.default_rng(C)
    kv = copy.deepcopy(kv0)
    out, last = [], int(first[0])
    while len(out) < steps:
        pos = len(out)
        ns, toks, kvs = [], [], []
        for c in range(C):
            d = np.array(ar[pos:pos + gamma])
            d = np.where(rng.random(gamma) < corrupt, (d + 1 + c) % wts.vocab, d)
            kc = copy.deepcopy(kv)
            logits = dec.forward(wts, np.concatenate([[last], d])[None, :], kc)
            n, t, _ = rules.verify_greedy(logits, d[None, :])
            ns.append(n[0]); toks.append(t[0]); kvs.append(kc)
        idx, nb, tb = rounds.select_candidates(np.array([ns]), np.array([toks]))
        kv = kvs[int(idx[0])]
        dec.commit(kv, nb)
        emitted = tb[0, :nb[0] + 1].tolist()
        out += emitted
        last = emitted[-1]
    assert out[:steps] == ar[:steps].tolist()
