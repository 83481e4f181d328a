"""Pins of the oracle's centroid-masked drafter LM head (CPU only).

[X-thread] "Gemma 4's MTP", efficient embedder; [MTP-deep-dive] 3.4.  The selection is pinned by a
hand-checked fixture with ties and by the top-k set property; the cluster scores by
linearity against the plain LM head; the token logits by the all-clusters case (a
reordering of the full LM head) and a brute-force loop.
"""
import json
import os

import numpy as np

from oracle import masked_head as mh
from oracle import rules

HERE = os.path.dirname(os.path.abspath(__file__))


def test_selection_fixture():
    g = json.load(open(os.path.join(HERE, "golden", "masked_head_selection.json")))
    cl = np.array(g["cluster_logits"], dtype=np.float64)
    for case in g["cases"]:
        sel, _ = mh.select_clusters(cl, case["top_k"])
        assert sel.tolist() == case["clusters"]


def test_selection_set_property_and_order():
    rng = np.random.default_rng(5)
    for trial in range(50):
        C = int(rng.integers(2, 40))
        k = int(rng.integers(1, C + 1))
        # coarse values so that ties occur
        cl = rng.integers(-4, 5, size=(3, C)).astype(np.float64) * 0.5
        sel, _ = mh.select_clusters(cl, k)
        for m in range(3):
            kept = cl[m, sel[m]]
            rest = np.delete(cl[m], sel[m])
            assert len(set(sel[m].tolist())) == k
            if rest.size:
                assert kept.min() >= rest.max()
            # descending, lower id first on equal values
            for a, b in zip(sel[m][:-1], sel[m][1:]):
                assert cl[m, a] > cl[m, b] or (cl[m, a] == cl[m, b] and a < b)
            # a tie straddling the cut keeps the lower ids
            if rest.size and kept.min() == rest.max():
                v = kept.min()
                tied_out = [c for c in range(C) if cl[m, c] == v and c not in sel[m]]
                tied_in = [c for c in sel[m] if cl[m, c] == v]
                assert max(tied_in) < min(tied_out)


def test_cluster_scores_are_member_means():
    """Linearity: scoring a cluster with the mean of its members' embeddings gives the
    mean of the members' token logits."""
    rng = np.random.default_rng(6)
    V, d, C = 96, 16, 12
    w = rng.standard_normal((V, d))
    h = rng.standard_normal((4, d))
    cs = mh.cluster_size(V, C)
    cent = w.reshape(C, cs, d).mean(axis=1)
    full = rules.lm_head_logits(h, w)
    np.testing.assert_allclose(mh.cluster_logits(h, cent), full.reshape(4, C, cs).mean(axis=2), rtol=0, atol=1e-12)


def test_all_clusters_kept_is_the_full_head():
    rng = np.random.default_rng(7)
    V, d, C = 128, 32, 16
    w = rng.standard_normal((V, d))
    cent = rng.standard_normal((C, d))
    h = rng.standard_normal((3, d))
    sel, logits, _ = mh.masked_head(h, w, cent, C)
    cs = V // C
    full = rules.lm_head_logits(h, w)
    for m in range(3):
        tok = (sel[m][:, None] * cs + np.arange(cs)[None, :]).reshape(-1)
        assert sorted(tok.tolist()) == list(range(V))
        np.testing.assert_allclose(logits[m], full[m, tok], rtol=0, atol=1e-12)   # summation order only


def test_token_logits_brute_force():
    rng = np.random.default_rng(8)
    V, d, C, k = 24, 5, 6, 2
    w = rng.integers(-3, 4, size=(V, d)).astype(np.float64)
    h = rng.integers(-3, 4, size=(2, d)).astype(np.float64)
    sel = np.array([[4, 1], [0, 5]])
    out = mh.masked_logits(h, w, sel, V // C)
    for m in range(2):
        for j in range(k):
            for t in range(V // C):
                tok = sel[m, j] * (V // C) + t
                acc = 0.0
                for i in range(d):
                    acc += h[m, i] * w[tok, i]
                assert out[m, j * (V // C) + t] == acc


def test_flags_mark_near_ties_at_the_cut():
    cl = np.array([[1.0, 0.9995, 0.5], [1.0, 0.9, 0.5]])
    _, flags = mh.select_clusters(cl, 1)
    assert flags.tolist() == [True, False]
