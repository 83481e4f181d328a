"""Host round policies around the verify step (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

* Variable draft length per sequence by padding ([MTP-drafters] 6, adaptive k; [Self-spec]
  3.3 on trimming each sequence to what it accepted): a batch verifies gamma_max slots, and
  sequence b drafts only gamma_b of them.  Reading: the slots gamma_b .. gamma_max - 1 are
  padded with the draft id -1 and a q row of zeros.  The plain rule then rejects at slot
  gamma_b at the latest (no id matches), and the residual there is max(0, p - 0) = p, the
  bonus distribution, drawn at the bonus's position: the padded batch gives each sequence
  exactly what verifying it alone with gamma_b drafts gives.
* Heuristic schedule ([MTP-deep-dive] 5.1, the HF assistant setting): every draft accepted
  -> the next round drafts two more, any rejection -> one fewer; kept within
  [gamma_min, gamma_max].
* Confidence cut ([MTP-drafters] 6, adaptive k): the drafter stops at the first step whose
  distribution is flat.  Reading: gamma_b becomes the number of leading steps whose
  largest q is at least tau (at least one draft is kept), then padding as above.
* Several draft candidates per sequence ([MTP-drafters] 6, multiple candidates): the target
  verifies each and the longest accepted one is kept.  Reading: under the greedy rule the
  accepted prefix of every candidate is the target's own argmax chain, so keeping the
  longest (the lower candidate index on equal lengths) is lossless; under the sampling
  rule picking the best of several independent verifications biases the output, so
  only the greedy rule is offered.

Pinned by (tests/test_oracle_rounds.py): a padded batch equals sequence-by-sequence
verification with each gamma_b (greedy and sampling, bit for bit); the schedule's
sequence on a hand-written run of outcomes; the confidence cut on hand-made q rows; the
candidate choice by brute force, and the greedy multi-candidate result equals the
argmax continuation.
"""
import numpy as np


def pad_drafts(draft, q, gamma_b):
    """Padded copies: draft[b, i] = -1 and q[b, i] = 0 for i >= gamma_b[b].  ``q`` may
    be None (greedy)."""
    draft = np.array(draft, dtype=np.int64, copy=True)
    gamma_b = np.asarray(gamma_b, dtype=np.int64)
    B, G = draft.shape
    mask = np.arange(G)[None, :] >= gamma_b[:, None]
    draft[mask] = -1
    if q is None:
        return draft, None
    q = np.array(q, copy=True)
    q[mask] = 0
    return draft, q


def confidence_gamma(q, gamma_b, tau):
    """gamma_b cut to the leading steps whose largest q is >= tau, at least 1.
    ``q`` [B, G, V]."""
    q = np.asarray(q, dtype=np.float64)
    gamma_b = np.asarray(gamma_b, dtype=np.int64)
    B, G, _ = q.shape
    out = np.empty(B, dtype=np.int64)
    for b in range(B):
        k = 0
        while k < gamma_b[b] and q[b, k].max() >= tau:
            k += 1
        out[b] = max(1, k)
    return out


def heuristic_gamma(n, gamma_b, gamma_min, gamma_max):
    """Next round's draft length: +2 if every draft was accepted (n == gamma_b), else -1,
    within [gamma_min, gamma_max].  An invalid round (n < 0) keeps gamma_b."""
    n = np.asarray(n, dtype=np.int64)
    g = np.asarray(gamma_b, dtype=np.int64)
    nxt = np.where(n >= g, g + 2, g - 1)
    nxt = np.clip(nxt, gamma_min, gamma_max)
    return np.where(n < 0, g, nxt)


def select_candidates(n, tokens):
    """Among C candidates per sequence (``n`` [B, C], ``tokens`` [B, C, G1]) the one
    with the largest n, the lower index on ties; an invalid candidate (n < 0) never wins
    unless all are.  Returns (index [B], n [B], tokens [B, G1])."""
    n = np.asarray(n, dtype=np.int64)
    tokens = np.asarray(tokens, dtype=np.int64)
    B, C = n.shape
    idx = np.empty(B, dtype=np.int64)
    for b in range(B):
        best = 0
        for c in range(1, C):
            if n[b, c] > n[b, best]:
                best = c
        idx[b] = best
    return idx, n[np.arange(B), idx], tokens[np.arange(B), idx]
