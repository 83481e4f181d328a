"""The verify step's arithmetic and acceptance rules (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Notation.  A batch has B sequences.  Each carries gamma drafted tokens
x_1..x_gamma; with the last accepted token in front, the target model sees
gamma+1 positions ("slots") 0..gamma.  Slot i's output distribution is the
target's prediction for the token after input i, so slot i judges draft
x_{i+1} (stored at ``draft[:, i]``), and slot gamma yields the bonus token.
[Infra-ch8] "why one forward pass can verify several tokens" (causal mask:
L inputs give L next-token predictions) and "where the extra token comes from"
(N drafts give N+1 prediction positions).

Precision.  Logit values are computed exactly in float64 from the bf16/f32
inputs, then rounded to float32, the precision the GPU stores logits in.  Every
integer decision (argmax, accept/reject, Gumbel argmax) is taken on float32
quantities, as the kernel takes it:

* greedy argmax over the float32 logits (lowest index on ties);
* acceptance: u * q(x) < p(x) with p(x) the correctly rounded float32 target
  probability, evaluated exactly (u has 24 bits and q at most 24, so the
  product is exact in float64);
* resampling: float32 scores log(r_v) + G_v.

Decisions whose margin is below 1e-3 are *flagged*; the GPU may legitimately
differ there because its float32 values carry accumulation rounding.
"""
import numpy as np

from . import philox

FLAG_MARGIN = 1e-3


def lm_head_logits(h, w):
    """logits = h . w^T in float64.

    ``h``: [..., d] hidden states, ``w``: [V, d] LM-head table, both float64
    holding exact bf16/f32 values (bf16 products are exact in float64).
    [Infra-ch8] "why one forward pass can verify several tokens": the target
    returns a next-token distribution at every one of the L input positions;
    [MTP-deep-dive] section 3.4 for the LM head as hidden state times the
    (tied) embedding table.

    Pinned by: a one-hot hidden state selects a column of w exactly; small
    integer-valued inputs equal a brute-force triple loop.
    """
    return np.matmul(np.asarray(h, dtype=np.float64), np.asarray(w, dtype=np.float64).T)


def f32_logits(logits64):
    """Round float64 logits to float32, the storage precision of the kernel."""
    return np.asarray(logits64, dtype=np.float64).astype(np.float32)


def top2(l32):
    """(argmax, top-2 gap) along the last axis; argmax is the lowest index."""
    a = np.argmax(l32, axis=-1)
    part = np.partition(l32.astype(np.float64), -2, axis=-1)
    gap = part[..., -1] - part[..., -2]
    return a, gap


def target_probs(l32, temperature):
    """p = softmax(l / T) over the vocabulary, returned as float32.

    Computed in float64 from the float32 logits (max-subtracted), then rounded
    once to float32.  [Infra-ch8] "why the output does not change" and
    [MTP-drafters] section 5.2 problem 2: sampling parameters (temperature)
    must be the same for draft and verify, so p uses the caller's T.

    Pinned by: scipy.special.softmax on the same inputs.
    """
    l = np.asarray(l32, dtype=np.float32).astype(np.float64)
    t = float(temperature)
    if not (t > 0.0 and np.isfinite(t)):
        raise ValueError("target_probs: temperature must be finite and > 0")
    m = l.max(axis=-1, keepdims=True)
    e = np.exp((l - m) / t)
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def greedy_rule(l32, draft):
    """Greedy acceptance with truncation and the N+1 bonus token.

    Accept draft x_{i+1} while it equals the argmax of slot i; at the first
    mismatch stop and emit the slot's argmax in its place; if all gamma drafts
    match, emit slot gamma's argmax as the bonus.
    [MTP-drafters] section 3.2 (compare each draft with the target's greedy
    prediction, reject from the first disagreement, substitute the target's
    token), [Self-spec] section 3.1 (compare with the *mode*, not a probability
    threshold), [Infra-ch8] "a concrete example" and "where the extra token
    comes from" (all four accepted gives five tokens).

    ``l32``: [B, gamma+1, V] float32; ``draft``: [B, gamma] int.
    Returns (n_accepted [B], tokens [B, gamma+1] with -1 past n, flagged [B]).
    A draft id outside [0, V) never equals an argmax, so it is rejected.

    Pinned by: brute force over every argmax/draft tuple on a tiny vocabulary;
    the worked example of [Infra-ch8]; greedy speculative output equal to
    plain greedy autoregressive output on a tiny random decoder.
    """
    l32 = np.asarray(l32, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.int64)
    B, G1, V = l32.shape
    gamma = G1 - 1
    assert draft.shape == (B, gamma)
    am, gap = top2(l32)
    n = np.full(B, gamma, dtype=np.int64)
    live = np.ones(B, dtype=bool)
    for i in range(gamma):
        mism = live & (draft[:, i] != am[:, i])
        n[mism] = i
        live &= ~mism
    tokens = assemble_tokens(draft, n, am[np.arange(B), n])
    reached = np.arange(G1)[None, :] <= n[:, None]
    flagged = np.any(reached & (gap < FLAG_MARGIN), axis=1)
    return n, tokens, flagged


def sample_rule(l32, draft, q, temperature, seed, pos0, seq0=0):
    """Speculative sampling: accept with probability min(1, p/q), resample the
    first rejected slot from max(0, p - q)/Z, bonus from p_gamma.

    [MTP-deep-dive] section 2.2 (acceptance probability min(1, p(x)/q(x)) and
    the corrected distribution max(0, p - q)/Z), [Infra-ch8] "why the output
    does not change" (q <= p accept outright, otherwise reject with probability
    1 - p/q, resample from the clipped and renormalised p - q), [Self-spec]
    section 3.2 (same rule), section 3.3 (independent randomness per position),
    [Infra-ch8] "where the extra token comes from" (the bonus).

    Readings where the pages leave a step open:

    * u is a 24-bit uniform in [0, 1) from the Philox stream at the position
      of the token being decided (``pos0 + i + 1``); accept iff
      u * q(x) < p(x).  So p >= q always accepts, q(x) = 0 < p(x) accepts and
      p(x) = q(x) = 0 rejects.  q is used exactly as given (not renormalised).
    * Out-of-range draft ids are rejected (treated as p(x) = q(x) = 0).
    * The residual is r = max(0, p - q) evaluated in float32; if it is zero
      everywhere (only possible when q >= p everywhere) the slot samples p.
    * Sampling from r/Z is Gumbel-max: y = argmax_v log r_v + G_v over r_v > 0,
      G_v = -log(-log U_v) with U_v the per-vocab Philox uniforms; exact in law
      and independent of summation order.

    ``l32``: [B, gamma+1, V] float32 logits; ``draft``: [B, gamma] int;
    ``q``: [B, gamma, V] draft probabilities (float64 holding exact bf16/f32
    values); ``pos0``: [B] absolute position of slot 0.  Sequence ids are
    ``seq0 + b`` (``seq0`` lets a caller process one large batch in chunks).

    Returns (n_accepted [B], tokens [B, gamma+1], flagged [B]).

    Pinned by: exact-rational enumeration of the output law on V <= 8,
    gamma <= 2 (equals p position by position); the closed form
    E = (1 - a^(g+1))/(1 - a) and the law of the emitted count; a chi-square
    test of emitted tokens against p; q = p accepts everything; disjoint
    supports reject at slot 0.
    """
    l32 = np.asarray(l32, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    B, G1, V = l32.shape
    gamma = G1 - 1
    assert draft.shape == (B, gamma) and q.shape == (B, gamma, V)
    pos0 = np.broadcast_to(np.asarray(pos0, dtype=np.int64), (B,))
    seq = seq0 + np.arange(B, dtype=np.int64)
    p32 = target_probs(l32, temperature)
    u = np.stack([philox.accept_uniform(seed, seq, pos0 + i + 1) for i in range(gamma)], axis=1) \
        if gamma else np.zeros((B, 0))
    n, flagged = accept_slots(p32, q, draft, u)
    y, gflag = resample(p32, q, n, seed, pos0, seq0)
    flagged |= gflag
    tokens = assemble_tokens(draft, n, y)
    return n, tokens, flagged


def accepts(u, qx, px):
    """The acceptance test of one draft: u * q(x) < p(x), exact in float64.

    Equivalent to u < min(1, p/q) for q > 0 without a division; u is uniform
    on the 24-bit grid of [0, 1).  ([MTP-deep-dive] section 2.2; [Infra-ch8]
    "why the output does not change".)
    """
    return np.asarray(u, dtype=np.float64) * np.asarray(qx, dtype=np.float64) < np.asarray(px, dtype=np.float64)


def accept_slots(p32, q, draft, u):
    """Acceptance decisions over slots 0..gamma-1 and the first rejection.

    ``p32``: [B, gamma+1, V] float32 target probabilities; ``q``: [B, gamma, V];
    ``draft``: [B, gamma]; ``u``: [B, gamma] acceptance uniforms.
    Returns (n [B] = index of the first rejected slot, gamma if none;
    flagged [B] = a decided slot had |u - p(x)/q(x)| < 1e-3).
    Slots after the first rejection are not decided (their drafts were built
    on a rejected prefix; [Self-spec] section 3.3).
    """
    draft = np.asarray(draft, dtype=np.int64)
    B, gamma = draft.shape
    V = p32.shape[-1]
    n = np.full(B, gamma, dtype=np.int64)
    live = np.ones(B, dtype=bool)
    flagged = np.zeros(B, dtype=bool)
    bi = np.arange(B)
    for i in range(gamma):
        x = draft[:, i]
        inr = (x >= 0) & (x < V)
        xc = np.where(inr, x, 0)
        px = np.where(inr, p32[bi, i, xc].astype(np.float64), 0.0)
        qx = np.where(inr, np.asarray(q, dtype=np.float64)[bi, i, xc], 0.0)
        ok = accepts(u[:, i], qx, px)
        with np.errstate(divide="ignore", invalid="ignore"):
            margin = np.where(qx > 0, np.abs(u[:, i] - px / np.where(qx > 0, qx, 1.0)), np.inf)
        flagged |= live & (margin < FLAG_MARGIN)
        n[live & ~ok] = i
        live &= ok
    return n, flagged


def residual_rows(p_rows32, q_rows):
    """r = max(0, p - q) in float32, row-wise; a row that is zero everywhere
    falls back to p.

    [MTP-deep-dive] section 2.2: p'(x) = max(0, p(x) - q(x)) / Z; the
    normalisation Z is left implicit because the sampler only needs r up to a
    constant factor.
    """
    p = np.asarray(p_rows32, dtype=np.float32)
    r = np.maximum(p - np.asarray(q_rows, dtype=np.float32), np.float32(0.0))
    empty = ~np.any(r > 0, axis=-1)
    r[empty] = p[empty]
    return r


def gumbel_scores(r32, seed, seq, pos, tag=philox.TAG_GUMBEL):
    """float32 scores log r_v + G_v (-inf where r_v = 0), one row per sequence.

    ``r32``: [B, V]; ``seq``, ``pos``: [B].  G_v = -log(-log U_v) with U_v the
    Philox uniform of (seed, seq, pos, v) in stream ``tag``.
    """
    B, V = r32.shape
    U = philox.gumbel_uniform_rows(seed, seq, pos, V, tag).astype(np.float32)
    G = -np.log(-np.log(U))
    with np.errstate(divide="ignore"):
        s = np.where(r32 > 0, np.log(r32) + G, np.float32(-np.inf)).astype(np.float32)
    return s


def resample_rows(p32, q, n):
    """The distribution (up to a factor) each sequence's last token is drawn from.

    Row n_b only: the residual max(0, p - q) of the first rejected slot when
    n_b < gamma, or p_gamma (the bonus, N+1-th token) when every draft was
    accepted.  Returns float32 [B, V].
    """
    B, G1, V = p32.shape
    gamma = G1 - 1
    bi = np.arange(B)
    n = np.asarray(n, dtype=np.int64)
    r = np.array(p32[bi, n], dtype=np.float32)
    rej = n < gamma
    if np.any(rej):
        r[rej] = residual_rows(r[rej], np.asarray(q)[bi[rej], n[rej]])
    return r


def resample(p32, q, n, seed, pos0, seq0=0):
    """Correction or bonus token of every sequence (step a7): Gumbel-max over
    :func:`resample_rows` with the Philox noise at position pos0 + n + 1.

    Returns (tokens [B], flagged [B]) where a flag marks a top-2 Gumbel score
    gap below 1e-3.
    """
    B, G1, V = p32.shape
    bi = np.arange(B)
    r = resample_rows(p32, q, n)
    s = gumbel_scores(r, seed, seq0 + bi, np.asarray(pos0, dtype=np.int64) + np.asarray(n) + 1)
    y = np.argmax(s, axis=-1)
    if V >= 2:
        t2 = np.partition(s.astype(np.float64), -2, axis=-1)
        with np.errstate(invalid="ignore"):
            gap = t2[:, -1] - t2[:, -2]
        flag = gap < FLAG_MARGIN
    else:
        flag = np.zeros(B, dtype=bool)
    return y.astype(np.int64), flag


def assemble_tokens(draft, n, last):
    """tokens[b] = draft[b, :n_b] + [last_b], padded with -1 (step a8)."""
    B, gamma = draft.shape
    j = np.arange(gamma + 1)[None, :]
    d = np.concatenate([draft, np.zeros((B, 1), dtype=np.int64)], axis=1)
    tok = np.where(j < n[:, None], d, -1)
    tok[np.arange(B), n] = last
    return tok


def verify_greedy(logits64, draft):
    """Greedy verify step from exact logits: (n, tokens, flagged)."""
    return greedy_rule(f32_logits(logits64), draft)


def verify_sample(logits64, draft, q, temperature, seed, pos0, seq0=0):
    """Sampling verify step from exact logits; T == 0 is exactly the greedy rule
    (the limit of the sampling rule as T -> 0, [Infra-ch8] "how the benefit is
    computed": lower temperature, sharper distribution)."""
    if float(temperature) == 0.0:
        return verify_greedy(logits64, draft)
    return sample_rule(f32_logits(logits64), draft, q, temperature, seed, pos0, seq0)


def verify_diag(logits64, draft, q, temperature, seed, pos0, n, seq0=0):
    """How close each decision of a verify step came to going the other way: float64
    [B, gamma+1], NaN where a slot was not decided ([Self-spec] 3.1: the greedy rule
    compares the draft with the target's mode; 3.2: the sampling rule accepts with
    probability min(1, p/q) and draws the correction from max(0, p - q)).

    * T = 0: entry i <= n_b is the gap between the largest and second-largest float32
      logit of slot i (0 when two tokens share the maximum).
    * T > 0: entry i <= min(n_b, gamma - 1) is |u_i - p_i(x) / q_i(x)| (infinity when
      q_i(x) = 0; out-of-range drafts have q = 0); entry gamma is the gap between the two
      best scores log r_v + G_v of the final draw (:func:`resample`), infinity if only
      one entry can win.
    * Rows with n_b < 0 (invalid) are NaN.

    These are the quantities the flags of :func:`greedy_rule`, :func:`accept_slots` and
    :func:`resample` compare with FLAG_MARGIN.  ``n``: the step's accepted counts.

    Pinned by: a hand-computed greedy example; a sequence is flagged exactly when one of
    its defined entries is below FLAG_MARGIN (random greedy and sampling steps).
    """
    l32 = f32_logits(logits64)
    B, G1, V = l32.shape
    gamma = G1 - 1
    n = np.asarray(n, dtype=np.int64)
    out = np.full((B, G1), np.nan)
    valid = n >= 0
    if float(temperature) == 0.0:
        _, gap = top2(l32)
        reached = np.arange(G1)[None, :] <= n[:, None]
        out = np.where(reached & valid[:, None], gap.astype(np.float64), np.nan)
        return out
    draft = np.asarray(draft, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    pos0 = np.broadcast_to(np.asarray(pos0, dtype=np.int64), (B,))
    seq = seq0 + np.arange(B, dtype=np.int64)
    p32 = target_probs(l32, temperature)
    bi = np.arange(B)
    for i in range(gamma):
        u = philox.accept_uniform(seed, seq, pos0 + i + 1)
        x = draft[:, i]
        inr = (x >= 0) & (x < V)
        xc = np.where(inr, x, 0)
        px = np.where(inr, p32[bi, i, xc].astype(np.float64), 0.0)
        qx = np.where(inr, q[bi, i, xc], 0.0)
        with np.errstate(divide="ignore", invalid="ignore"):
            margin = np.where(qx > 0, np.abs(u - px / np.where(qx > 0, qx, 1.0)), np.inf)
        out[:, i] = np.where((i <= n) & valid, margin, np.nan)
    nn = np.where(valid, n, gamma)
    r = resample_rows(p32, q, nn)
    sc = gumbel_scores(r, seed, seq, pos0 + nn + 1).astype(np.float64)
    t2 = np.sort(sc, axis=-1)
    with np.errstate(invalid="ignore"):
        gap = np.where(np.isfinite(t2[:, -2]), t2[:, -1] - t2[:, -2], np.inf) if V >= 2 else np.full(B, np.inf)
    out[:, gamma] = np.where(valid, gap, np.nan)
    return out


def filtered_probs(l32, temperature, top_k, top_p):
    """Target probabilities after the top-k and top-p filters, float32, zero outside the
    kept tokens, together with the kept masks and boundary flags.

    [Infra-ch8] "why the output does not change" and [MTP-drafters] 5.2 (problem 2):
    temperature, top-k and top-p must be handled by one rule in drafting and verifying,
    or the distribution drifts; the deployment example runs temperature 1.0, top_p 0.95,
    top_k 64 ([MTP-deep-dive] 5.1); top-k samples among the k most probable tokens and
    top-p among the smallest set whose cumulative probability exceeds p ([MTP-drafters]
    3.1, draft-token strategies).

    Readings: the filters apply in the order temperature, top-k, top-p; the k kept
    tokens are the k largest float32 logits, the lower index first on equal values
    (exactly k are kept); top-p walks the kept tokens in that order with their
    probabilities renormalised over the top-k set and keeps every token whose
    predecessors' cumulative probability is still below top_p (the smallest prefix whose
    sum reaches top_p); the result is renormalised over the kept tokens, computed in
    float64 from the float32 logits and rounded once to float32.

    ``l32``: [..., V]; returns (p float32 [..., V], kept bool [..., V], flags [...]);
    a flag marks a row whose top-k cut falls between logits closer than 1e-3, or whose
    top-p cut has a cumulative probability within 1e-3 of top_p on either side.

    Pinned by: a hand-checked fixture with a tie at the top-k cut; top_k = V and
    top_p = 1 give target_probs exactly; kept sets are prefixes of the descending
    order with the stated top-p property.
    """
    l = np.asarray(l32, dtype=np.float32)
    t = float(temperature)
    if not (t > 0.0 and np.isfinite(t)):
        raise ValueError("filtered_probs: temperature must be finite and > 0")
    if not 1 <= int(top_k):
        raise ValueError("filtered_probs: top_k must be >= 1")
    if not 0.0 < float(top_p) <= 1.0:
        raise ValueError("filtered_probs: top_p must be in (0, 1]")
    shape = l.shape
    V = shape[-1]
    rows = l.reshape(-1, V)
    out = np.zeros(rows.shape, dtype=np.float32)
    kept = np.zeros(rows.shape, dtype=bool)
    flags = np.zeros(rows.shape[0], dtype=bool)
    k = min(int(top_k), V)
    for r in range(rows.shape[0]):
        x = rows[r].astype(np.float64)
        order = np.lexsort((np.arange(V), -x))          # descending logit, lower index first
        top = order[:k]
        if k < V and x[order[k - 1]] - x[order[k]] < FLAG_MARGIN:
            flags[r] = True
        e = np.exp((x[top] - x[top[0]]) / t)
        pk = e / e.sum()
        keep = 0
        cum = 0.0
        for j in range(k):
            if cum >= float(top_p):
                break
            keep += 1
            cum += pk[j]
        if keep < k:
            before = cum - pk[keep - 1]
            if abs(cum - float(top_p)) < FLAG_MARGIN or abs(before - float(top_p)) < FLAG_MARGIN:
                flags[r] = True
        sel = top[:keep]
        out[r, sel] = (pk[:keep] / pk[:keep].sum()).astype(np.float32)
        kept[r, sel] = True
    return out.reshape(shape), kept.reshape(shape), flags.reshape(shape[:-1])


def sample_rule_filtered(l32, draft, q, temperature, top_k, top_p, seed, pos0, seq0=0):
    """The sampling rule of :func:`sample_rule` on the filtered target distribution of
    :func:`filtered_probs` (the same top-k / top-p the drafter applied to q): accept with
    probability min(1, p~/q), resample the first rejected slot from max(0, p~ - q), the
    bonus from p~_gamma.  The output law is p~ ([Infra-ch8] "why the output does not
    change": the rule preserves whatever target distribution it is given).  q is used as
    given.  Returns (n_accepted [B], tokens [B, gamma+1], flagged [B]).

    Pinned by: top_k = V, top_p = 1 reproduces sample_rule bit for bit; the rule's law
    is pinned through accept_slots / resample_rows (exact enumeration)."""
    l32 = np.asarray(l32, dtype=np.float32)
    draft = np.asarray(draft, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    B, G1, V = l32.shape
    gamma = G1 - 1
    pos0 = np.broadcast_to(np.asarray(pos0, dtype=np.int64), (B,))
    seq = seq0 + np.arange(B, dtype=np.int64)
    p32, _, fflags = filtered_probs(l32, temperature, top_k, top_p)
    u = np.stack([philox.accept_uniform(seed, seq, pos0 + i + 1) for i in range(gamma)], axis=1) \
        if gamma else np.zeros((B, 0))
    n, flagged = accept_slots(p32, q, draft, u)
    y, gflag = resample(p32, q, n, seed, pos0, seq0)
    reached = np.arange(G1)[None, :] <= n[:, None]
    flagged |= gflag | np.any(reached & fflags, axis=1)
    return n, assemble_tokens(draft, n, y), flagged


def verify_sample_filtered(logits64, draft, q, temperature, top_k, top_p, seed, pos0, seq0=0):
    """Aligned-filter sampling verify from exact logits; T == 0 is the greedy rule (the
    filters always keep the argmax)."""
    if float(temperature) == 0.0:
        return verify_greedy(logits64, draft)
    return sample_rule_filtered(f32_logits(logits64), draft, q, temperature, top_k, top_p, seed, pos0, seq0)


def acceptance_rate(p, q):
    """alpha = sum_v min(p_v, q_v): the probability that a draft x ~ q is
    accepted ([Infra-ch8] "how the benefit is computed"; [Self-spec] 4.1)."""
    return np.minimum(np.asarray(p, dtype=np.float64), np.asarray(q, dtype=np.float64)).sum(axis=-1)
