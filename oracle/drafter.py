"""The MTP drafter's draft step (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What the drafter computes ([X-thread] "Gemma 4's MTP": target activations, KV cache
sharing, efficient embedder; [MTP-deep-dive] 3.1-3.4): a small decoder attached to the
target.  At every step its input is the embedding of the current token (the target's
own table, D wide) joined with a D-wide hidden state, projected down to the drafter's
width H.  Four decoder layers follow whose attention has query projections only: keys
and values come from the target's KV cache, and the drafter keeps no cache of its own.
A final RMSNorm and a projection back up to D give the new hidden state, which the LM
head tied to the token table (or the centroid-masked head) turns into logits.  The
first step's hidden state is the target's last hidden state; each later step takes the
drafter's own up-projected state of the step before and the token it just drafted.

Readings (the pages give the structure, not these details):

* the joined input is [embedding, hidden] in that order;
* drafter layer l reads the cache of one target layer chosen by the caller, laid out
  [B, n_heads, max_len, head_dim] with one key/value head per query head; every cached
  position [0, len) is visible (no sliding window); the cache is never written;
* the query of step k sits at position len + k (the token being processed), rotated
  with RoPE (rotate-half, the target's theta);
* bf16 rounding as in the target decoder (RMSNorm outputs, attention output, SiLU * up,
  final-norm output), plus the up-projected hidden state, which is stored in bf16 (it
  feeds the LM head and the next step);
* q_k = softmax(l / T) over the scored tokens (every token with the tied head, the kept
  clusters' members with the masked head; 0 elsewhere), in float64 from float32 logits,
  rounded once to float32;
* the draft is argmax over scored v of float32 log q_v + G_v, G_v = -log(-log U_v) with
  U_v from Philox stream tag 2 at the drafted token's absolute position len + k + 1
  (sequence = batch index), the lower id first on ties; T = 0 drafts the argmax of the
  float32 logits (lower id first);
* a sequence whose len is outside [1, max_len] or whose first token is no token gets
  drafts -1 and q = 0.

Pinned by (tests/test_oracle_drafter.py): gamma steps equal gamma single steps chained
by hand (the token and the hidden state fed back); the input order (with the hidden half
of the down-projection zeroed the drafts ignore the target state, with the embedding half
zeroed they ignore the token); the attention reads exactly the cached positions [0, len)
(changes at or beyond len do nothing, a one-entry cache ignores its key); the masked head
with every cluster kept equals the tied head; the drafted tokens follow q (chi-square) and
T -> 0 gives the argmax.  End-to-end values of a random drafter are "parity unpinned"
beyond these properties.
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from . import masked_head as mh
from . import philox
from . import rules
from .bf16 import bf16_to_f64, f64_to_bf16, round_bf16
from .decoder import attention, rmsnorm, rope, silu

DRAFTER_LAYER_KEYS = ("attn_norm", "wq", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
FLAG = 1e-3


@dataclass
class DrafterWeights:
    """bf16 weights (uint16 bit patterns), row-major [out, in] matrices."""
    d_model: int                      # D, the target's hidden size (token table width)
    hidden: int                       # H, the drafter's width
    n_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    rms_eps: float
    rope_theta: float
    embed: np.ndarray                 # [vocab, D], shared with the target; the tied LM head
    pre_proj: np.ndarray              # [H, 2D]
    layers: List[dict] = field(default_factory=list)   # DRAFTER_LAYER_KEYS -> array
    final_norm: np.ndarray = None     # [H]
    post_proj: np.ndarray = None      # [D, H]
    centroids: Optional[np.ndarray] = None   # [C, D]: the centroid-masked head if given
    top_k_clusters: int = 0


@dataclass
class SharedKV:
    """The target cache layers the drafter layers read: k[l], v[l] bf16 [B, n_heads,
    max_len, head_dim], and the cached lengths [B]."""
    k: List[np.ndarray]
    v: List[np.ndarray]
    length: np.ndarray


def _w(a):
    return bf16_to_f64(a)


def valid_rows(kv: SharedKV, tokens, vocab):
    lens = np.asarray(kv.length, dtype=np.int64)
    max_len = kv.k[0].shape[2]
    t = np.asarray(tokens, dtype=np.int64)
    return (lens >= 1) & (lens <= max_len) & (t >= 0) & (t < vocab)


def step_hidden(wts: DrafterWeights, kv: SharedKV, tokens, g_bits, k):
    """One drafter pass: the new hidden state (bf16 bits [B, D]) from the current
    tokens [B] and hidden states g_bits [B, D] at step k (query position len + k).
    Rows that are not valid (see :func:`valid_rows`) come back as zeros."""
    tokens = np.asarray(tokens, dtype=np.int64)
    B = tokens.shape[0]
    nh, hd = wts.n_heads, wts.head_dim
    lens = np.asarray(kv.length, dtype=np.int64)
    ok = valid_rows(kv, tokens, wts.vocab)
    e = np.zeros((B, wts.d_model))
    e[ok] = _w(wts.embed[tokens[ok]])
    z = np.concatenate([e, _w(g_bits)], axis=1)                       # exact bf16 values
    x = z @ _w(wts.pre_proj).T                                         # [B, H]
    pos = lens + k
    for li, L in enumerate(wts.layers):
        h = round_bf16(rmsnorm(x, _w(L["attn_norm"]), wts.rms_eps))
        q = rope((h @ _w(L["wq"]).T).reshape(B, nh, hd), pos, wts.rope_theta)
        o = np.zeros((B, nh, hd))
        for b in range(B):
            if not ok[b]:
                continue
            n = int(lens[b])
            kk = _w(kv.k[li][b, :, :n, :])
            vv = _w(kv.v[li][b, :, :n, :])
            for hh in range(nh):
                o[b, hh] = attention(q[b, hh][None, :], kk[hh], vv[hh])[0]
        a = round_bf16(o.reshape(B, nh * hd))
        x = x + a @ _w(L["wo"]).T
        h2 = round_bf16(rmsnorm(x, _w(L["ffn_norm"]), wts.rms_eps))
        f = round_bf16(silu(h2 @ _w(L["w_gate"]).T) * (h2 @ _w(L["w_up"]).T))
        x = x + f @ _w(L["w_down"]).T
    hf = round_bf16(rmsnorm(x, _w(wts.final_norm), wts.rms_eps))
    g = f64_to_bf16(hf @ _w(wts.post_proj).T)
    g[~ok] = 0
    return g


def scored_logits(wts: DrafterWeights, g_bits, chunk=16384, margin=FLAG):
    """The head over the new hidden states: (vocabulary ids [B, n], float64 logits
    [B, n], selection flags [B]).  Tied head: every token, logits g . embed^T.  Masked
    head: the members of the top_k_clusters clusters (oracle.masked_head); a row is
    flagged when its k-th and (k+1)-th float32 cluster scores are closer than
    ``margin``."""
    g = _w(g_bits)
    B = g.shape[0]
    V = wts.vocab
    if wts.centroids is None:
        out = np.empty((B, V))
        for v0 in range(0, V, chunk):
            out[:, v0:v0 + chunk] = g @ _w(wts.embed[v0:v0 + chunk]).T
        return np.broadcast_to(np.arange(V), (B, V)).copy(), out, np.zeros(B, dtype=bool)
    C = wts.centroids.shape[0]
    cs = mh.cluster_size(V, C)
    cl = mh.cluster_logits(g, _w(wts.centroids))
    sel, _ = mh.select_clusters(cl, wts.top_k_clusters)
    k = wts.top_k_clusters
    flags = np.zeros(B, dtype=bool)
    if k < C:
        c32 = np.sort(cl.astype(np.float32).astype(np.float64), axis=1)
        flags = c32[:, C - k] - c32[:, C - k - 1] < margin
    ids = (sel[:, :, None] * cs + np.arange(cs)[None, None, :]).reshape(B, k * cs)
    out = np.empty((B, k * cs))
    for b in range(B):
        out[b] = mh.masked_logits(g[b:b + 1], _w(wts.embed[ids[b]]), np.arange(k)[None, :], cs)[0]
    return ids, out, flags


def sample_step(ids, l64, V, temperature, seed, pos, ok, margin=FLAG):
    """Drafts and dense q for one step.  ``ids`` [B, n] scored vocabulary ids,
    ``l64`` their logits, ``pos`` [B] the drafted tokens' absolute positions.
    Returns (draft int64 [B], q float32 [B, V] or None, flags [B]): a row is flagged
    when its two best logits (T = 0) or scores (T > 0) are closer than ``margin``."""
    B = ids.shape[0]
    l32 = np.asarray(l64, dtype=np.float64).astype(np.float32)
    draft = np.full(B, -1, dtype=np.int64)
    flags = np.zeros(B, dtype=bool)
    if float(temperature) == 0.0:
        for b in range(B):
            if not ok[b]:
                continue
            dense = np.full(V, -np.inf, dtype=np.float32)
            dense[ids[b]] = l32[b]
            draft[b] = int(np.argmax(dense))
            _, gap = rules.top2(l32[b])
            flags[b] = l32.shape[1] > 1 and gap < margin
        return draft, None, flags
    q = np.zeros((B, V), dtype=np.float32)
    for b in range(B):
        if ok[b]:
            q[b, ids[b]] = rules.target_probs(l32[b], temperature)
    sc = rules.gumbel_scores(q, seed, np.arange(B), pos, tag=philox.TAG_DRAFT)
    for b in range(B):
        if not ok[b]:
            q[b] = 0.0
            continue
        draft[b] = int(np.argmax(sc[b]))
        fin = np.sort(sc[b][np.isfinite(sc[b])].astype(np.float64))
        flags[b] = fin.size > 1 and fin[-1] - fin[-2] < margin
    return draft, q, flags


def cut_band(wts: DrafterWeights, g_bits, margin):
    """The masked head's clusters near its cut, per row: (kept, excluded) lists of
    cluster ids -- the kept clusters whose float32 score is within ``margin`` of the
    best excluded one, and the excluded clusters within ``margin`` of the worst kept
    one.  A perturbation of the scores smaller than ``margin / 2`` can only move
    clusters of the band across the cut."""
    g = _w(g_bits)
    cl = mh.cluster_logits(g, _w(wts.centroids))
    c32 = cl.astype(np.float32).astype(np.float64)
    sel, _ = mh.select_clusters(cl, wts.top_k_clusters)
    out = []
    for b in range(g.shape[0]):
        kept = np.zeros(c32.shape[1], dtype=bool)
        kept[sel[b]] = True
        if kept.all():
            out.append(([], []))
            continue
        vk, vk1 = c32[b][kept].min(), c32[b][~kept].max()
        out.append((np.nonzero(kept & (c32[b] < vk1 + margin))[0].tolist(),
                    np.nonzero(~kept & (c32[b] > vk - margin))[0].tolist()))
    return out


def cut_flags(wts: DrafterWeights, g_bits, ids, l64, drafts, temperature, seed, pos, ok, margin):
    """Rows whose draft could change if the clusters of :func:`cut_band` moved across the
    cut: the draft's own cluster is a kept one of the band (it could be dropped), or an
    excluded cluster of the band holds a token whose score comes within ``margin`` of the
    draft's (it could be added and win).  Scores as the draw takes them: the float32
    logit at T = 0; log q + G with q normalised over the kept tokens otherwise.  Returns
    (flags [B], band per row)."""
    B = ids.shape[0]
    flags = np.zeros(B, dtype=bool)
    band = cut_band(wts, g_bits, margin)
    cs = mh.cluster_size(wts.vocab, wts.centroids.shape[0])
    g = _w(g_bits)
    t = float(temperature)
    for b in range(B):
        near_in, near_out = band[b]
        if not ok[b] or (not near_in and not near_out):
            continue
        x = int(drafts[b])
        if x // cs in near_in:
            flags[b] = True
            continue
        if not near_out:
            continue
        extra = (np.asarray(near_out)[:, None] * cs + np.arange(cs)[None, :]).reshape(-1)
        l_extra = (g[b] @ _w(wts.embed[extra]).T).astype(np.float32).astype(np.float64)
        l_kept = np.asarray(l64[b], dtype=np.float64).astype(np.float32).astype(np.float64)
        j = int(np.nonzero(ids[b] == x)[0][0])
        if t == 0.0:
            s_win, s_extra = l_kept[j], l_extra
        else:
            mx = l_kept.max()
            lz = np.log(np.exp((l_kept - mx) / t).sum())
            U = philox.gumbel_uniform_rows(seed, [b], [int(pos[b])], wts.vocab, tag=philox.TAG_DRAFT)[0]
            G = -np.log(-np.log(U))
            s_win = (l_kept[j] - mx) / t - lz + G[x]
            s_extra = (l_extra - mx) / t - lz + G[extra]
        flags[b] = bool(s_extra.max() > s_win - margin)
    return flags, band


def draft(wts: DrafterWeights, kv: SharedKV, last_token, h_target_bits, gamma, temperature, seed, margin=FLAG,
          force=None):
    """gamma autoregressive drafter steps.  Returns a dict with ``draft`` int64 [B, gamma]
    (-1 for rows that are not valid), ``q`` float32 [B, gamma, V] (None at T = 0),
    ``g`` the hidden states after every step (bf16 bits [gamma, B, D]), ``logits`` the
    scored (ids, float64 logits) of every step, and ``flags`` [B, gamma]: the step's
    draft could change under perturbations of ``margin`` -- its two best scores are
    closer than ``margin`` (``flags_draw``), or, with the masked head, clusters near the
    cut could move across it and change the draft (``flags_cut``; :func:`cut_flags`;
    ``band`` lists those clusters per step and row).  Later steps of a flagged row depend
    on it.  ``margin`` is one value or one per step.

    ``force`` (int [B, gamma], optional): the tokens fed back after each step in place
    of the drafts drawn here (entries < 0 keep the drawn draft).  Every step still
    draws and flags its own draft; forcing only chooses the token the next step
    processes, so another implementation's path can be followed past a flagged step.
    Forcing the drafts this function draws reproduces the unforced result."""
    tokens = np.asarray(last_token, dtype=np.int64).copy()
    B = tokens.shape[0]
    ok = valid_rows(kv, tokens, wts.vocab)
    g = np.asarray(h_target_bits, dtype=np.uint16).copy()
    lens = np.asarray(kv.length, dtype=np.int64)
    drafts = np.full((B, gamma), -1, dtype=np.int64)
    qs = None if float(temperature) == 0.0 else np.zeros((B, gamma, wts.vocab), dtype=np.float32)
    flags_draw = np.zeros((B, gamma), dtype=bool)
    flags_cut = np.zeros((B, gamma), dtype=bool)
    bands = []
    gs, ls = [], []
    for k in range(gamma):
        g = step_hidden(wts, kv, np.where(ok, tokens, 0), g, k)
        mk = float(np.broadcast_to(np.asarray(margin, dtype=np.float64), (gamma,))[k])
        ids, l64, _ = scored_logits(wts, g, margin=mk)
        x, q, dflag = sample_step(ids, l64, wts.vocab, temperature, seed, lens + k + 1, ok, mk)
        drafts[:, k] = np.where(ok, x, -1)
        if qs is not None:
            qs[:, k] = q
        flags_draw[:, k] = ok & dflag
        if wts.centroids is not None:
            cf, band = cut_flags(wts, g, ids, l64, x, temperature, seed, lens + k + 1, ok, mk)
            flags_cut[:, k] = ok & cf
            bands.append(band)
        else:
            bands.append([([], [])] * B)
        fed = x if force is None else np.where(np.asarray(force)[:, k] >= 0, np.asarray(force)[:, k], x)
        tokens = np.where(ok, fed, 0)
        gs.append(g.copy())
        ls.append((ids, l64))
    return dict(draft=drafts, q=qs, g=np.stack(gs), logits=ls, flags=flags_draw | flags_cut, flags_draw=flags_draw,
                flags_cut=flags_cut, band=bands)
