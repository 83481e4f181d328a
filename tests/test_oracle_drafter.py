"""Pins of the drafter oracle (oracle/drafter.py) against properties the pages and the
mathematics fix: autoregressive chaining, the order of the joined input, the attention
reading exactly the cached positions, the masked head with every cluster kept equal to
the tied head, the law of the drafted tokens, and the T -> 0 limit."""
import numpy as np
import pytest
from scipy import stats

import workloads
from oracle import drafter as od
from oracle import rules


def weights(c, masked=True, top_k=None):
    layers = [dict(L) for L in c.layers]
    return od.DrafterWeights(d_model=c.d_model, hidden=c.hidden, n_heads=c.n_heads, head_dim=c.head_dim,
                             d_ff=c.d_ff, vocab=c.vocab, rms_eps=1e-5, rope_theta=10000.0, embed=c.embed,
                             pre_proj=c.pre_proj.copy(), layers=layers, final_norm=c.final_norm,
                             post_proj=c.post_proj, centroids=c.centroids if masked else None,
                             top_k_clusters=top_k or c.top_k)


def shared(c):
    return od.SharedKV(k=[a.copy() for a in c.kv_k], v=[a.copy() for a in c.kv_v], length=c.length.copy())


def small(B=3, **kw):
    args = dict(V=4096, D=256, H=128, n_layers=2, n_heads=2, head_dim=64, d_ff=256, C=64, top_k=8, B=B,
                length=[5, 40, 100][:B] if B <= 3 else 50)
    args.update(kw)
    return workloads.drafter_case(**args)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_gamma_steps_equal_chained_single_steps(T):
    c = small()
    w, kv = weights(c), shared(c)
    full = od.draft(w, kv, c.last_token, c.h_target, 3, T, c.seed)
    tok, g = c.last_token.astype(np.int64), c.h_target
    lens = c.length.astype(np.int64)
    for k in range(3):
        # one step by hand: the hidden state, the head, the draw at position len + k + 1
        g = od.step_hidden(w, kv, tok, g, k)
        ids, l64, _ = od.scored_logits(w, g)
        x, q, _ = od.sample_step(ids, l64, c.vocab, T, c.seed, lens + k + 1, np.ones(3, bool))
        assert np.array_equal(g, full["g"][k])
        assert np.array_equal(x, full["draft"][:, k])
        if T > 0:
            assert np.array_equal(q, full["q"][:, k])
        tok = x
    # the cache is read, never written
    assert all(np.array_equal(a, b) for a, b in zip(kv.k, c.kv_k))


def test_joined_input_order():
    """Zeroing the hidden half of pre_proj makes the drafts ignore the target state;
    zeroing the embedding half makes them ignore the token ([embedding, hidden])."""
    c = small()
    D = c.d_model
    other_h = workloads.normal_bf16(c.h_target.shape, 1.0, 5, (77,))
    other_t = (c.last_token + 1000) % c.vocab
    w = weights(c)
    w.pre_proj = c.pre_proj.copy()
    w.pre_proj[:, D:] = 0
    a = od.draft(w, shared(c), c.last_token, c.h_target, 2, 0.0, 1)
    b = od.draft(w, shared(c), c.last_token, other_h, 2, 0.0, 1)
    assert np.array_equal(a["g"], b["g"])
    t = od.draft(w, shared(c), other_t, c.h_target, 2, 0.0, 1)
    assert not np.array_equal(a["g"][0], t["g"][0])
    w.pre_proj = c.pre_proj.copy()
    w.pre_proj[:, :D] = 0
    a = od.draft(w, shared(c), c.last_token, c.h_target, 1, 0.0, 1)
    t = od.draft(w, shared(c), other_t, c.h_target, 1, 0.0, 1)
    assert np.array_equal(a["g"], t["g"])
    b = od.draft(w, shared(c), c.last_token, other_h, 1, 0.0, 1)
    assert not np.array_equal(a["g"][0], b["g"][0])


def test_attention_reads_exactly_the_cached_positions():
    c = small()
    w = weights(c)
    base = od.draft(w, shared(c), c.last_token, c.h_target, 2, 0.0, 1)["g"]
    kv = shared(c)
    for l in range(len(kv.k)):
        for b in range(3):
            n = int(c.length[b])
            kv.k[l][b, :, n:, :] = 0x3f80        # bf16 1.0 at and beyond len: invisible
            kv.v[l][b, :, n:, :] = 0x4000
    assert np.array_equal(od.draft(w, kv, c.last_token, c.h_target, 2, 0.0, 1)["g"], base)
    kv = shared(c)
    kv.v[0][1, :, int(c.length[1]) - 1, :] = 0x4000   # the last cached value is visible
    assert not np.array_equal(od.draft(w, kv, c.last_token, c.h_target, 1, 0.0, 1)["g"][0][1], base[0][1])
    # a one-entry cache: softmax over one key is 1 whatever the key
    c1 = small(length=[1, 1, 1])
    kv = shared(c1)
    g0 = od.draft(w, kv, c1.last_token, c1.h_target, 1, 0.0, 1)["g"]
    for l in range(len(kv.k)):
        kv.k[l][:, :, 0, :] = workloads.normal_bf16(kv.k[l][:, :, 0, :].shape, 3.0, 9, (l,))
    assert np.array_equal(od.draft(w, kv, c1.last_token, c1.h_target, 1, 0.0, 1)["g"], g0)


def test_masked_head_with_every_cluster_kept_is_the_tied_head():
    c = small(C=64)
    a = od.draft(weights(c, masked=True, top_k=64), shared(c), c.last_token, c.h_target, 2, 0.8, 11)
    b = od.draft(weights(c, masked=False), shared(c), c.last_token, c.h_target, 2, 0.8, 11)
    assert np.array_equal(a["draft"], b["draft"])
    np.testing.assert_allclose(a["q"], b["q"], rtol=1e-6, atol=1e-12)
    ids, l64 = a["logits"][0]
    o = np.argsort(ids[0])
    np.testing.assert_allclose(l64[0][o], b["logits"][0][1][0], rtol=0, atol=1e-12)


def test_drafts_follow_q_and_zero_temperature_is_argmax():
    """One step over many seeds: the drafted token's frequencies match q (chi-square);
    a tiny temperature drafts the argmax of the logits."""
    c = small(B=1, V=512, C=8, top_k=8, length=30)
    w = weights(c)
    kv = shared(c)
    g = od.step_hidden(w, kv, c.last_token.astype(np.int64), c.h_target, 0)
    ids, l64, _ = od.scored_logits(w, g)
    T = 2.5
    counts = np.zeros(c.vocab)
    n = 6000
    q = None
    for s in range(n):
        x, q, _ = od.sample_step(ids, l64, c.vocab, T, 1000 + s, np.array([31]), np.ones(1, bool))
        counts[x[0]] += 1
    p = q[0].astype(np.float64)
    keep = p * n >= 5
    exp = p[keep] * n
    obs = counts[keep]
    chi = ((obs - exp) ** 2 / exp).sum() + (counts[~keep].sum() - p[~keep].sum() * n) ** 2 / max(p[~keep].sum() * n, 1e-9)
    assert stats.chi2.sf(chi, keep.sum()) > 1e-4
    x0, _, _ = od.sample_step(ids, l64, c.vocab, 0.0, 1, np.array([31]), np.ones(1, bool))
    xt, _, _ = od.sample_step(ids, l64, c.vocab, 1e-4, 1, np.array([31]), np.ones(1, bool))
    assert x0[0] == xt[0] == ids[0][np.argmax(l64[0].astype(np.float32))]
    assert np.isclose(q.sum(), 1.0, atol=1e-5)


def test_invalid_rows_draft_nothing():
    c = small(length=[0, 40, 100])
    out = od.draft(weights(c), shared(c), c.last_token, c.h_target, 2, 1.0, 3)
    assert np.all(out["draft"][0] == -1) and np.all(out["q"][0] == 0)
    assert np.all(out["draft"][1:] >= 0)
    c = small()
    t = c.last_token.copy()
    t[2] = c.vocab + 5
    out = od.draft(weights(c), shared(c), t, c.h_target, 2, 1.0, 3)
    assert np.all(out["draft"][2] == -1) and np.all(out["draft"][:2] >= 0)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_forcing_own_drafts_changes_nothing_and_other_tokens_are_fed(T):
    """force = the drafts the oracle draws reproduces the unforced result exactly; forcing
    another token at step 0 changes what step 1 processes (the hidden state and the draw
    of step 1 follow the forced token) while step 0 itself is unchanged."""
    c = small()
    w, kv = weights(c), shared(c)
    free = od.draft(w, kv, c.last_token, c.h_target, 3, T, c.seed)
    same = od.draft(w, kv, c.last_token, c.h_target, 3, T, c.seed, force=free["draft"])
    for key in ("draft", "flags", "g"):
        assert np.array_equal(free[key], same[key])
    other = free["draft"].copy()
    other[:, 0] = (other[:, 0] + 17) % c.vocab
    other[:, 1:] = -1                               # later steps keep their own drafts
    forced = od.draft(w, kv, c.last_token, c.h_target, 3, T, c.seed, force=other)
    assert np.array_equal(forced["draft"][:, 0], free["draft"][:, 0])
    assert np.array_equal(forced["g"][0], free["g"][0])
    assert not np.array_equal(forced["g"][1], free["g"][1])
    # and step 1 of the forced run is the unforced step taken from the forced token
    tok = other[:, 0].astype(np.int64)
    g1 = od.step_hidden(w, kv, tok, free["g"][0], 1)
    assert np.array_equal(g1, forced["g"][1])


def _draw_over(w, g_bits, clusters, T, seed, pos, b):
    """The draft of row b drawn over the member tokens of ``clusters`` (brute force)."""
    from oracle import philox
    from oracle.bf16 import bf16_to_f64
    cs = c_size(w)
    toks = (np.sort(np.asarray(clusters))[:, None] * cs + np.arange(cs)[None, :]).reshape(-1)
    l32 = (bf16_to_f64(g_bits[b]) @ bf16_to_f64(w.embed[toks]).T).astype(np.float32)
    if T == 0.0:
        return int(toks[np.argmax(l32)])
    q = rules.target_probs(l32, T).astype(np.float32)
    U = philox.gumbel_uniform_rows(seed, [b], [pos], w.vocab, tag=philox.TAG_DRAFT)[0][toks].astype(np.float32)
    sc = np.where(q > 0, np.log(q) + (-np.log(-np.log(U))), -np.inf)
    return int(toks[np.argmax(sc)])


def c_size(w):
    return w.vocab // w.centroids.shape[0]


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_cut_flags_by_moving_each_band_cluster(T):
    """A step is cut-flagged only if moving a cluster of the band across the cut can change
    its draft: for every unflagged row, dropping any kept band cluster or adding any
    excluded one (one at a time) leaves the draft unchanged (brute force), and a margin
    of 0 gives an empty band."""
    c = small(B=3, top_k=8)
    w, kv = weights(c), shared(c)
    lens = c.length.astype(np.int64)
    g = od.step_hidden(w, kv, c.last_token.astype(np.int64), c.h_target, 0)
    ids, l64, _ = od.scored_logits(w, g)
    ok = np.ones(3, bool)
    x, _, _ = od.sample_step(ids, l64, c.vocab, T, c.seed, lens + 1, ok)
    assert all(not a and not e for a, e in od.cut_band(w, g, 0.0))
    checked = 0
    for mg in (0.05, 0.2, 0.5):
        flags, band = od.cut_flags(w, g, ids, l64, x, T, c.seed, lens + 1, ok, mg)
        sel = (ids[:, ::c_size(w)] // c_size(w))
        for b in range(3):
            if flags[b]:
                continue
            kept = set(sel[b].tolist())
            near_in, near_out = band[b]
            for cl in near_in:
                assert _draw_over(w, g, sorted(kept - {cl}), T, c.seed, int(lens[b] + 1), b) == x[b]
                checked += 1
            for cl in near_out:
                assert _draw_over(w, g, sorted(kept | {cl}), T, c.seed, int(lens[b] + 1), b) == x[b]
                checked += 1
    assert checked > 0
