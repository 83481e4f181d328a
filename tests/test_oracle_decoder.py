"""Pins of the oracle's reference decoder (full-model verify forward)."""
import copy

import numpy as np
import pytest

from oracle import decoder as dec
from oracle import rules
from oracle.bf16 import f64_to_bf16
import workloads


def test_rmsnorm_constant_vector():
    for c in (0.5, -3.0, 1e-3):
        x = np.full((2, 16), c)
        out = dec.rmsnorm(x, np.full(16, 2.0), 1e-5)
        assert np.allclose(out, 2.0 * c / np.sqrt(c * c + 1e-5), rtol=1e-14)
    # scale invariance without eps
    rng = np.random.default_rng(0)
    x = rng.standard_normal(64)
    assert np.allclose(dec.rmsnorm(7.0 * x, 1.0, 0.0), dec.rmsnorm(x, 1.0, 0.0), rtol=1e-13)
    assert np.isclose(np.mean(dec.rmsnorm(x, 1.0, 0.0) ** 2), 1.0, rtol=1e-13)


def test_rope_is_a_rotation_with_relative_scores():
    rng = np.random.default_rng(1)
    hd = 128
    q = rng.standard_normal((1, 1, hd))
    k = rng.standard_normal((1, 1, hd))
    assert np.array_equal(dec.rope(q, np.array([0]), 10000.0), q)       # position 0
    for m in (1, 17, 2050):
        r = dec.rope(q, np.array([m]), 10000.0)
        half = hd // 2
        # each (j, j + half) pair keeps its length
        assert np.allclose(r[..., :half] ** 2 + r[..., half:] ** 2,
                           q[..., :half] ** 2 + q[..., half:] ** 2, rtol=1e-12)
    # q(m) . k(n) depends on m - n only
    s1 = (dec.rope(q, np.array([2050]), 1e4) * dec.rope(k, np.array([2047]), 1e4)).sum()
    s2 = (dec.rope(q, np.array([10]), 1e4) * dec.rope(k, np.array([7]), 1e4)).sum()
    assert np.isclose(s1, s2, rtol=1e-9)
    # j = 0 pair rotates by exactly pos radians
    e = np.zeros((1, 1, hd))
    e[..., 0] = 1.0
    r = dec.rope(e, np.array([3]), 1e4)
    assert np.isclose(r[..., 0], np.cos(3.0)) and np.isclose(r[..., half], np.sin(3.0))


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((1, 8))
    v = rng.standard_normal((1, 8))
    assert np.allclose(dec.attention(q, k, v), np.repeat(v, 3, 0), rtol=1e-14)
    k2 = np.repeat(k, 5, 0)
    v2 = rng.standard_normal((5, 8))
    assert np.allclose(dec.attention(q, k2, v2), np.repeat(v2.mean(0, keepdims=True), 3, 0), rtol=1e-13)
    # a dominant key
    k3 = np.zeros((4, 8))
    k3[2] = 100 * q[0]
    out = dec.attention(q[:1], k3, v2[:4])
    assert np.allclose(out[0], v2[2], atol=1e-12)


def test_silu_values():
    assert dec.silu(np.array([0.0]))[0] == 0.0
    x = np.linspace(-5, 5, 11)
    assert np.allclose(dec.silu(x) - dec.silu(-x), x, rtol=1e-14)   # silu(x) - silu(-x) = x
    assert np.isclose(dec.silu(np.array([1.0]))[0], 1 / (1 + np.exp(-1)))


def tiny_model(seed=0, L=2, d=32, H=4, hd=8, ff=48, V=40, cache_len=6, B=2, max_len=64, std=0.3):
    rng = np.random.default_rng(seed)

    def w(*shape):
        return f64_to_bf16(rng.standard_normal(shape) * std)

    layers = []
    for _ in range(L):
        layers.append({"attn_norm": f64_to_bf16(1 + 0.1 * rng.standard_normal(d)),
                       "wq": w(H * hd, d), "wk": w(H * hd, d), "wv": w(H * hd, d), "wo": w(d, H * hd),
                       "ffn_norm": f64_to_bf16(1 + 0.1 * rng.standard_normal(d)),
                       "w_gate": w(ff, d), "w_up": w(ff, d), "w_down": w(d, ff)})
    wts = dec.DecoderWeights(L, d, H, hd, ff, V, 1e-5, 10000.0, embed=w(V, d), layers=layers,
                             final_norm=f64_to_bf16(np.ones(d)), lm_head=f64_to_bf16(rng.standard_normal((V, d))))
    k = np.zeros((L, B, H, max_len, hd), np.uint16)
    v = np.zeros_like(k)
    k[:, :, :, :cache_len] = f64_to_bf16(rng.standard_normal((L, B, H, cache_len, hd)))
    v[:, :, :, :cache_len] = f64_to_bf16(rng.standard_normal((L, B, H, cache_len, hd)))
    kv = dec.KVCache(k, v, np.full(B, cache_len, np.int64))
    return wts, kv


def test_one_pass_equals_sequential_passes():
    wts, kv = tiny_model()
    rng = np.random.default_rng(3)
    toks = rng.integers(0, wts.vocab, (2, 5))
    kv1 = copy.deepcopy(kv)
    full = dec.forward(wts, toks, kv1)
    kv2 = copy.deepcopy(kv)
    for i in range(5):
        one = dec.forward(wts, toks[:, i:i + 1], kv2)
        dec.commit(kv2, np.zeros(2, np.int64))
        assert np.allclose(one[:, 0], full[:, i], rtol=0, atol=1e-12 * np.abs(full).max())
    assert np.array_equal(kv1.k[:, :, :, :11], kv2.k[:, :, :, :11])
    assert np.array_equal(kv1.v[:, :, :, :11], kv2.v[:, :, :, :11])


def test_causality_later_tokens_do_not_change_earlier_slots():
    wts, kv = tiny_model(seed=4)
    rng = np.random.default_rng(4)
    toks = rng.integers(0, wts.vocab, (2, 5))
    a = dec.forward(wts, toks, copy.deepcopy(kv))
    for j in range(1, 5):
        t2 = toks.copy()
        t2[:, j] = (t2[:, j] + 1 + rng.integers(0, wts.vocab - 1)) % wts.vocab
        b = dec.forward(wts, t2, copy.deepcopy(kv))
        assert np.array_equal(a[:, :j], b[:, :j])
        assert not np.allclose(a[:, j], b[:, j])


@pytest.mark.parametrize("gamma,corrupt", [(4, 0.3), (2, 0.5), (6, 0.15)])
def test_greedy_speculative_equals_greedy_autoregressive(gamma, corrupt):
    """[MTP-deep-dive] section 2.2: under greedy decoding the speculative output
    is identical to the target's own autoregressive output, whatever the
    drafter proposes; cache length equals sequence length after every round
    ([Self-spec] section 3.3)."""
    wts, kv0 = tiny_model(seed=5 + gamma, B=2, max_len=256)
    steps = 30
    first = np.array([3, 17])
    ar = dec.greedy_autoregressive(wts, first, copy.deepcopy(kv0), steps + gamma + 2)
    rng = np.random.default_rng(gamma)
    kv = copy.deepcopy(kv0)
    B = 2
    out = [[] for _ in range(B)]
    last = first.copy()
    seen_n = set()
    while min(len(o) for o in out) < steps:
        # drafter: the true continuation, with some tokens corrupted
        draft = np.zeros((B, gamma), np.int64)
        for b in range(B):
            pos = len(out[b])
            cont = np.zeros(gamma, np.int64)
            avail = ar[b, pos:pos + gamma]
            cont[:len(avail)] = avail
            bad = rng.random(gamma) < corrupt
            draft[b] = np.where(bad, (cont + 1 + rng.integers(0, wts.vocab - 1, gamma)) % wts.vocab, cont)
        toks = np.concatenate([last[:, None], draft], axis=1)
        logits = dec.forward(wts, toks, kv)
        n, tok, _ = rules.verify_greedy(logits, draft)
        dec.commit(kv, n)
        for b in range(B):
            emitted = [int(t) for t in tok[b, :n[b] + 1]]
            out[b].extend(emitted)
            last[b] = emitted[-1]
            seen_n.add(int(n[b]))
            # cache length == context + emitted tokens (slot-0 token now cached)
            assert kv.length[b] == kv0.length[b] + len(out[b])
    for b in range(B):
        assert out[b][:steps] == [int(t) for t in ar[b, :steps]]
    assert len(seen_n) >= 3


def test_generated_small_decoder_case_runs():
    c = workloads.small_decoder_case(n_layers=1, d_model=64, n_heads=1, head_dim=64, d_ff=128,
                                     vocab=100, cache_len=10)
    wts = dec.DecoderWeights(c.n_layers, c.d_model, c.n_heads, c.head_dim, c.d_ff, c.vocab, c.rms_eps,
                             c.rope_theta, c.embed, c.layers, c.final_norm, c.lm_head)
    kv = dec.KVCache(c.k_cache.copy(), c.v_cache.copy(), c.length.astype(np.int64))
    logits = dec.forward(wts, c.tokens, kv)
    assert logits.shape == (1, 5, 100) and np.all(np.isfinite(logits))
