"""The oracle's multi-round decoding is a function of its carried state alone: 40 rounds
of speculative sampling on the small decoder equal 20 rounds, the state (KV cache and
lengths, last tokens, seed) written to a file and read back, then 20 more rounds
([Self-spec] 3.3; the random draws are keyed by seed, sequence and position).  The GPU
counterpart is tests/test_gpu_resume.py."""
import numpy as np

import workloads
from oracle import decoder as dec
from oracle import rules

GAMMA, B, T = 4, 2, 1.0


def run(c, wts, kv, last, r0, r1):
    q = np.full((B, GAMMA, c.vocab), 1.0 / c.vocab)
    out = []
    for r in range(r0, r1):
        draft = np.random.default_rng([91, r]).integers(0, c.vocab, size=(B, GAMMA))
        toks = np.concatenate([last[:, None], draft], axis=1)
        pos0 = np.asarray(kv.length, dtype=np.int64).copy()
        logits = dec.forward(wts, toks, kv)
        n, tok, _ = rules.verify_sample(logits, draft, q, T, c.seed, pos0)
        dec.commit(kv, n)
        last = tok[np.arange(B), n]
        out.append((n, tok))
    return out, last


def test_40_rounds_equal_20_plus_20_resumed(tmp_path):
    c = workloads.small_decoder_case(n_layers=1, d_model=64, n_heads=2, head_dim=32, d_ff=128, vocab=50,
                                     cache_len=4, B=B, gamma=GAMMA, max_len=4 + 41 * (GAMMA + 1), std=0.2)
    wts = dec.DecoderWeights(c.n_layers, c.d_model, c.n_heads, c.head_dim, c.d_ff, c.vocab, c.rms_eps,
                             c.rope_theta, c.embed, c.layers, c.final_norm, c.lm_head)
    first = c.tokens[:, 0].astype(np.int64)
    kv = dec.KVCache(c.k_cache.copy(), c.v_cache.copy(), c.length.astype(np.int64))
    whole, _ = run(c, wts, kv, first, 0, 40)
    k_whole, v_whole, len_whole = kv.k.copy(), kv.v.copy(), np.asarray(kv.length).copy()

    kv = dec.KVCache(c.k_cache.copy(), c.v_cache.copy(), c.length.astype(np.int64))
    part1, last = run(c, wts, kv, first, 0, 20)
    np.savez(tmp_path / "state.npz", k=kv.k, v=kv.v, length=kv.length, last=last)
    st = np.load(tmp_path / "state.npz")
    kv = dec.KVCache(st["k"].copy(), st["v"].copy(), st["length"].copy())
    part2, _ = run(c, wts, kv, st["last"], 20, 40)

    for (n0, t0), (n1, t1) in zip(whole, part1 + part2):
        assert np.array_equal(n0, n1) and np.array_equal(t0, t1)
    assert np.array_equal(kv.k, k_whole) and np.array_equal(kv.v, v_whole)
    assert np.array_equal(kv.length, len_whole)
    # the cache length is the sequence length: initial length plus every emitted token
    emitted = sum(n + 1 for n, _ in whole)
    assert np.array_equal(len_whole, c.length + emitted)
    assert len(np.unique(np.array([n for n, _ in whole]))) >= 2
