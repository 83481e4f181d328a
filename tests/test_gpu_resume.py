"""Checkpoint and resume of multi-round speculative decoding on the GPU.

The state of a decoding run between rounds is the emitted tokens (the next round's slot
0), the KV cache with its lengths, the positions (pos0 = the cache length) and the seed:
the random draws are counter-based (Philox keyed by seed, sequence and position), so
nothing else carries over ([Self-spec] 3.3: the cache length must equal the sequence
length).  A run of 1000 rounds must therefore equal a run of 500 rounds whose state is
copied to the host, written to a file and read back into fresh device buffers (a new
model, cache and workspace) for the remaining 500: the same accepted counts and tokens
in every round and the same cache bits at the end.  Greedy and sampling (T = 1), two
sequences that advance by different amounts."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from tests.gpu_util import dev, dev_bf16, log

pytestmark = pytest.mark.gpu

ROUNDS, SPLIT, GAMMA, B = 1000, 500, 4, 2


def case():
    return workloads.small_decoder_case(n_layers=2, d_model=128, n_heads=2, head_dim=64, d_ff=256, vocab=200,
                                        cache_len=8, B=B, gamma=GAMMA, max_len=8 + (ROUNDS + 1) * (GAMMA + 1),
                                        std=0.1)


def drafts(r, last, V):
    """The drafts of round r, a function of the round and the carried state only: the
    last emitted token (the small random decoder often repeats its argmax) or, 30 % of
    the time, a random token."""
    rng = np.random.default_rng([91, r])
    rnd = rng.integers(0, V, size=(B, GAMMA))
    keep = rng.random((B, GAMMA)) < 0.7
    return np.where(keep, last[:, None], rnd).astype(np.int32)


def model_on_device(c):
    layers = [{k: dev_bf16(L[k]) for k in sv.LAYER_KEYS} for L in c.layers]
    return sv.decoder_model(dev_bf16(c.embed), layers, dev_bf16(c.final_norm), dev_bf16(c.lm_head), c.n_heads,
                            c.head_dim, c.rms_eps, c.rope_theta)


def run_rounds(c, model, kv, last, r0, r1, T, ws):
    q = dev(np.full((B, GAMMA, c.vocab), 1.0 / c.vocab, dtype=np.float32))
    length = kv.length.cpu().numpy().astype(np.int64)
    out = []
    for r in range(r0, r1):
        toks = dev(np.concatenate([last[:, None], drafts(r, last, c.vocab)], axis=1).astype(np.int32))
        if T == 0.0:
            n, tok = sv.spec_verify_greedy(model, sv.SV_IN_TOKENS, toks, B, GAMMA, None, kv=kv, ws=ws)
        else:
            n, tok = sv.spec_verify_sample(model, sv.SV_IN_TOKENS, toks, B, GAMMA, None, q, T, c.seed, dev(length),
                                           kv=kv, ws=ws)
        n, tok = n.cpu().numpy(), tok.cpu().numpy()
        assert np.all(n >= 0), f"round {r}: invalid sequence"
        last = tok[np.arange(B), n].astype(np.int32)
        length = length + n + 1
        assert np.array_equal(kv.length.cpu().numpy(), length), f"round {r}: cache length != sequence length"
        out.append((n, tok))
    return out, last


def bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1.0, 0.0])
def test_1000_rounds_equal_500_plus_500_resumed(T, tmp_path):
    c = case()
    first = c.tokens[:, 0].astype(np.int32)
    log(f"[resume] T={T}: {ROUNDS} rounds uninterrupted")
    model = model_on_device(c)
    kv = sv.KVCache(dev_bf16(c.k_cache), dev_bf16(c.v_cache), dev(c.length.astype(np.int32)))
    whole, _ = run_rounds(c, model, kv, first, 0, ROUNDS, T, sv.Workspace())
    k_whole, v_whole, len_whole = bits(kv.k), bits(kv.v), kv.length.cpu().numpy()
    del model, kv

    log(f"[resume] T={T}: {SPLIT} rounds, checkpoint to a file, {ROUNDS - SPLIT} rounds on fresh buffers")
    model = model_on_device(c)
    kv = sv.KVCache(dev_bf16(c.k_cache), dev_bf16(c.v_cache), dev(c.length.astype(np.int32)))
    part1, last = run_rounds(c, model, kv, first, 0, SPLIT, T, sv.Workspace())
    ck = tmp_path / "state.npz"
    np.savez(ck, k=bits(kv.k), v=bits(kv.v), length=kv.length.cpu().numpy(), last=last, round=SPLIT, seed=c.seed)
    del model, kv
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    st = np.load(ck)
    assert int(st["round"]) == SPLIT and int(st["seed"]) == c.seed
    model = model_on_device(c)
    kv = sv.KVCache(dev_bf16(st["k"]), dev_bf16(st["v"]), dev(st["length"]))
    part2, _ = run_rounds(c, model, kv, st["last"], SPLIT, ROUNDS, T, sv.Workspace())

    resumed = part1 + part2
    for r, ((n0, t0), (n1, t1)) in enumerate(zip(whole, resumed)):
        assert np.array_equal(n0, n1) and np.array_equal(t0, t1), f"round {r} differs after resume"
    assert np.array_equal(kv.length.cpu().numpy(), len_whole)
    assert np.array_equal(bits(kv.k), k_whole) and np.array_equal(bits(kv.v), v_whole)
    ns = np.array([n for n, _ in whole])
    log(f"[resume] T={T}: identical; accepted per round mean {ns.mean(axis=0)}, counts "
        f"{np.bincount(ns.reshape(-1), minlength=GAMMA + 1).tolist()}, final lengths {len_whole.tolist()}")
    assert len(np.unique(ns)) >= 3 and not np.array_equal(ns[:, 0], ns[:, 1])
