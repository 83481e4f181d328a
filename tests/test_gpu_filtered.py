"""GPU parity of spec_verify_sample_filtered (speculative sampling with the drafter's
top-k / top-p filters applied alike to the target) against the oracle's
verify_sample_filtered: n and tokens bit-exact except on sequences the oracle flags
(a filter cut or a sampling decision within its rounding margin).  q is the drafter's
distribution filtered with the same parameters, as a drafter that follows the rule
would send it; the drafts are drawn from it."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import rules
from tests.gpu_util import (check_token_structure, compare_decisions, dev, dev_bf16, log, oracle_logits_bf16,
                            row_rel_err)

pytestmark = pytest.mark.gpu


def filtered_drafter(target_f32, noise, T, top_k, top_p, rng):
    """Drafter logits = target + noise; q = the filtered distribution (the same filters);
    drafts x ~ q by inverse CDF.  Returns (draft int32 [B, gamma], q bf16 bits)."""
    z = (target_f32 + noise).astype(np.float32)
    q, _, _ = rules.filtered_probs(z, T, top_k, top_p)
    qb = workloads.to_bf16_bits(q)
    qf = workloads.bf16_bits_to_f32(qb).astype(np.float64)
    B, g, V = q.shape
    cdf = np.cumsum(qf, axis=-1)
    u = rng.random((B, g)) * cdf[..., -1]
    x = np.empty((B, g), dtype=np.int32)
    for b in range(B):
        for i in range(g):
            j = min(int(np.searchsorted(cdf[b, i], u[b, i], side="right")), V - 1)
            while qf[b, i, j] == 0.0:           # never land on a zero of the rounded q
                j -= 1
            x[b, i] = j
    return x, qb


def case(V, d, B, gamma, T, top_k, top_p, seed, noise_std=0.7, w=None, bad_drafts=True):
    rng = np.random.default_rng(seed)
    if w is None:
        w = workloads.to_bf16_bits((rng.standard_normal((V, d)) * 0.3).astype(np.float32))
    h = workloads.to_bf16_bits(rng.standard_normal((B, gamma + 1, d)).astype(np.float32))
    ref = oracle_logits_bf16(h, w)
    lt = rules.f32_logits(ref[:, :gamma])
    noise = rng.standard_normal((B, gamma, V)).astype(np.float32) * noise_std
    draft, qb = filtered_drafter(lt, noise, T, top_k, top_p, rng)
    if bad_drafts:
        bad = rng.random((B, gamma)) < 0.05
        draft = np.where(bad, np.where(rng.random((B, gamma)) < 0.5, -3, V + 7), draft).astype(np.int32)
    pos0 = rng.integers(0, 5000, B).astype(np.int64)
    return dict(w=w, h=h, ref=ref, draft=draft, qb=qb, pos0=pos0, seed=777 + seed, T=T, k=top_k, p=top_p)


def run(model, c, B, gamma, logits_out=None, kind=sv.SV_IN_HIDDEN, inp=None):
    inp = dev_bf16(c["h"]) if inp is None else inp
    return sv.spec_verify_sample_filtered(model, kind, inp, B, gamma, dev(c["draft"]), dev_bf16(c["qb"]), c["T"],
                                          c["k"], c["p"], c["seed"], dev(c["pos0"]), logits_out=logits_out)


def oracle(c):
    qf = workloads.bf16_bits_to_f32(c["qb"]).astype(np.float64)
    return rules.verify_sample_filtered(c["ref"], c["draft"], qf, c["T"], c["k"], c["p"], c["seed"], c["pos0"])


SMALL = [
    # (V, d, B, gamma, T, top_k, top_p)
    (1000, 96, 3, 4, 1.0, 64, 0.95),     # one ragged chunk
    (9000, 64, 5, 4, 0.7, 20, 0.9),      # three chunks, the last ragged
    (4096, 256, 4, 3, 1.0, 64, 1.0),     # top_p = 1: the whole top-k set
    (4099, 128, 2, 15, 1.0, 8, 0.5),     # largest gamma, a 3-logit last chunk
    (30, 32, 4, 4, 1.0, 64, 0.95),       # fewer tokens than top_k
    (2, 32, 3, 1, 1.0, 64, 1.0),         # smallest vocabulary and gamma
    (5000, 64, 3, 4, 1.0, 1, 0.95),      # top_k 1: the argmax only
    (5000, 64, 3, 4, 1.0, 64, 0.01),     # top_p below the largest probability: one token
    (20000, 64, 2, 4, 2.0, 64, 0.95),    # flat distribution at high temperature
]


@pytest.mark.parametrize("V,d,B,gamma,T,top_k,top_p", SMALL)
def test_small_and_ragged(V, d, B, gamma, T, top_k, top_p):
    log(f"[filtered] V={V} d={d} B={B} gamma={gamma} T={T} top_k={top_k} top_p={top_p}")
    c = case(V, d, B, gamma, T, top_k, top_p, seed=V + d + B + gamma + top_k)
    model = sv.lm_head_model(dev_bf16(c["w"]))
    logits = torch.empty((B, gamma + 1, V), dtype=torch.float32, device="cuda")
    n, tok = run(model, c, B, gamma, logits)
    torch.cuda.synchronize()
    assert row_rel_err(logits.cpu().numpy(), c["ref"]).max() <= 1e-4
    n0, t0, fl = oracle(c)
    check_token_structure(n.cpu().numpy(), tok.cpu().numpy(), gamma)
    m, f = compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"V={V} k={top_k} p={top_p}")
    log(f"[filtered] n={n.cpu().numpy().tolist()} mismatched {m} flagged {f}")
    # the same logits given as logits input (the chunked selection over the logits
    # instead of the product's per-workgroup candidates) decide identically
    n2, tok2 = run(sv.logits_model(V), c, B, gamma, kind=sv.SV_IN_LOGITS, inp=logits)
    torch.cuda.synchronize()
    assert torch.equal(n, n2) and torch.equal(tok, tok2)
    # every emitted token lies in the kept set of its slot
    p32, kept, _ = rules.filtered_probs(rules.f32_logits(c["ref"]), T, top_k, top_p)
    nh, th = n.cpu().numpy(), tok.cpu().numpy()
    for b in range(B):
        y = int(th[b, nh[b]])
        assert kept[b, nh[b], y], (b, y)


def test_greedy_limit_and_logits_input():
    """T = 0 takes the greedy rule; the logits input path gives the same decisions."""
    V, d, B, gamma = 4099, 128, 4, 4
    c = case(V, d, B, gamma, 1.0, 64, 0.9, seed=11)
    model = sv.lm_head_model(dev_bf16(c["w"]))
    c0 = dict(c, T=0.0)
    n, tok = run(model, c0, B, gamma)
    torch.cuda.synchronize()
    n0, t0, fl = rules.verify_sample_filtered(c["ref"], c["draft"], None, 0.0, 64, 0.9, 0, c["pos0"])
    compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, "greedy")
    l32 = rules.f32_logits(c["ref"])
    n, tok = run(sv.logits_model(V), c, B, gamma, kind=sv.SV_IN_LOGITS, inp=dev(l32))
    torch.cuda.synchronize()
    n0, t0, fl = oracle(c)
    compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, "logits input")


LARGE = [(1, 1.0), (4, 1.0), (4, 0.7)]


@pytest.fixture(scope="module")
def large_w():
    log("[filtered large] generating the 262144 x 1536 table")
    return workloads.large_vocab(B=1, temperature=1.0).w


@pytest.mark.parametrize("B,T", LARGE)
def test_large_vocab_deployment_filters(large_w, B, T):
    """V = 262144, d = 1536, gamma = 4 with top_k 64, top_p 0.95, the deployment's filters."""
    log(f"[filtered large] B={B} T={T}")
    c = case(262144, 1536, B, 4, T, 64, 0.95, seed=100 + B, noise_std=1.0, w=large_w, bad_drafts=False)
    model = sv.lm_head_model(dev_bf16(large_w))
    n, tok = run(model, c, B, 4)
    torch.cuda.synchronize()
    n0, t0, fl = oracle(c)
    m, f = compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"B={B} T={T}")
    log(f"[filtered large] B={B} T={T} n={n.cpu().numpy().tolist()} mismatched {m} flagged {f}")
    n2, tok2 = run(model, c, B, 4)
    torch.cuda.synchronize()
    assert torch.equal(n, n2) and torch.equal(tok, tok2)


@pytest.mark.parametrize("V,top_k", [(10000, 64), (10000, 7), (4096, 64)])
def test_ties_at_the_top_k_cut(V, top_k):
    """Integer-valued float32 logits (given as logits input, so both sides see the same
    numbers) put many exact ties at the top-k cut, within and across chunks.  Drafts come
    from the tied class at the cut, with q tiny at every token: a draft the lower-index
    rule keeps is accepted surely, one it drops (p~ = 0) is rejected surely, so n is
    decided by kept-set membership alone and must equal the oracle's exactly."""
    B, gamma, T = 64, 4, 4.0
    rng = np.random.default_rng(V + top_k)
    l32 = np.floor(rng.standard_normal((B, gamma + 1, V)) * 3.0).astype(np.float32)
    draft = np.empty((B, gamma), dtype=np.int32)
    for b in range(B):
        for i in range(gamma):
            row = l32[b, i].astype(np.float64)
            order = np.lexsort((np.arange(V), -row))
            cut = row[order[top_k - 1]]
            tied = np.nonzero(row == cut)[0]
            draft[b, i] = tied[rng.integers(len(tied))]
    q = np.full((B, gamma, V), 1e-7, dtype=np.float32)
    pos0 = rng.integers(0, 1000, B).astype(np.int64)
    n, tok = sv.spec_verify_sample_filtered(sv.logits_model(V), sv.SV_IN_LOGITS, dev(l32), B, gamma, dev(draft),
                                            dev(q), T, top_k, 1.0, 99, dev(pos0))
    torch.cuda.synchronize()
    n, tok = n.cpu().numpy(), tok.cpu().numpy()
    n0, t0, _ = rules.sample_rule_filtered(l32, draft, q.astype(np.float64), T, top_k, 1.0, 99, pos0)
    assert n.tolist() == n0.tolist()
    _, kept, _ = rules.filtered_probs(l32, T, top_k, 1.0)
    for b in range(B):
        assert tok[b, :n[b]].tolist() == draft[b, :n[b]].tolist()
        assert kept[b, n[b], tok[b, n[b]]]
    log(f"[filtered ties] V={V} top_k={top_k} accepted drafts {int(n.sum())} of {B * gamma}")


@pytest.mark.parametrize("V,top_k,seed", [(10000, 64, 0), (10000, 7, 1), (4096, 64, 2), (3001, 33, 3)])
def test_ties_at_the_top_k_cut_hidden_input(V, top_k, seed):
    """The same exact-tie check through the LM-head product, whose workgroups keep their
    own top_k per row: one-hot hidden states pick an integer-valued column of W, so the
    logits are those integers exactly and many tie at the cut, within and across the
    workgroups' shares of the vocabulary.  n must equal the oracle's exactly."""
    B, gamma, T, d = 4, 4, 4.0, 32
    G1 = gamma + 1
    rng = np.random.default_rng(1000 + seed)
    cols = np.floor(rng.standard_normal((V, d)) * 3.0).astype(np.float32)     # bf16-exact integers
    h = np.zeros((B, G1, d), dtype=np.float32)
    for b in range(B):
        for i in range(G1):
            h[b, i, (b * G1 + i + seed) % d] = 1.0
    l32 = np.einsum("bgd,vd->bgv", h, cols).astype(np.float32)                 # exact: one nonzero term
    draft = np.empty((B, gamma), dtype=np.int32)
    for b in range(B):
        for i in range(gamma):
            row = l32[b, i].astype(np.float64)
            order = np.lexsort((np.arange(V), -row))
            cut = row[order[top_k - 1]]
            tied = np.nonzero(row == cut)[0]
            draft[b, i] = tied[rng.integers(len(tied))]
    q = np.full((B, gamma, V), 1e-7, dtype=np.float32)
    pos0 = rng.integers(0, 1000, B).astype(np.int64)
    model = sv.lm_head_model(dev_bf16(workloads.to_bf16_bits(cols)))
    logits = torch.empty((B, G1, V), dtype=torch.float32, device="cuda")
    n, tok = sv.spec_verify_sample_filtered(model, sv.SV_IN_HIDDEN, dev_bf16(workloads.to_bf16_bits(h)), B, gamma,
                                            dev(draft), dev(q), T, top_k, 1.0, 99, dev(pos0), logits_out=logits)
    torch.cuda.synchronize()
    assert np.array_equal(logits.cpu().numpy(), l32)
    n, tok = n.cpu().numpy(), tok.cpu().numpy()
    n0, t0, _ = rules.sample_rule_filtered(l32, draft, q.astype(np.float64), T, top_k, 1.0, 99, pos0)
    assert n.tolist() == n0.tolist()
    _, kept, _ = rules.filtered_probs(l32, T, top_k, 1.0)
    for b in range(B):
        assert tok[b, :n[b]].tolist() == draft[b, :n[b]].tolist()
        assert kept[b, n[b], tok[b, n[b]]]
    log(f"[filtered ties, hidden input] V={V} top_k={top_k} accepted drafts {int(n.sum())} of {B * gamma}")
