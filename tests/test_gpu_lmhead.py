"""GPU parity of the LM-head verify path (logits / hidden-state inputs) against
the CPU oracle, through the C ABI.

Configurations: tiny fp32 reference (V=1024, d=64, 1000 rounds), acceptance
statistics (V=32, 1e6 rounds), large vocabulary (V=262144, d=1536, B in
{1,2,4,8}, T in {0, 0.7, 1}), plus ragged and degenerate shapes.  The batch/
gamma sweep at d=4096 is in test_gpu_sweep.py.

Bar: n_accepted and tokens bit-exact except on sequences the oracle flags (a
decision margin below 1e-3); logits within 1e-5 (fp32 inputs) / 1e-4 (bf16
inputs, tighter than the 2e-2 stated for the method) of the row's max |logit|.
"""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import closed_form, rules
from tests.gpu_util import (check_token_structure, compare_decisions, dev, dev_bf16, log, oracle_logits_bf16,
                            row_rel_err)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# configuration 1: tiny fp32 reference, 1000 rounds

@pytest.mark.parametrize("T", [0.0, 1.0])
def test_config1_tiny_ref_rounds(T):
    log(f"[config1] T={T}")
    w, rounds = workloads.tiny_ref(rounds=1000, temperature=T)
    model = sv.lm_head_model(dev(w))
    seed = workloads.philox_seed(1)
    pos = 0
    mism = flagged_total = 0
    worst = 0.0
    emitted = []
    for r, (h, draft, q) in enumerate(rounds):
        ref64 = rules.lm_head_logits(h.astype(np.float64), w.astype(np.float64))
        if T == 0.0:
            n0, t0, fl = rules.verify_greedy(ref64, draft)
        else:
            n0, t0, fl = rules.verify_sample(ref64, draft, q, T, seed, np.array([pos]))
        logits = torch.empty((1, 5, 1024), dtype=torch.float32, device="cuda")
        hd, dd = dev(h), dev(draft.astype(np.int32))
        if T == 0.0:
            n, tok = sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, hd, 1, 4, dd, logits_out=logits)
        else:
            n, tok = sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, hd, 1, 4, dd, dev(q), T, seed,
                                           dev(np.array([pos], np.int64)), logits_out=logits)
        torch.cuda.synchronize()
        worst = max(worst, float(row_rel_err(logits.cpu().numpy(), ref64).max()))
        m, f = compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"round {r}")
        mism += m
        flagged_total += f
        emitted.append(int(n0[0]) + 1)
        pos += int(n0[0]) + 1          # the oracle's trajectory drives both sides
    log(f"[config1] T={T} worst logit rel err {worst:.2e} mismatched {mism} flagged {flagged_total} "
        f"mean emitted {np.mean(emitted):.3f}")
    assert worst <= 1e-5
    assert mism <= flagged_total


# ---------------------------------------------------------------------------
# configuration 2: acceptance statistics, 1e6 rounds in one call

def test_config2_acceptance_statistics():
    R = 1_000_000
    log("[config2] generating")
    c = workloads.acceptance_stats(rounds=R)
    gamma, V = 4, 32
    logits = np.broadcast_to(c.logits, (R, gamma + 1, V))
    q = np.broadcast_to(c.q, (R, gamma, V))
    model = sv.logits_model(V)
    log("[config2] GPU call")
    n, tok = sv.spec_verify_sample(model, sv.SV_IN_LOGITS, dev(logits), R, gamma, dev(c.draft), dev(q), 1.0, c.seed,
                                   torch.zeros(R, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    n = n.cpu().numpy().astype(np.int64)
    tok = tok.cpu().numpy().astype(np.int64)
    check_token_structure(n[:1000], tok[:1000], gamma)
    log("[config2] oracle")
    mism = nflag = 0
    chunk = 100_000
    for c0 in range(0, R, chunk):
        B = min(chunk, R - c0)
        n0, t0, fl = rules.sample_rule(logits[c0:c0 + B], c.draft[c0:c0 + B].astype(np.int64), q[c0:c0 + B], 1.0,
                                       c.seed, np.zeros(B, np.int64), seq0=c0)
        m, f = compare_decisions(n[c0:c0 + B], tok[c0:c0 + B], n0, t0, fl, f"rounds {c0}+")
        mism += m
        nflag += f
    log(f"[config2] mismatched {mism} flagged {nflag} of {R}")
    # statistics of the GPU's own output
    p32 = rules.target_probs(c.logits, 1.0).astype(np.float64)
    alphas = rules.acceptance_rate(p32[:gamma], c.q)
    assert np.allclose(alphas, 0.8, atol=1e-5)
    law = closed_form.emitted_law_per_slot(alphas)
    mean = closed_form.expected_emitted_per_slot(alphas)
    emitted = n + 1
    var = float(((np.arange(1, gamma + 2) - mean) ** 2 * law).sum())
    se = np.sqrt(var / R)
    log(f"[config2] mean emitted {emitted.mean():.5f} expected {mean:.5f} (closed form 3.3616) se {se:.5f}")
    assert abs(emitted.mean() - mean) < 5 * se
    assert abs(closed_form.expected_emitted(0.8, 4) - 3.3616) < 1e-12
    cnt = np.bincount(emitted, minlength=gamma + 2)[1:]
    chi2 = ((cnt - law * R) ** 2 / (law * R)).sum()
    assert chi2 < 25
    for k in range(gamma + 1):
        sel = n >= k
        counts = np.bincount(tok[sel, k], minlength=V).astype(float)
        e = p32[k] * sel.sum()
        keep = e >= 5
        chi = ((counts[keep] - e[keep]) ** 2 / e[keep]).sum()
        dof = int(keep.sum()) - 1
        log(f"[config2] slot {k}: reached {int(sel.sum())} chi2 {chi:.1f} dof {dof}")
        assert chi < dof + 6 * np.sqrt(2 * dof) + 10


# ---------------------------------------------------------------------------
# configuration 3: V = 262144, d = 1536

C3_CASES = [(B, T) for B in (1, 2, 4, 8) for T in (0.0, 0.7, 1.0)]


@pytest.fixture(scope="module")
def config3():
    log("[config3] generating inputs")
    w = None
    cases = {}
    for B, T in C3_CASES:
        cs = workloads.large_vocab(B=B, temperature=T, w=w)
        w = cs.w
        cases[(B, T)] = cs
    log("[config3] oracle logits")
    hs = np.concatenate([cases[k].h.reshape(-1, 1536) for k in C3_CASES])
    ref = oracle_logits_bf16(hs, w)
    refs, o = {}, 0
    for k in C3_CASES:
        M = cases[k].h.shape[0] * 5
        refs[k] = ref[o:o + M].reshape(cases[k].B, 5, -1)
        o += M
    wd = dev_bf16(w)
    return cases, refs, sv.lm_head_model(wd)


def run_case(model, cs, logits_out=None):
    hd = dev_bf16(cs.h)
    dd = dev(cs.draft.astype(np.int32))
    if cs.temperature == 0.0:
        return sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, hd, cs.B, cs.gamma, dd, logits_out=logits_out)
    return sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, hd, cs.B, cs.gamma, dd, dev_bf16(cs.q), cs.temperature,
                                 cs.seed, dev(cs.pos0), logits_out=logits_out)


def oracle_case(cs, ref64):
    if cs.temperature == 0.0:
        return rules.verify_greedy(ref64, cs.draft)
    qf = (cs.q.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return rules.verify_sample(ref64, cs.draft, qf, cs.temperature, cs.seed, cs.pos0)


@pytest.mark.parametrize("B,T", C3_CASES)
def test_config3_large_vocab(config3, B, T):
    cases, refs, model = config3
    cs, ref = cases[(B, T)], refs[(B, T)]
    log(f"[config3] B={B} T={T}")
    logits = torch.empty((B, 5, cs.V), dtype=torch.float32, device="cuda")
    n, tok = run_case(model, cs, logits)
    torch.cuda.synchronize()
    err = row_rel_err(logits.cpu().numpy(), ref).max()
    n0, t0, fl = oracle_case(cs, ref)
    m, f = compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"B={B} T={T}")
    log(f"[config3] B={B} T={T} logit rel err {err:.2e} n={n.cpu().numpy().tolist()} mismatched {m} flagged {f}")
    assert err <= 1e-4
    # run twice: identical bits (no races)
    n2, tok2 = run_case(model, cs)
    torch.cuda.synchronize()
    assert torch.equal(n, n2) and torch.equal(tok, tok2)


def test_config3_logits_input_path(config3):
    """The same decisions from SV_IN_LOGITS (row statistics over 262144 entries
    computed by the logits-input kernel)."""
    cases, refs, _ = config3
    cs, ref = cases[(8, 1.0)], refs[(8, 1.0)]
    l32 = rules.f32_logits(ref)
    qf = (cs.q.astype(np.uint32) << np.uint32(16)).view(np.float32)
    n, tok = sv.spec_verify_sample(sv.logits_model(cs.V), sv.SV_IN_LOGITS, dev(l32), cs.B, 4,
                                   dev(cs.draft.astype(np.int32)), dev(qf), 1.0, cs.seed, dev(cs.pos0))
    torch.cuda.synchronize()
    n0, t0, fl = rules.sample_rule(l32, cs.draft, qf.astype(np.float64), 1.0, cs.seed, cs.pos0)
    compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, "logits input")
    ng, tg = sv.spec_verify_greedy(sv.logits_model(cs.V), sv.SV_IN_LOGITS, dev(l32), cs.B, 4,
                                   dev(cs.draft.astype(np.int32)))
    torch.cuda.synchronize()
    n1, t1, f1 = rules.greedy_rule(l32, cs.draft)
    compare_decisions(ng.cpu().numpy(), tg.cpu().numpy(), n1, t1, f1, "logits input greedy")


# ---------------------------------------------------------------------------
# ragged / degenerate shapes (small, fast)

SMALL = [
    # (V, d, B, gamma, T)
    (1000, 96, 3, 4, 1.0),      # V not a multiple of 16, d not a multiple of 256
    (4099, 64, 20, 4, 0.7),     # M = 100: two row groups of the product
    (2000, 1024, 16, 3, 1.0),   # M = 64, K chunked through LDS
    (2000, 2048, 13, 4, 1.0),   # M = 65, K chunked, two row groups
    (2, 32, 5, 1, 1.0),         # smallest vocabulary and gamma
    (517, 256, 2, 15, 1.0),     # largest gamma
    (1000, 96, 3, 4, 0.0),      # greedy on ragged shapes
    (4099, 64, 20, 15, 0.0),
    # K % 256 == 0 with X resident in LDS: the streaming product, 1-4 row blocks
    (4096, 256, 2, 8, 0.0),     # M = 18
    (4096, 256, 4, 4, 1.0),     # M = 20
    (4099, 256, 3, 10, 0.0),    # M = 33
    (4096, 1536, 8, 4, 0.0),    # M = 40
    (4096, 1536, 8, 4, 0.7),
    (4096, 256, 4, 15, 0.0),    # M = 64
    # k-split product with split factor 4 (K % 512 == 0 or K = 1536), 1-5 column blocks
    (777, 1024, 1, 1, 1.0),     # M = 2
    (3001, 512, 1, 4, 1.0),     # M = 5: two blocks
    (4099, 512, 3, 3, 0.7),     # M = 12: three blocks
    (1000, 1024, 4, 3, 0.0),    # M = 16: four blocks, greedy
    (2503, 512, 4, 4, 1.0),     # M = 20: five blocks
    (2503, 1536, 2, 4, 1.0),    # M = 10, the large-vocabulary hidden size
    # K not a whole number of work items: the last item of each tile runs over zeros
    (1500, 640, 1, 4, 1.0),     # 5 steps of 128: items of 4, tail of 1
    (2001, 1408, 2, 4, 0.0),    # 11 steps: tail of 3, greedy
    (3000, 192, 1, 2, 1.0),     # split factor 2, 3 steps in one item of 4
    (999, 2304, 1, 4, 0.7),     # 18 steps: items of 6, no tail
]


def small_case(V, d, B, gamma, T, seed):
    rng = np.random.default_rng(seed)
    w = workloads.to_bf16_bits((rng.standard_normal((V, d)) * 0.3).astype(np.float32))
    h = workloads.to_bf16_bits(rng.standard_normal((B, gamma + 1, d)).astype(np.float32))
    lt = rules.f32_logits(oracle_logits_bf16(h[:, :gamma], w))
    noise = rng.standard_normal((B, gamma, V)).astype(np.float32) * 0.7
    draft, q = workloads.drafter(lt, noise, T, rng)
    # some out-of-range drafts
    bad = rng.random((B, gamma)) < 0.05
    draft = np.where(bad, np.where(rng.random((B, gamma)) < 0.5, -3, V + 7), draft).astype(np.int32)
    qb = None if q is None else workloads.to_bf16_bits(q)
    return workloads.LMHeadCase(w=w, h=h, draft=draft, q=qb, temperature=T, seed=12345 + seed,
                                pos0=rng.integers(0, 5000, B).astype(np.int64), dtype="bf16")


@pytest.mark.parametrize("V,d,B,gamma,T", SMALL)
def test_small_and_ragged_shapes(V, d, B, gamma, T):
    log(f"[small] V={V} d={d} B={B} gamma={gamma} T={T}")
    cs = small_case(V, d, B, gamma, T, seed=V + d + B + gamma)
    ref = oracle_logits_bf16(cs.h, cs.w)
    model = sv.lm_head_model(dev_bf16(cs.w))
    logits = torch.empty((B, gamma + 1, V), dtype=torch.float32, device="cuda")
    n, tok = run_case(model, cs, logits)
    torch.cuda.synchronize()
    assert row_rel_err(logits.cpu().numpy(), ref).max() <= 1e-4
    n0, t0, fl = oracle_case(cs, ref)
    compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"V={V} d={d} B={B} g={gamma}")
    # verify_forward gives the same logits bit for bit
    lf = sv.verify_forward(model, sv.SV_IN_HIDDEN, dev_bf16(cs.h), B, gamma)
    torch.cuda.synchronize()
    assert torch.equal(lf, logits)


def test_fp32_head_ragged():
    rng = np.random.default_rng(3)
    V, d, B, g = 777, 48, 2, 4
    w = (rng.standard_normal((V, d)) / 7).astype(np.float32)
    h = rng.standard_normal((B, g + 1, d)).astype(np.float32)
    ref = rules.lm_head_logits(h.astype(np.float64), w.astype(np.float64))
    draft = np.argmax(ref[:, :g], axis=-1).astype(np.int32)
    draft[1, 2] = (draft[1, 2] + 1) % V
    n, tok = sv.spec_verify_greedy(sv.lm_head_model(dev(w)), sv.SV_IN_HIDDEN, dev(h), B, g, dev(draft))
    torch.cuda.synchronize()
    n0, t0, fl = rules.verify_greedy(ref, draft)
    compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, "fp32 ragged")
    assert n.cpu().numpy().tolist() == [4, 2]


def test_fused_sampler_wait_timeout():
    """The fused sampler's waits are bounded.  With the bound forced to zero from the
    host (sv_set_option), workgroups give up before the others have published: the step
    must mark every sequence invalid (n = -1, tokens -1) instead of drawing from partial
    data, and the next step on the same workspace, with the default bound, must match
    the oracle without the workspace being zero-filled (the step advanced the epoch past
    the records it left), over several epochs."""
    V, d, B, gamma, T = 65536, 512, 2, 4, 1.0
    cs = small_case(V, d, B, gamma, T, seed=99)
    ref = oracle_logits_bf16(cs.h, cs.w)
    model = sv.lm_head_model(dev_bf16(cs.w))
    ws = sv.Workspace()
    args = (model, sv.SV_IN_HIDDEN, dev_bf16(cs.h), B, gamma, dev(cs.draft.astype(np.int32)), dev_bf16(cs.q), T,
            cs.seed, dev(cs.pos0))
    n0, t0, fl = oracle_case(cs, ref)
    for rnd in range(2):
        sv.set_option(sv.SV_OPT_WAIT_LIMIT, 0)
        try:
            n, tok = sv.spec_verify_sample(*args, ws=ws)
            torch.cuda.synchronize()
        finally:
            sv.set_option(sv.SV_OPT_WAIT_LIMIT, -1)
        log(f"[timeout] round {rnd}: n={n.cpu().numpy().tolist()}")
        assert (n.cpu().numpy() == -1).all() and (tok.cpu().numpy() == -1).all()
        for _ in range(3):                           # recovered, and stays right over several epochs
            n, tok = sv.spec_verify_sample(*args, ws=ws)
            torch.cuda.synchronize()
            compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"after timeout {rnd}")


def test_tuning_keeps_every_bit():
    """sv_tune_verify picks the fused step's item size for this device; logits, accepted
    counts and tokens are the same bits before and after (the item size groups the
    loads, it does not reorder the sums)."""
    cs = workloads.large_vocab(B=1, temperature=1.0)
    model = sv.lm_head_model(dev_bf16(cs.w))
    h, d, q, p0 = dev_bf16(cs.h), dev(cs.draft.astype(np.int32)), dev_bf16(cs.q), dev(cs.pos0)

    def run():
        lg = torch.empty((1, 5, 262144), dtype=torch.float32, device="cuda")
        n, tok = sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, h, 1, 4, d, q, 1.0, cs.seed, p0, logits_out=lg)
        ng, tg = sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, h, 1, 4, d)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in (n, tok, lg, ng, tg)]

    before = run()
    item = sv.tune_verify(model, 1, 4)
    log(f"[tune] V=262144 d=1536 M=5: item size {item}")
    assert item in (4, 6, 8)
    after = run()
    for a, b in zip(before, after):
        assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                              b.view(np.uint32) if b.dtype == np.float32 else b)
    assert sv.tune_verify(model, 1, 4) in (4, 6, 8)
