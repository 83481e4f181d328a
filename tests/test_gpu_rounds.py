"""GPU parity of the round policies against oracle/rounds.py (index work: bit-exact),
and of a padded verify batch against per-sequence verification (same kernels, same
logits: bit-exact; and against the oracle with its flags)."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import rounds, rules
from tests.gpu_util import compare_decisions, dev, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("qdt,tau", [(torch.float32, 0.0), (torch.float32, 0.05), (torch.bfloat16, 0.02), (None, 0.0)])
def test_pad_and_confidence_cut(qdt, tau):
    log(f"[rounds] pad q={qdt} tau={tau}")
    rng = np.random.default_rng(4)
    B, G, V = 7, 6, 5000
    gamma_b = np.array([1, 2, 6, 4, 0, 9, 3], dtype=np.int32)      # 0 and 9 are clamped to [1, G]
    draft = rng.integers(0, V, (B, G)).astype(np.int32)
    q = None
    if qdt is not None:
        z = rng.standard_normal((B, G, V)) * rng.uniform(0.5, 6.0, (B, G, 1))
        q = np.exp(z - z.max(-1, keepdims=True))
        q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
        if qdt == torch.bfloat16:
            q = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(q))
    g_dev = dev(gamma_b.copy())
    d_dev = dev(draft.copy())
    q_dev = None if q is None else torch.from_numpy(q).to(qdt).cuda()
    sv.round_pad_drafts(g_dev, d_dev, q_dev, tau)
    torch.cuda.synchronize()
    g_ref = np.clip(gamma_b, 1, G)
    if tau > 0:
        g_ref = rounds.confidence_gamma(q, g_ref, tau)
    d_ref, q_ref = rounds.pad_drafts(draft, q, g_ref)
    assert g_dev.cpu().numpy().tolist() == g_ref.tolist()
    assert d_dev.cpu().numpy().tolist() == d_ref.tolist()
    if q is not None:
        assert np.array_equal(q_dev.float().cpu().numpy(), q_ref)
    if tau > 0:
        assert set(g_ref.tolist()) != {int(x) for x in np.clip(gamma_b, 1, G)}   # the cut changed something


def test_heuristic_schedule():
    rng = np.random.default_rng(5)
    B = 300
    g = rng.integers(1, 9, B).astype(np.int32)
    n = np.minimum(rng.integers(-1, 9, B), g).astype(np.int32)
    g_dev = dev(g.copy())
    sv.round_update_gamma(dev(n), g_dev, 1, 8)
    torch.cuda.synchronize()
    assert g_dev.cpu().numpy().tolist() == rounds.heuristic_gamma(n, g, 1, 8).tolist()


def test_candidate_selection():
    rng = np.random.default_rng(6)
    B, C, G1 = 257, 4, 6
    n = rng.integers(-1, 5, (B, C)).astype(np.int32)
    tok = rng.integers(0, 1000, (B, C, G1)).astype(np.int32)
    best, nb, tb = sv.round_select_candidates(dev(n), dev(tok))
    torch.cuda.synchronize()
    i0, n0, t0 = rounds.select_candidates(n, tok)
    assert best.cpu().numpy().tolist() == i0.tolist()
    assert nb.cpu().numpy().tolist() == n0.tolist()
    assert tb.cpu().numpy().tolist() == t0.tolist()


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_padded_verify_equals_per_sequence_verify(T):
    """A batch of 6 sequences at gamma_max = 5 with draft lengths 1..5, padded on the
    device, verified in one call (logits input): each sequence's n and tokens equal those
    of verifying it alone with its own draft length, and the oracle's."""
    log(f"[rounds] padded verify T={T}")
    rng = np.random.default_rng(11)
    B, G, V = 6, 5, 3000
    gamma_b = np.array([5, 1, 3, 2, 4, 5], dtype=np.int32)
    logits = rng.standard_normal((B, G + 1, V)) * 2.5
    l32 = rules.f32_logits(logits)
    arg = np.argmax(l32, axis=-1)
    seed = 321
    pos0 = rng.integers(0, 4000, B).astype(np.int64)
    if T == 0.0:
        draft = np.where(rng.random((B, G)) < 0.8, arg[:, :G], (arg[:, :G] + 3) % V).astype(np.int32)
        q = None
    else:
        p = rules.target_probs(l32[:, :G], T).astype(np.float64)
        q = p * np.exp(0.2 * rng.standard_normal(p.shape))
        q = (q / q.sum(-1, keepdims=True)).astype(np.float32)
        draft = np.array([[rng.choice(V, p=q[b, i] / q[b, i].sum()) for i in range(G)] for b in range(B)], np.int32)
    model = sv.logits_model(V)
    g_dev, d_dev = dev(gamma_b.copy()), dev(draft.copy())
    q_dev = None if q is None else dev(q.copy())
    sv.round_pad_drafts(g_dev, d_dev, q_dev)
    if T == 0.0:
        n, tok = sv.spec_verify_greedy(model, sv.SV_IN_LOGITS, dev(l32), B, G, d_dev)
    else:
        n, tok = sv.spec_verify_sample(model, sv.SV_IN_LOGITS, dev(l32), B, G, d_dev, q_dev, T, seed, dev(pos0))
    torch.cuda.synchronize()
    n, tok = n.cpu().numpy(), tok.cpu().numpy()
    for b in range(B):
        g = int(gamma_b[b])
        lb = dev(np.ascontiguousarray(l32[b:b + 1, :g + 1]))
        db = dev(np.ascontiguousarray(draft[b:b + 1, :g]))
        if T == 0.0:
            n1, t1 = sv.spec_verify_greedy(model, sv.SV_IN_LOGITS, lb, 1, g, db)
            r = rules.verify_greedy(logits[b:b + 1, :g + 1], draft[b:b + 1, :g])
        else:
            # sequence id b: the random stream of sequence b in the batch
            big = np.zeros((b + 1, g + 1, V), np.float32)
            big[b] = l32[b, :g + 1]
            dd = np.zeros((b + 1, g), np.int32)
            dd[b] = draft[b, :g]
            qq = np.full((b + 1, g, V), 1.0 / V, np.float32)
            qq[b] = q[b, :g]
            pp = np.zeros(b + 1, np.int64)
            pp[b] = pos0[b]
            n1, t1 = sv.spec_verify_sample(model, sv.SV_IN_LOGITS, dev(big), b + 1, g, dev(dd), dev(qq), T, seed,
                                           dev(pp))
            n1, t1 = n1[b:b + 1], t1[b:b + 1]
            r = rules.verify_sample(logits[b:b + 1, :g + 1], draft[b:b + 1, :g], q[b:b + 1, :g].astype(np.float64),
                                    T, seed, pos0[b:b + 1], seq0=b)
        torch.cuda.synchronize()
        n1, t1 = n1.cpu().numpy(), t1.cpu().numpy()
        assert n[b] == n1[0] and tok[b, :g + 1].tolist() == t1[0].tolist() and np.all(tok[b, g + 1:] == -1), b
        compare_decisions(n[b:b + 1], tok[b:b + 1, :g + 1], r[0], r[1], r[2], f"seq {b}")
    log(f"[rounds] n={n.tolist()} gamma_b={gamma_b.tolist()}")


def test_one_workspace_serves_every_entry_point():
    """Calls that only need scratch (masked head, drafter, padding) share the default
    workspace with the verify calls that keep counters and a launch epoch in it: the
    filtered verify (one-shot tickets) and the fused sampling verify (epoch) still give
    the results of a fresh workspace afterwards."""
    rng = np.random.default_rng(13)
    V, d, B, G = 4096, 256, 2, 4
    w = workloads.to_bf16_bits((rng.standard_normal((V, d)) * 0.3).astype(np.float32))
    h = workloads.to_bf16_bits(rng.standard_normal((B, G + 1, d)).astype(np.float32))
    from tests.gpu_util import dev_bf16
    model = sv.lm_head_model(dev_bf16(w))
    draft = dev(rng.integers(0, V, (B, G)).astype(np.int32))
    qn = rng.random((B, G, V)).astype(np.float32)
    q = dev(qn / qn.sum(-1, keepdims=True))
    pos0 = dev(np.array([5, 9], np.int64))

    def verify_pair(ws):
        a = sv.spec_verify_sample_filtered(model, sv.SV_IN_HIDDEN, dev_bf16(h), B, G, draft, q, 1.0, 64, 0.95, 3,
                                           pos0, ws=ws)
        b = sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, dev_bf16(h), B, G, draft, q, 1.0, 3, pos0, ws=ws)
        torch.cuda.synchronize()
        return [t.cpu().numpy() for t in a + b]

    fresh = verify_pair(sv.Workspace())
    # scratch-only calls on the default workspace, then the verifies on it
    head = sv.masked_head(dev_bf16(w), dev_bf16(w[::64].copy()))
    sv.draft_masked_logits(head, dev_bf16(h[:, 0].copy()), 8)
    gb = dev(np.array([4, 2], np.int32))
    sv.round_pad_drafts(gb, dev(np.zeros((B, G), np.int32)), q.clone(), tau=1e-9)
    shared = verify_pair(None)
    for x, y in zip(fresh, shared):
        assert np.array_equal(x, y)
    assert np.all((shared[0] >= 0) & (shared[0] <= G))
