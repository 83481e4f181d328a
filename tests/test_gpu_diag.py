"""GPU parity of the optional per-slot margins (diag) of spec_verify_greedy and
spec_verify_sample against oracle/rules.verify_diag, element by element: the same slots
defined (NaN past the decision), the greedy top-two gaps within twice the row's logit
error, the acceptance margins |u - p/q| within a relative 1e-4 (p is float32 on both
sides, the oracle's rounded once from float64), the final draw's score gap within 1e-3
(float32 logarithms of the same float32 residual on both sides).  Paths: the fused
large-vocabulary step (B = 1, 4), the unfused large-batch step (M = 40) and logits input,
with out-of-range drafts; a call without diag is unchanged."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import rules
from tests.gpu_util import dev, dev_bf16, log, oracle_logits_bf16, row_rel_err

pytestmark = pytest.mark.gpu


def check_diag(d_gpu, d_ref, n_gpu, n_ref, T, logit_err, label):
    d_gpu = np.asarray(d_gpu, dtype=np.float64)
    same_n = np.asarray(n_gpu) == np.asarray(n_ref)
    assert same_n.mean() > 0.5, label
    g, r = d_gpu[same_n], d_ref[same_n]
    assert np.array_equal(np.isnan(g), np.isnan(r)), f"{label}: defined slots differ"
    assert np.array_equal(np.isinf(g), np.isinf(r)), f"{label}: infinite entries differ"
    fin = np.isfinite(r)
    if T == 0.0:
        tol = 2 * np.broadcast_to(np.asarray(logit_err)[same_n][:, None], r.shape)[fin] + 1e-6
        err = np.abs(g[fin] - r[fin])
    else:
        gamma = r.shape[1] - 1
        acc = np.zeros_like(r, dtype=bool)
        acc[:, :gamma] = True
        tol = np.where(acc, 1e-4 * (1.0 + np.abs(r)), 1e-3)[fin]
        err = np.abs(g[fin] - r[fin])
    bad = err > tol
    assert not bad.any(), f"{label}: {int(bad.sum())} margins off, worst {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


def run_hidden(model, cs, ws=None, with_diag=True):
    B, G1 = cs.h.shape[0], cs.h.shape[1]
    logits = torch.empty((B, G1, cs.w.shape[0]), dtype=torch.float32, device="cuda")
    diag = torch.full((B, G1), 123.0, dtype=torch.float32, device="cuda") if with_diag else None
    if cs.temperature == 0.0:
        n, tok = sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, dev_bf16(cs.h), B, G1 - 1, dev(cs.draft.astype(np.int32)),
                                       logits_out=logits, ws=ws, diag=diag)
    else:
        n, tok = sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, dev_bf16(cs.h), B, G1 - 1,
                                       dev(cs.draft.astype(np.int32)), dev_bf16(cs.q), cs.temperature, cs.seed,
                                       dev(cs.pos0), logits_out=logits, ws=ws, diag=diag)
    torch.cuda.synchronize()
    return n.cpu().numpy(), tok.cpu().numpy(), logits.cpu().numpy(), None if diag is None else diag.cpu().numpy()


def oracle(cs, ref):
    qf = None if cs.q is None else (cs.q.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    n, tok, fl = rules.verify_sample(ref, cs.draft, qf, cs.temperature, cs.seed, cs.pos0)
    return n, tok, rules.verify_diag(ref, cs.draft, qf, cs.temperature, cs.seed, cs.pos0, n)


@pytest.fixture(scope="module")
def table():
    return workloads.lm_head_case(262144, 1536, 1, 4, 1.0, 1.0, 3).w


@pytest.mark.parametrize("B,T", [(1, 1.0), (4, 1.0), (1, 0.0), (4, 0.0)])
def test_diag_large_vocab(table, B, T):
    cs = workloads.lm_head_case(262144, 1536, B, 4, T, 1.0, 3, w=table, pos0=40, variant=B + 3)
    ref = oracle_logits_bf16(cs.h, cs.w)
    model = sv.lm_head_model(dev_bf16(cs.w))
    n, tok, logits, d = run_hidden(model, cs)
    n0, t0, d0 = oracle(cs, ref)
    lerr = np.abs(logits.astype(np.float64) - ref).max(axis=(1, 2))
    worst = check_diag(d, d0, n, n0, T, lerr, f"B={B} T={T}")
    log(f"[diag] V=262144 B={B} T={T} n={n.tolist()} diag={np.array2string(d, precision=4)} worst {worst:.2e}")
    # the same step without diag returns the same decisions
    n2, tok2, _, _ = run_hidden(model, cs, with_diag=False)
    assert np.array_equal(n, n2) and np.array_equal(tok, tok2)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_diag_unfused_batch_and_bad_drafts(T):
    """M = 8 x 5 = 40 rows: the two-launch step; 5 % of the drafts out of range."""
    rng = np.random.default_rng(21)
    V, d, B, gamma = 20011, 256, 8, 4
    w = workloads.to_bf16_bits((rng.standard_normal((V, d)) * 0.3).astype(np.float32))
    h = workloads.to_bf16_bits(rng.standard_normal((B, gamma + 1, d)).astype(np.float32))
    lt = rules.f32_logits(oracle_logits_bf16(h[:, :gamma], w))
    draft, q = workloads.drafter(lt, rng.standard_normal((B, gamma, V)).astype(np.float32) * 0.7, T, rng)
    bad = rng.random((B, gamma)) < 0.05
    draft = np.where(bad, V + 3, draft).astype(np.int32)
    cs = workloads.LMHeadCase(w=w, h=h, draft=draft, q=None if q is None else workloads.to_bf16_bits(q),
                              temperature=T, seed=991, pos0=rng.integers(0, 999, B).astype(np.int64), dtype="bf16")
    ref = oracle_logits_bf16(h, w)
    n, tok, logits, dg = run_hidden(sv.lm_head_model(dev_bf16(w)), cs)
    n0, t0, d0 = oracle(cs, ref)
    lerr = np.abs(logits.astype(np.float64) - ref).max(axis=(1, 2))
    worst = check_diag(dg, d0, n, n0, T, lerr, f"unfused T={T}")
    log(f"[diag] unfused B={B} T={T} n={n.tolist()} worst {worst:.2e}")


def test_diag_logits_input():
    """SV_IN_LOGITS: the margins from the caller's logits (exactly the oracle's float32)."""
    rng = np.random.default_rng(4)
    B, gamma, V = 3, 3, 5000
    l32 = (rng.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    q = rng.dirichlet(np.ones(V) * 0.3, size=(B, gamma)).astype(np.float32)
    draft = np.array([[rng.choice(V, p=q[b, i] / q[b, i].sum()) for i in range(gamma)] for b in range(B)],
                     dtype=np.int32)
    pos0 = np.array([5, 50, 500], dtype=np.int64)
    model = sv.logits_model(V)
    for T in (1.0, 0.0):
        diag = torch.empty((B, gamma + 1), dtype=torch.float32, device="cuda")
        if T == 0.0:
            n, _ = sv.spec_verify_greedy(model, sv.SV_IN_LOGITS, dev(l32), B, gamma, dev(draft), diag=diag)
        else:
            n, _ = sv.spec_verify_sample(model, sv.SV_IN_LOGITS, dev(l32), B, gamma, dev(draft), dev(q), T, 17,
                                         dev(pos0), diag=diag)
        torch.cuda.synchronize()
        n0, _, _ = rules.verify_sample(l32.astype(np.float64), draft, q.astype(np.float64), T, 17, pos0)
        d0 = rules.verify_diag(l32.astype(np.float64), draft, q.astype(np.float64), T, 17, pos0, n0)
        check_diag(diag.cpu().numpy(), d0, n.cpu().numpy(), n0, T, np.zeros(B), f"logits T={T}")
