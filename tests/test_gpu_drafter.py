"""GPU parity of mtp_draft (the MTP drafter's gamma steps) against the oracle's
drafter.draft: drafts bit-exact step by step until the first step the oracle flags
(a draw or a cluster cut within its rounding margin; every later step of that sequence
depends on it), q within a tolerance derived from the bf16 rounding of the hidden state,
exact zeros outside the scored tokens, -1 drafts for invalid rows."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import drafter as od
from tests.gpu_util import dev, dev_bf16, log

pytestmark = pytest.mark.gpu

# The drafter's hidden state passes through the target decoder's bf16 rounding points
# and is fed back at every step, so its drift from the float64 oracle compounds with the
# depth traversed.  A float32 evaluation of the same recipe on the CPU at the full shapes
# (D = 1536, H = 256, four layers, 700-2048 cached positions, masked head; 12 rows)
# drifts in the logits by up to 3.4e-2, 5.2e-2, 7.0e-2 at steps 0, 1, 2 (about 1 % of
# the row maximum; by step 2 about 1100 of the 1536 hidden entries round to another
# bf16 value) and in q by up to 1.6e-2, 3.7e-2, 3.4e-2.  Decisions closer than MARGIN
# (a score difference moves by up to two logit errors) are flagged, and q is held to
# Q_TOL, both times the square root of the depth, (k + 1) * layers / 4.
MARGIN = 8e-2
Q_TOL = 4e-2      # max |q_gpu - q_oracle| / max q_oracle per row, at four layers deep


def depth_scale(k, n_layers):
    return max(1.0, np.sqrt((k + 1) * n_layers / 4.0))


def oracle_weights(c, masked):
    return od.DrafterWeights(d_model=c.d_model, hidden=c.hidden, n_heads=c.n_heads, head_dim=c.head_dim,
                             d_ff=c.d_ff, vocab=c.vocab, rms_eps=1e-5, rope_theta=10000.0, embed=c.embed,
                             pre_proj=c.pre_proj, layers=c.layers, final_norm=c.final_norm, post_proj=c.post_proj,
                             centroids=c.centroids if masked else None, top_k_clusters=c.top_k)


def device_drafter(c, masked, embed_dev=None):
    emb = embed_dev if embed_dev is not None else dev_bf16(c.embed)
    layers = [{k: dev_bf16(L[k]) for k in sv.DRAFTER_LAYER_KEYS} for L in c.layers]
    dr = sv.drafter(emb, dev_bf16(c.pre_proj), layers, dev_bf16(c.final_norm), dev_bf16(c.post_proj), c.n_heads,
                    c.head_dim, centroids=dev_bf16(c.centroids) if masked else None, top_k_clusters=c.top_k)
    kvk = {}
    ks = [kvk.setdefault(id(a), dev_bf16(a)) for a in c.kv_k]
    vs = [kvk.setdefault(id(a), dev_bf16(a)) for a in c.kv_v]
    return dr, sv.shared_kv(ks, vs, dev(c.length.astype(np.int32)))


def compare(c, out, gd, gq, label):
    """Step by step per sequence: the draft must match the oracle's, and (T > 0) the
    support of q (the kept clusters) too, with q within the depth-scaled Q_TOL.  A
    mismatch is allowed only at a step the oracle flags: another draft ends the
    comparison of that sequence (its later steps start from another token), another
    kept cluster set skips that step's q.  Returns (steps compared, sequences that
    diverged at a flagged step)."""
    B, gamma = out["draft"].shape
    steps, diverged = 0, 0
    for b in range(B):
        for k in range(gamma):
            if gd[b, k] != out["draft"][b, k]:
                assert out["flags"][b, k], (f"{label}: b={b} step {k}: gpu draft {gd[b, k]} oracle "
                                            f"{out['draft'][b, k]} (unflagged)")
                diverged += 1
                break
            steps += 1
            if out["q"] is None:
                continue
            qo, qg = out["q"][b, k].astype(np.float64), gq[b, k].astype(np.float64)
            if not np.array_equal(qo > 0, qg > 0):       # another kept cluster set: the cut must be flagged
                assert out["flags"][b, k], f"{label}: b={b} step {k}: kept clusters differ (unflagged)"
                continue
            if qo.max() > 0:
                err = np.abs(qg - qo).max() / qo.max()
                assert err <= Q_TOL * depth_scale(k, len(c.layers)), f"{label}: b={b} step {k} q err {err:.2e}"
    return steps, diverged


def run(c, masked, gamma, T, q_dtype=torch.float32, seed=None):
    dr, kv = device_drafter(c, masked)
    seed = c.seed if seed is None else seed
    gd, gq = sv.mtp_draft(dr, kv, dev(c.last_token.astype(np.int32)), dev_bf16(c.h_target), gamma, T, seed,
                          q_dtype=q_dtype)
    torch.cuda.synchronize()
    gd = gd.cpu().numpy()
    gq = None if gq is None else gq.float().cpu().numpy()
    out = od.draft(oracle_weights(c, masked), od.SharedKV(k=c.kv_k, v=c.kv_v, length=c.length), c.last_token,
                   c.h_target, gamma, T, seed, margin=[MARGIN * depth_scale(k, len(c.layers)) for k in range(gamma)])
    if q_dtype == torch.bfloat16 and out["q"] is not None:
        out["q"] = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(out["q"]))
    return gd, gq, out


SMALL = [
    # (V, D, H, layers, heads, head_dim, d_ff, C, top_k, B, lengths, gamma, T, masked)
    (4096, 256, 128, 2, 2, 64, 256, 64, 8, 3, [5, 40, 300], 3, 1.0, True),
    (4096, 256, 128, 2, 2, 64, 256, 64, 8, 3, [5, 40, 300], 3, 0.0, True),
    (4096, 256, 128, 2, 2, 64, 256, 64, 8, 3, [1, 257, 513], 2, 0.7, False),   # tied head, split edges
    (8192, 512, 256, 4, 4, 128, 512, 128, 32, 2, [100, 1000], 4, 1.0, True),
    (2048, 256, 64, 1, 1, 128, 128, 16, 16, 4, [3, 9, 27, 81], 5, 1.3, True),  # every cluster kept
    (4096, 256, 128, 2, 2, 64, 256, 64, 64, 1, [700], 15, 1.0, True),          # largest gamma, top_k 64
]


@pytest.mark.parametrize("V,D,H,nl,nh,hd,ff,C,tk,B,lens,gamma,T,masked", SMALL)
def test_small_and_ragged(V, D, H, nl, nh, hd, ff, C, tk, B, lens, gamma, T, masked):
    log(f"[drafter] V={V} D={D} H={H} layers={nl} heads={nh}x{hd} C={C} top_k={tk} B={B} lens={lens} "
        f"gamma={gamma} T={T} masked={masked}")
    c = workloads.drafter_case(V=V, D=D, H=H, n_layers=nl, n_heads=nh, head_dim=hd, d_ff=ff, C=C, top_k=tk, B=B,
                               length=lens, shared_layers=tuple(min(l, 1) for l in range(nl)), variant=V + B)
    gd, gq, out = run(c, masked, gamma, T)
    steps, div = compare(c, out, gd, gq, f"V={V} B={B}")
    assert np.all((gd >= 0) & (gd < V))
    if gq is not None:
        np.testing.assert_allclose(gq.sum(-1), 1.0, atol=1e-4)
    log(f"[drafter] drafts {gd.tolist()}: {steps} of {B * gamma} steps compared, {div} diverged at a flagged step")


def test_invalid_rows_and_bf16_q():
    c = workloads.drafter_case(V=4096, D=256, H=128, n_layers=2, n_heads=2, head_dim=64, d_ff=256, C=64, top_k=8,
                               B=4, length=[0, 40, 300, 60], max_len=320, shared_layers=(0, 1), variant=5)
    c.length[3] = 321                            # beyond max_len
    c.last_token[2] = c.vocab + 3                # no token
    gd, gq, out = run(c, True, 3, 1.0, q_dtype=torch.bfloat16)
    assert np.all(gd[[0, 2, 3]] == -1) and np.all(gq[[0, 2, 3]] == 0)
    compare(c, out, gd, gq, "invalid rows")


@pytest.fixture(scope="module")
def full_case():
    log("[drafter full] generating the E2B-shaped drafter and its 262144-token table")
    return workloads.drafter_case(B=4, length=[2048, 1500, 700, 2040], max_len=2048, variant=1)


@pytest.mark.parametrize("B,T,qdt", [(1, 1.0, torch.float32), (4, 1.0, torch.bfloat16), (4, 0.0, None)])
def test_full_size(full_case, B, T, qdt):
    """V = 262144, D = 1536, H = 256, four layers of 4 x 128 query heads over 2048 cached
    positions, 2048 clusters with 32 kept, gamma = 4."""
    c = full_case
    if B < c.last_token.shape[0]:
        c = workloads.DrafterCase(**{**c.__dict__, "length": c.length[:B], "last_token": c.last_token[:B],
                                     "h_target": c.h_target[:B], "kv_k": [a[:B] for a in c.kv_k],
                                     "kv_v": [a[:B] for a in c.kv_v]})
    log(f"[drafter full] B={B} T={T}")
    gd, gq, out = run(c, True, 4, T, q_dtype=qdt or torch.float32)
    steps, div = compare(c, out, gd, gq, f"full B={B} T={T}")
    log(f"[drafter full] B={B} T={T} drafts {gd.tolist()}: {steps} of {B * 4} steps compared, {div} diverged")
    assert steps >= B * 2
