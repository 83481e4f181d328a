"""GPU parity of mtp_draft (the MTP drafter's gamma steps) against the oracle's
drafter.draft: drafts bit-exact at every step of every sequence except where the oracle
flags the step (a draw or a cluster cut within the derived margin), q within the derived
tolerance, exact zeros outside the scored tokens, -1 drafts for invalid rows.  The oracle
follows the GPU's drafted tokens (teacher forcing), so a flagged divergence does not end
the comparison: every one of the B * gamma steps is compared.

The margin and the q tolerance come from tests/drafter_bounds.py: a float32 evaluation of
the same recipe on the CPU drifts from the float64 oracle by a measured amount per step
(tests/test_drafter_drift_cpu.py recomputes it at the full shapes and checks that these
bounds cover it); they are not fitted to the GPU."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import drafter as od
from tests import drafter_bounds as dbnd
from tests.gpu_util import dev, dev_bf16, log

pytestmark = pytest.mark.gpu


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
    """Every step of every sequence: the draft must be the oracle's unless the oracle
    flags the step (two scores within the margin, or clusters near the cut whose move
    could change the draft).  With T > 0, q must keep the oracle's clusters except for
    clusters of the oracle's band around the cut, and where the kept clusters agree q
    lies within the step's tolerance.  Returns a dict of counts."""
    B, gamma = out["draft"].shape
    nl = len(c.layers)
    cs = c.vocab // c.centroids.shape[0] if out["band"] and c.centroids is not None else 1
    n = dict(steps=0, draft_differs=0, cut_differs=0, flagged=int(out["flags"].sum()),
             flagged_draw=int(out["flags_draw"].sum()), flagged_cut=int(out["flags_cut"].sum()))
    for b in range(B):
        for k in range(gamma):
            n["steps"] += 1
            if gd[b, k] != out["draft"][b, k]:
                assert out["flags"][b, k], (f"{label}: b={b} step {k}: gpu draft {gd[b, k]} oracle "
                                            f"{out['draft'][b, k]} (unflagged)")
                n["draft_differs"] += 1
            if out["q"] is None:
                continue
            qo, qg = out["q"][b, k].astype(np.float64), gq[b, k].astype(np.float64)
            if not np.array_equal(qo > 0, qg > 0):       # another kept cluster set: only band clusters may move
                co = set((np.nonzero(qo > 0)[0] // cs).tolist())
                cg = set((np.nonzero(qg > 0)[0] // cs).tolist())
                near_in, near_out = out["band"][k][b]
                assert (co ^ cg) <= set(near_in) | set(near_out), (
                    f"{label}: b={b} step {k}: kept clusters differ outside the band: {sorted(co ^ cg)}")
                n["cut_differs"] += 1
                continue
            if qo.max() > 0:
                err = np.abs(qg - qo).max() / qo.max()
                assert err <= dbnd.q_tol(k, nl), f"{label}: b={b} step {k} q err {err:.2e}"
    return n


def run(c, masked, gamma, T, q_dtype=torch.float32, seed=None):
    dr, kv = device_drafter(c, masked)
    seed = c.seed if seed is None else seed
    gd, gq = sv.mtp_draft(dr, kv, dev(c.last_token.astype(np.int32)), dev_bf16(c.h_target), gamma, T, seed,
                          q_dtype=q_dtype)
    torch.cuda.synchronize()
    gd = gd.cpu().numpy()
    gq = None if gq is None else gq.float().cpu().numpy()
    nl = len(c.layers)
    out = od.draft(oracle_weights(c, masked), od.SharedKV(k=c.kv_k, v=c.kv_v, length=c.length), c.last_token,
                   c.h_target, gamma, T, seed, margin=[dbnd.margin(k, nl, T) for k in range(gamma)], force=gd)
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
    n = compare(c, out, gd, gq, f"V={V} B={B}")
    assert n["steps"] == B * gamma
    assert np.all((gd >= 0) & (gd < V))
    if gq is not None:
        np.testing.assert_allclose(gq.sum(-1), 1.0, atol=1e-4)
    log(f"[drafter] drafts {gd.tolist()}: {n}")


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
    n = compare(c, out, gd, gq, f"full B={B} T={T}")
    log(f"[drafter full] B={B} T={T} drafts {gd.tolist()}: {n}")
    assert n["steps"] == B * 4
