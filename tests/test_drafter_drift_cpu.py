"""The drafter test's parity bounds, reproduced on the CPU: a float32 evaluation of the
drafter recipe (tests/drafter_bounds.py) drifts from the float64 oracle by a measured
amount at every step, and the margin and q tolerance that tests/test_gpu_drafter.py
applies must cover that drift ([X-thread] "Gemma 4's MTP"; [MTP-deep-dive] 3.1-3.3 for
the drafter's structure).  Full shapes: V = 262144 token table in 2048 clusters with 32
kept, D = 1536, H = 256, four layers of 4 x 128 query heads over 700-2048 cached
positions, d_ff 2048, twelve rows, gamma = 4."""
import numpy as np
import pytest

import workloads
from oracle import drafter as od
from tests import drafter_bounds as dbnd


def oracle_weights(c):
    return od.DrafterWeights(d_model=c.d_model, hidden=c.hidden, n_heads=c.n_heads, head_dim=c.head_dim,
                             d_ff=c.d_ff, vocab=c.vocab, rms_eps=1e-5, rope_theta=10000.0, embed=c.embed,
                             pre_proj=c.pre_proj, layers=c.layers, final_norm=c.final_norm, post_proj=c.post_proj,
                             centroids=c.centroids, top_k_clusters=c.top_k)


def test_float32_model_matches_oracle_on_exact_inputs():
    """The float32 model is the oracle's recipe: with every product exact in float32 (a
    one-layer drafter whose weights and inputs are small powers of two, so no rounding
    happens anywhere) it reproduces the oracle's hidden state bit for bit."""
    c = workloads.drafter_case(V=256, D=32, H=32, n_layers=1, n_heads=1, head_dim=64, d_ff=32, C=16, top_k=4,
                               B=2, length=[3, 5], variant=3)
    for arr in [c.pre_proj, c.post_proj] + [L[k] for L in c.layers for k in ("wq", "wo", "w_gate", "w_up",
                                                                             "w_down")]:
        arr[...] = 0
    wts = oracle_weights(c)
    kv = od.SharedKV(k=c.kv_k, v=c.kv_v, length=c.length)
    g64 = od.step_hidden(wts, kv, c.last_token, c.h_target, 0)
    g32 = dbnd.step_hidden_f32(wts, kv, c.last_token, dbnd._f32(c.h_target), 0)
    assert np.array_equal(dbnd._f32(g64), g32)          # all zeros through zero weights, the norms intact
    # and a perturbation the recipe must carry: the rounding helper is round-to-nearest-even
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8], dtype=np.float32)
    assert dbnd._round_bf16_f32(x).tolist() == [1.0, 1.0 + 2.0 ** -6, -1.0]


@pytest.fixture(scope="module")
def full_case():
    lengths = [2048, 1500, 700, 2040, 1024, 1900, 800, 2000, 1234, 1777, 950, 2047]
    return workloads.drafter_case(B=len(lengths), length=lengths, max_len=2048, variant=11)


def test_bounds_cover_float32_drift_at_full_shapes(full_case):
    c = full_case
    wts = oracle_weights(c)
    kv = od.SharedKV(k=c.kv_k, v=c.kv_v, length=c.length)
    dl, dq = dbnd.float32_drift(wts, kv, c.last_token, c.h_target, 4, 1.0, c.seed)
    nl = len(c.layers)
    print("float32 drift per step: logits", np.array2string(dl, precision=4), "q", np.array2string(dq, precision=4))
    for k in range(4):
        m, qt = dbnd.margin(k, nl, 1.0), dbnd.q_tol(k, nl)
        print(f"step {k}: 2 x logit drift {2 * dl[k]:.4f} <= margin {m:.4f}; q drift {dq[k]:.4f} <= {qt:.4f}")
        assert 2 * dl[k] <= m, (k, dl[k], m)
        assert dq[k] <= qt, (k, dq[k], qt)
    # the drift is real (the bound is not vacuous) and grows with the depth traversed
    assert dl[0] > 1e-3 and dl[-1] > dl[0]
