"""GPU parity of the drafter's centroid-masked LM head against the CPU oracle, through
the C ABI ([X-thread] "Gemma 4's MTP", efficient embedder; [MTP-deep-dive] 3.4).

Bar: the kept clusters bit-exact as a set and in order, except where the oracle flags
a near tie (score gap below 1e-3: at the top_k cut the set may differ; inside the kept
list neighbours may swap); the cluster scores and the token logits of the kept
clusters within 1e-4 of the row's max |value| (bf16 inputs, float32 accumulation),
the token logits checked for whatever clusters the GPU kept.
"""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import bf16 as obf16
from oracle import masked_head as mh
from tests.gpu_util import dev_bf16, log, row_rel_err

pytestmark = pytest.mark.gpu

FLAG = 1e-3


def run_and_compare(w, cent, h, top_k, label):
    V, d = w.shape
    C, M = cent.shape[0], h.shape[0]
    cs = V // C
    head = sv.masked_head(dev_bf16(w), dev_bf16(cent))
    cl_gpu = torch.empty((M, C), dtype=torch.float32, device="cuda")
    sel, logits = sv.draft_masked_logits(head, dev_bf16(h), top_k, cluster_logits=cl_gpu)
    torch.cuda.synchronize()
    sel, logits, cl_gpu = sel.cpu().numpy(), logits.cpu().numpy(), cl_gpu.cpu().numpy()
    hf, cf = obf16.bf16_to_f64(h), obf16.bf16_to_f64(cent)
    cl_ref = mh.cluster_logits(hf, cf)
    assert row_rel_err(cl_gpu, cl_ref).max() <= 1e-4, label
    ref_sel, flags = mh.select_clusters(cl_ref, top_k)
    c32 = cl_ref.astype(np.float32).astype(np.float64)
    for m in range(M):
        g, r = sel[m].tolist(), ref_sel[m].tolist()
        assert len(set(g)) == top_k and all(0 <= c < C for c in g), label
        if not flags[m]:
            assert set(g) == set(r), f"{label}: row {m} kept {sorted(g)} vs oracle {sorted(r)}"
        # order: descending oracle score, swaps only between near-equal neighbours
        sc = c32[m, g]
        assert np.all(sc[:-1] >= sc[1:] - FLAG), f"{label}: row {m} order"
        exact = [a == b for a, b in zip(g, r)]
        if not all(exact):
            i = exact.index(False)
            assert flags[m] or abs(c32[m, g[i]] - c32[m, r[i]]) < FLAG, f"{label}: row {m} position {i}"
    # token logits of the clusters the GPU kept (only their rows of the table converted)
    ref_logits = np.empty_like(logits, dtype=np.float64)
    for m in range(M):
        tok = (sel[m].astype(np.int64)[:, None] * cs + np.arange(cs)[None, :]).reshape(-1)
        w_sub = obf16.bf16_to_f64(w[tok])
        ref_logits[m] = mh.masked_logits(hf[m:m + 1], w_sub, np.arange(top_k)[None, :], cs)[0]
    err = row_rel_err(logits, ref_logits).max()
    assert err <= 1e-4, f"{label}: token logits rel err {err}"
    return int(flags.sum())


SMALL = [
    # V, d, C, M, top_k
    (4096, 256, 64, 1, 5),
    (4096, 256, 64, 3, 64),      # every cluster kept
    (6000, 96, 48, 2, 7),        # 125 tokens per cluster: ragged 32-row chunks
    (2048, 1536, 2048, 2, 32),   # one token per cluster
    (1024, 512, 1, 1, 1),        # a single cluster
    (8192, 160, 4096, 4, 17),    # the largest cluster count the selection sorts
    (65536, 1536, 512, 24, 32),  # the largest M
]


@pytest.mark.parametrize("V,d,C,M,top_k", SMALL)
def test_small_and_ragged(V, d, C, M, top_k):
    log(f"[masked] V={V} d={d} C={C} M={M} top_k={top_k}")
    case = workloads.masked_head_case(V=V, d=d, C=C, M=M, top_k=top_k, k=60 + C % 7, variant=M)
    run_and_compare(case.w, case.centroids, case.h, top_k, f"V={V} C={C}")


@pytest.fixture(scope="module")
def full_case():
    return workloads.masked_head_case()


@pytest.mark.parametrize("M", [1, 4])
def test_full_size(full_case, M):
    """The pages' sizes: V = 262144, d = 1536, 2048 clusters, 32 kept."""
    log(f"[masked] full size M={M}")
    case = full_case
    h = workloads.normal_bf16((M, case.w.shape[1]), 1.0, 4242, (M,))
    nflag = run_and_compare(case.w, case.centroids, h, case.top_k, f"full M={M}")
    log(f"[masked] full M={M}: {nflag} flagged rows")


def test_workspace_and_caller_cluster_scores_agree(full_case):
    case = full_case
    head = sv.masked_head(dev_bf16(case.w), dev_bf16(case.centroids))
    h = dev_bf16(workloads.normal_bf16((3, case.w.shape[1]), 1.0, 99, (3,)))
    a_sel, a_log = sv.draft_masked_logits(head, h, 32)
    cl = torch.empty((3, case.centroids.shape[0]), dtype=torch.float32, device="cuda")
    b_sel, b_log = sv.draft_masked_logits(head, h, 32, cluster_logits=cl)
    torch.cuda.synchronize()
    assert torch.equal(a_sel, b_sel) and torch.equal(a_log, b_log)


@pytest.mark.parametrize("distinct,top_k", [(3, 17), (3, 64), (1, 64), (40, 33)])
def test_selection_with_ties_is_exact(distinct, top_k):
    """Cluster tables with only ``distinct`` different rows give scores with many exact
    ties: the kept clusters must be the top_k of the returned float32 scores, the lower id
    first on equal scores, in that order (index work: bit-exact).  One distinct row makes
    every score equal, which takes the selection's refinement down to the id bits."""
    log(f"[masked] ties distinct={distinct} top_k={top_k}")
    case = workloads.masked_head_case(V=8192, d=160, C=4096, M=2, top_k=top_k, k=5, variant=distinct)
    cent = case.centroids[np.arange(4096) % distinct]
    head = sv.masked_head(dev_bf16(case.w), dev_bf16(cent))
    cl = torch.empty((2, 4096), dtype=torch.float32, device="cuda")
    sel, _ = sv.draft_masked_logits(head, dev_bf16(case.h), top_k, cluster_logits=cl)
    torch.cuda.synchronize()
    sel, cl = sel.cpu().numpy(), cl.cpu().numpy()
    for m in range(2):
        order = np.lexsort((np.arange(4096), -cl[m].astype(np.float64)))
        assert sel[m].tolist() == order[:top_k].tolist(), f"row {m}"
