"""Centroid-masked LM head of the drafter (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[X-thread], section "Gemma 4's MTP", part "efficient embedder", and [MTP-deep-dive] 3.4
("centroids masking"): the token embeddings are grouped into clusters of tokens
with similar meaning and each cluster gets one representative embedding.  The
drafter's hidden state is multiplied by the table of representatives, which
scores the clusters instead of the tokens; the most likely clusters are kept, and
exact token logits are computed only for the tokens inside them (the pages quote
2048 clusters and 32 kept, about 4K of 262,144 tokens).

Readings (where the pages leave a step open):

* ordered embeddings: cluster c holds the contiguous token block
  [c * cs, (c + 1) * cs) with cs = V / C (the pages' ``use_ordered_embeddings``);
* the kept clusters are the top_k cluster logits in descending order, the lower
  cluster id first on equal values; cluster logits are compared in float32, the
  precision the kernel stores them in (computed exactly in float64, rounded once);
* the output is the kept clusters and the exact logits of their member tokens,
  block j holding tokens clusters[j] * cs + [0, cs); tokens outside the kept
  clusters are masked (never scored).

A selection whose k-th and (k+1)-th cluster logits differ by less than 1e-3 is
flagged: the GPU's float32 accumulation may order them differently there.
"""
import numpy as np

from .rules import FLAG_MARGIN


def cluster_size(V, C):
    """Tokens per cluster of the ordered embeddings (V must be a multiple of C)."""
    if V % C:
        raise ValueError("vocabulary not a multiple of the cluster count")
    return V // C


def cluster_logits(h, centroids):
    """Cluster scores h . centroid_c^T in float64 ([X-thread] "Gemma 4's MTP", efficient embedder:
    the hidden state times the new lookup table gives cluster logits instead of token
    logits).  ``h`` [M, d], ``centroids`` [C, d], float64 holding exact bf16 values.

    Pinned by: linearity (a mean-of-members centroid scores the mean of the members'
    token logits) and the plain LM head when every cluster is kept."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(centroids, dtype=np.float64).T


def select_clusters(cl, top_k):
    """The top_k clusters per row, descending float32 cluster logit, lower id first on
    ties ([MTP-deep-dive] 3.4: predict the top-k most likely clusters).  Returns
    (int64 [M, top_k], flags [M]): flags mark rows whose k-th and (k+1)-th values are
    closer than 1e-3.

    Pinned by: a hand-checked fixture with ties; the set property min(kept) >= max(rest)
    over every row of random inputs."""
    c32 = np.asarray(cl, dtype=np.float64).astype(np.float32)
    M, C = c32.shape
    if not 1 <= top_k <= C:
        raise ValueError("top_k out of range")
    out = np.empty((M, top_k), dtype=np.int64)
    flags = np.zeros(M, dtype=bool)
    for m in range(M):
        order = sorted(range(C), key=lambda c: (-float(c32[m, c]), c))
        out[m] = order[:top_k]
        if top_k < C:
            flags[m] = float(c32[m, order[top_k - 1]]) - float(c32[m, order[top_k]]) < FLAG_MARGIN
    return out, flags


def masked_logits(h, w, clusters, cs):
    """Exact logits of the member tokens of the kept clusters ([MTP-drafters] "efficient
    embedder": all tokens of the chosen clusters are used to compute the final token
    logits).  ``w`` [V, d] float64 token table (cluster-ordered), ``clusters`` [M, k].
    Returns float64 [M, k * cs], block j = tokens clusters[m, j] * cs + [0, cs).

    Pinned by: with every cluster kept, a reordering of the full LM-head logits; a
    brute-force loop on small integer inputs."""
    h = np.asarray(h, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    M, k = clusters.shape
    out = np.empty((M, k * cs))
    for m in range(M):
        tok = (clusters[m][:, None] * cs + np.arange(cs)[None, :]).reshape(-1)
        out[m] = w[tok] @ h[m]
    return out


def masked_head(h, w, centroids, top_k):
    """The whole masked head: (clusters, token logits float64, flags)."""
    C = np.asarray(centroids).shape[0]
    cs = cluster_size(np.asarray(w).shape[0], C)
    sel, flags = select_clusters(cluster_logits(h, centroids), top_k)
    return sel, masked_logits(h, w, sel, cs), flags
