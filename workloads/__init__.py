"""Seeded synthetic inputs for the verify step.

This module only draws random inputs; it holds none of the verify step's
arithmetic.  It is shared by the tests, ``bench.py`` and ``smoke()``: the
oracle and the GPU path consume the same arrays it returns.

Inputs stand in for the pages' workloads (no public dataset or trained weight
is used): a V = 262144, d = 1536 LM head like the Gemma 4 E2B table, gamma = 4
drafts, temperatures 0 / 0.7 / 1, draft/target agreement around 0.6-0.8, and a
7B-shaped decoder.  Every generator is deterministic in its seed; large arrays
are filled in fixed 4 Mi-element chunks from per-chunk child seeds, in
parallel threads, so the result does not depend on the thread count.

The synthetic drafter.  A draft distribution q is the drafter's output, which
this module must invent: it perturbs float32 target logits (computed here with
a plain float32 numpy product, independent of both the oracle and the GPU
library) with Gaussian noise and applies the softmax at the verify
temperature.  That is the drafter, not the verify computation.

Conventions: bf16 arrays are ``numpy.uint16`` bit patterns (float32 rounded to
nearest even, by this module's own conversion); token ids are int32.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

CHUNK = 1 << 22
N_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)))
PHILOX_SEED_BASE = 0x5EED0000


def input_seed(k):
    """numpy seed of configuration k (1-based)."""
    return 1000 + k


def philox_seed(k):
    """Verify-stream seed of configuration k."""
    return PHILOX_SEED_BASE + k


# ----------------------------------------------------------------------------
# bulk random fills

def _flat_tag(tag):
    if isinstance(tag, (tuple, list)):
        out = []
        for t in tag:
            out.extend(_flat_tag(t))
        return out
    return [int(tag)]


def _fill(out_flat, seed, tag, kind):
    n = out_flat.size
    key = tuple(_flat_tag(tag))
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(i):
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=key + (i,))))
        sl = out_flat[i * CHUNK:min(n, (i + 1) * CHUNK)]
        if kind == "normal":
            g.standard_normal(out=sl, dtype=np.float32)
        else:
            g.random(out=sl, dtype=np.float32)

    if nchunks <= 1:
        for i in range(nchunks):
            work(i)
    else:
        with ThreadPoolExecutor(N_THREADS) as ex:
            list(ex.map(work, range(nchunks)))


def normal_f32(shape, std, seed, tag):
    """float32 N(0, std^2) array of ``shape``; deterministic in (seed, tag)."""
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    _fill(out, seed, tag, "normal")
    if std != 1.0:
        np.multiply(out, np.float32(std), out=out)
    return out.reshape(shape)


def to_bf16_bits(x):
    """float32 -> bf16 bit patterns, round to nearest even (chunked)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.size, dtype=np.uint16)

    def work(i):
        b = flat[i * CHUNK:(i + 1) * CHUNK]
        r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        out[i * CHUNK:(i + 1) * CHUNK] = r.astype(np.uint16)

    nchunks = (flat.size + CHUNK - 1) // CHUNK
    with ThreadPoolExecutor(N_THREADS) as ex:
        list(ex.map(work, range(nchunks)))
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std, seed, tag):
    """bf16 bit patterns of N(0, std^2) draws."""
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1)
    n = flat.size
    # generate in slabs to bound float32 temporaries
    slab = 1 << 26
    for s0 in range(0, n, slab):
        m = min(slab, n - s0)
        f = normal_f32((m,), std, seed, (tag, s0 // slab))
        flat[s0:s0 + m] = to_bf16_bits(f)
    return out


# ----------------------------------------------------------------------------
# the synthetic drafter

def _softmax_f32(z):
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def drafter(target_logits_f32, noise, temperature, rng):
    """Drafts and q from perturbed target logits.

    T > 0: q = softmax((l + noise) / T), drafts x ~ q (inverse CDF on the
    float32 q).  T == 0: drafts = argmax(l + noise), q = None.
    ``target_logits_f32``: [B, gamma, V] float32 logits of slots 0..gamma-1.
    """
    z = target_logits_f32 + noise
    if temperature == 0.0:
        return np.argmax(z, axis=-1).astype(np.int32), None
    q = _softmax_f32((z / np.float32(temperature)).astype(np.float32)).astype(np.float32)
    B, g, V = q.shape
    cdf = np.cumsum(q.astype(np.float64), axis=-1)
    u = rng.random((B, g)) * cdf[..., -1]
    x = np.empty((B, g), dtype=np.int32)
    for b in range(B):
        for i in range(g):
            x[b, i] = min(int(np.searchsorted(cdf[b, i], u[b, i], side="right")), V - 1)
    return x, q


def _f32_product(h_f32, w_bits_or_f32):
    """float32 h @ w^T for the drafter (w given as bf16 bits or float32)."""
    w = w_bits_or_f32
    if w.dtype == np.uint16:
        V = w.shape[0]
        out = np.empty(h_f32.shape[:-1] + (V,), dtype=np.float32)
        step = 1 << 15
        for v0 in range(0, V, step):
            wf = bf16_bits_to_f32(w[v0:v0 + step])
            out[..., v0:v0 + step] = h_f32 @ wf.T
        return out
    return h_f32 @ w.T


# ----------------------------------------------------------------------------
# LM-head workloads (configurations 1, 3, 4)

@dataclass
class LMHeadCase:
    """One verify call of the LM-head configurations."""
    w: np.ndarray                 # [V, d] bf16 bits or float32
    h: np.ndarray                 # [B, gamma+1, d] same dtype as w
    draft: np.ndarray             # [B, gamma] int32
    q: Optional[np.ndarray]       # [B, gamma, V] bf16 bits or float32 (None at T == 0)
    temperature: float
    seed: int                     # verify-stream seed
    pos0: np.ndarray              # [B] int64
    dtype: str                    # "bf16" or "f32"

    @property
    def B(self):
        return self.h.shape[0]

    @property
    def gamma(self):
        return self.h.shape[1] - 1

    @property
    def V(self):
        return self.w.shape[0]


def tiny_ref(rounds=1000, temperature=1.0, k=1):
    """Configuration 1: B=1, gamma=4, float32, V=1024, d=64.

    W ~ N(0, 1/64) (variance 1/d), per round hidden ~ N(0, 1) and drafter
    noise ~ N(0, 1).  Returns (W, list of per-round (h, draft, q)).
    """
    V, d, gamma = 1024, 64, 4
    seed = input_seed(k)
    w = normal_f32((V, d), 1.0 / np.sqrt(d), seed, 0)
    h = normal_f32((rounds, 1, gamma + 1, d), 1.0, seed, 1)
    noise = normal_f32((rounds, 1, gamma, V), 1.0, seed, 2)
    rng = np.random.default_rng(seed + 7)
    out = []
    for r in range(rounds):
        lt = _f32_product(h[r, :, :gamma], w)
        x, q = drafter(lt, noise[r], temperature, rng)
        out.append((h[r], x, q))
    return w, out


def lm_head_case(V, d, B, gamma, temperature, noise_std, k, w=None, pos0=0, variant=0):
    """Configurations 3 and 4: bf16 W ~ N(0, 0.02^2), hidden ~ N(0, 1).

    Draft q = softmax((l + N(0, noise_std^2)) / T) stored as bf16.
    ``w`` may be passed in to reuse a large table across cases; ``variant``
    draws an independent set of hidden states, noise and drafts.
    """
    seed = input_seed(k)
    if w is None:
        w = normal_bf16((V, d), 0.02, seed, 0)
    tag = (B, gamma, int(round(temperature * 1000))) + ((variant,) if variant else ())
    h = normal_bf16((B, gamma + 1, d), 1.0, seed, (1,) + tag)
    hf = bf16_bits_to_f32(h)
    lt = _f32_product(hf[:, :gamma], w)
    noise = normal_f32((B, gamma, V), noise_std, seed, (2,) + tag)
    rng = np.random.default_rng([seed, 7, B, gamma, int(round(temperature * 1000)), variant])
    x, q = drafter(lt, noise, temperature, rng)
    qb = None if q is None else to_bf16_bits(q)
    return LMHeadCase(w=w, h=h, draft=x, q=qb, temperature=float(temperature),
                      seed=philox_seed(k), pos0=np.full(B, pos0, dtype=np.int64), dtype="bf16")


def large_vocab(B=1, temperature=1.0, w=None):
    """Configuration 3: V=262144, d=1536, gamma=4, noise std 1."""
    return lm_head_case(262144, 1536, B, 4, temperature, 1.0, 3, w=w)


def batch_sweep(B=1, gamma=4, w=None):
    """Configuration 4: V=262144, d=4096, T=1, noise std 0.5."""
    return lm_head_case(262144, 4096, B, gamma, 1.0, 0.5, 4, w=w)


# ----------------------------------------------------------------------------
# configuration 2: acceptance statistics

@dataclass
class StatsCase:
    p: np.ndarray        # [gamma+1, V] float64 target distributions
    q: np.ndarray        # [gamma, V] float32 draft distributions (as stored)
    logits: np.ndarray   # [gamma+1, V] float32 = log p
    draft: np.ndarray    # [rounds, gamma] int32, x_i ~ q_i
    seed: int


def acceptance_stats(rounds=1_000_000, V=32, gamma=4, alpha=0.8, k=2):
    """Configuration 2: fixed p_j ~ Dir(0.5), r_j ~ Dir(0.5),
    q_j = (1 - lam_j) p_j + lam_j r_j with lam_j = (1 - alpha) / TV(p_j, r_j),
    so sum_v min(p_j, q_j) = alpha exactly (TV is linear along the segment).
    Logits input is log p (float32); one sequence per round, pos0 = 0.
    """
    rng = np.random.default_rng(input_seed(k))
    p = rng.dirichlet(np.full(V, 0.5), size=gamma + 1)
    q = np.empty((gamma, V))
    for j in range(gamma):
        while True:
            r = rng.dirichlet(np.full(V, 0.5))
            tv = 0.5 * np.abs(p[j] - r).sum()
            if tv >= (1.0 - alpha):
                break
        lam = (1.0 - alpha) / tv
        q[j] = (1.0 - lam) * p[j] + lam * r
    q32 = q.astype(np.float32)
    logits = np.log(p).astype(np.float32)
    draft = np.empty((rounds, gamma), dtype=np.int32)
    for j in range(gamma):
        cdf = np.cumsum(q32[j].astype(np.float64))
        u = rng.random(rounds) * cdf[-1]
        draft[:, j] = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1)
    return StatsCase(p=p, q=q32, logits=logits, draft=draft, seed=philox_seed(k))


# ----------------------------------------------------------------------------
# configuration 5: full-model verify

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


@dataclass
class DecoderCase:
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    rms_eps: float
    rope_theta: float
    embed: np.ndarray
    layers: List[dict]
    final_norm: np.ndarray
    lm_head: np.ndarray
    k_cache: np.ndarray          # [L, B, H, max_len, hd] bf16 bits
    v_cache: np.ndarray
    length: np.ndarray           # [B] int32
    tokens: np.ndarray           # [B, gamma+1] int32 (slot 0 = last accepted)
    q: np.ndarray                # [B, gamma, V] float32 (uniform drafter)
    seed: int
    pos0: np.ndarray             # [B] int64 == length


def decoder_case(n_layers=32, d_model=4096, n_heads=32, head_dim=128, d_ff=11008, vocab=32000,
                 cache_len=2048, B=1, gamma=4, max_len=None, k=5, std=0.02):
    """Configuration 5 (defaults): 32-layer random decoder, bf16 N(0, 0.02^2)
    weights, RMSNorm gains 1, KV cache of ``cache_len`` tokens ~ N(0, 1),
    gamma+1 new token ids uniform in [0, vocab), drafter q uniform 1/vocab.
    Smaller shapes give the small decoder cases used by the tests.
    """
    seed = input_seed(k)
    tagb = (n_layers, d_model, n_heads, d_ff, vocab, cache_len, B, gamma)
    ones = to_bf16_bits(np.ones(d_model, dtype=np.float32))
    embed = normal_bf16((vocab, d_model), std, seed, (0,) + tagb)
    layers = []
    for li in range(n_layers):
        L = {"attn_norm": ones.copy(), "ffn_norm": ones.copy()}
        for j, (name, shp) in enumerate((("wq", (n_heads * head_dim, d_model)),
                                          ("wk", (n_heads * head_dim, d_model)),
                                          ("wv", (n_heads * head_dim, d_model)),
                                          ("wo", (d_model, n_heads * head_dim)),
                                          ("w_gate", (d_ff, d_model)),
                                          ("w_up", (d_ff, d_model)),
                                          ("w_down", (d_model, d_ff)))):
            L[name] = normal_bf16(shp, std, seed, (1, li, j) + tagb)
        layers.append(L)
    lm_head = normal_bf16((vocab, d_model), std, seed, (2,) + tagb)
    if max_len is None:
        max_len = cache_len + gamma + 1
    kc = np.zeros((n_layers, B, n_heads, max_len, head_dim), dtype=np.uint16)
    vc = np.zeros_like(kc)
    kc[:, :, :, :cache_len] = normal_bf16((n_layers, B, n_heads, cache_len, head_dim), 1.0, seed, (3,) + tagb)
    vc[:, :, :, :cache_len] = normal_bf16((n_layers, B, n_heads, cache_len, head_dim), 1.0, seed, (4,) + tagb)
    rng = np.random.default_rng([seed, 9] + list(tagb))
    tokens = rng.integers(0, vocab, size=(B, gamma + 1), dtype=np.int64).astype(np.int32)
    q = np.full((B, gamma, vocab), 1.0 / vocab, dtype=np.float32)
    return DecoderCase(n_layers, d_model, n_heads, head_dim, d_ff, vocab, 1e-5, 10000.0,
                       embed, layers, ones.copy(), lm_head, kc, vc,
                       np.full(B, cache_len, dtype=np.int32), tokens, q, philox_seed(k),
                       np.full(B, cache_len, dtype=np.int64))


def small_decoder_case(**kw):
    """A small decoder with the same structure, for fast parity tests."""
    args = dict(n_layers=2, d_model=256, n_heads=2, head_dim=128, d_ff=512, vocab=1000,
                cache_len=100, B=1, gamma=4, k=5, std=0.05)
    args.update(kw)
    return decoder_case(**args)


# ----------------------------------------------------------------------------
# the drafter's centroid-masked LM head

@dataclass
class MaskedHeadCase:
    w: np.ndarray          # bf16 bits [V, d], cluster-ordered token table
    centroids: np.ndarray  # bf16 bits [C, d], one representative per cluster
    h: np.ndarray          # bf16 bits [M, d], drafter hidden states
    top_k: int


def masked_head_case(V=262144, d=1536, C=2048, M=1, top_k=32, k=6, spread=0.01, variant=0):
    """Synthetic cluster-ordered embeddings: cluster c has a centre mu_c ~ N(0, 0.02^2)
    and its cs = V / C member tokens are mu_c + N(0, spread^2) (rounded to bf16), so that
    members are close to their cluster's representative; the representative table is
    the bf16-rounded mean of the member rows (the classic k-means centre).  Hidden
    states ~ N(0, 1).  These stand in for a trained drafter's clustered embeddings."""
    seed = input_seed(k)
    cs = V // C
    mu = normal_f32((C, d), 0.02, seed, (10, C, d))
    eps = normal_f32((V, d), spread, seed, (11, V, d))
    wf = (eps.reshape(C, cs, d) + mu[:, None, :]).reshape(V, d)
    del eps
    w = to_bf16_bits(wf)
    del wf
    cent = np.zeros((C, d), dtype=np.float64)
    wb = bf16_bits_to_f32(w).reshape(C, cs, d)
    for c0 in range(0, C, 256):
        cent[c0:c0 + 256] = wb[c0:c0 + 256].astype(np.float64).mean(axis=1)
    del wb
    centroids = to_bf16_bits(cent.astype(np.float32))
    h = normal_bf16((M, d), 1.0, seed, (12, M, variant))
    return MaskedHeadCase(w=w, centroids=centroids, h=h, top_k=top_k)


# ----------------------------------------------------------------------------
# the MTP drafter's draft step

@dataclass
class DrafterCase:
    d_model: int
    hidden: int
    n_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    embed: np.ndarray            # bf16 bits [V, D] (cluster-ordered token table)
    centroids: np.ndarray        # bf16 bits [C, D]
    pre_proj: np.ndarray         # bf16 bits [H, 2D]
    layers: list                 # per layer: dict attn_norm, wq, wo, ffn_norm, w_gate, w_up, w_down
    final_norm: np.ndarray       # bf16 bits [H]
    post_proj: np.ndarray        # bf16 bits [D, H]
    kv_k: list                   # per drafter layer: bf16 bits [B, n_heads, max_len, head_dim]
    kv_v: list
    length: np.ndarray           # int32 [B]
    last_token: np.ndarray       # int32 [B]
    h_target: np.ndarray         # bf16 bits [B, D]
    seed: int
    top_k: int


def drafter_case(V=262144, D=1536, H=256, n_layers=4, n_heads=4, head_dim=128, d_ff=2048, C=2048, top_k=32,
                 B=1, length=2048, max_len=None, shared_layers=(0, 0, 0, 1), k=7, variant=0):
    """A random-init drafter of the E2B shapes (V = 262144, D = 1536, H = 256, four
    layers) with the masked head's synthetic clustered token table, and the target
    state it drafts from: cache layers of N(0, 1) keys and values (drafter layer l
    reads target layer shared_layers[l]), lengths ``length`` (an int or one per row),
    the last emitted tokens and the target's last hidden states ~ N(0, 1).  Weight
    scales keep every stage near unit size: pre_proj N(0, 1/(2D)), wq N(0, 1/H),
    wo N(0, 1/(heads * head_dim)), gate/up N(0, 1/H), down N(0, 1/d_ff), post_proj
    N(0, 0.2^2), norm gains 1."""
    seed = input_seed(k)
    mh = masked_head_case(V=V, d=D, C=C, M=1, top_k=top_k, k=k, variant=variant)
    HD = n_heads * head_dim
    one_h = to_bf16_bits(np.ones(H, dtype=np.float32))

    def nb(shape, std, tag):
        return normal_bf16(shape, std, seed, (20, variant) + tuple(tag))

    layers = []
    for l in range(n_layers):
        layers.append(dict(attn_norm=one_h.copy(), wq=nb((HD, H), H ** -0.5, (l, 1)),
                           wo=nb((H, HD), HD ** -0.5, (l, 2)), ffn_norm=one_h.copy(),
                           w_gate=nb((d_ff, H), H ** -0.5, (l, 3)), w_up=nb((d_ff, H), H ** -0.5, (l, 4)),
                           w_down=nb((H, d_ff), d_ff ** -0.5, (l, 5))))
    max_len = max_len or int(np.max(length)) + 8
    n_shared = max(shared_layers) + 1
    ks = [nb((B, n_heads, max_len, head_dim), 1.0, (100 + j, B, max_len)) for j in range(n_shared)]
    vs = [nb((B, n_heads, max_len, head_dim), 1.0, (200 + j, B, max_len)) for j in range(n_shared)]
    lens = np.broadcast_to(np.asarray(length, dtype=np.int32), (B,)).copy()
    rng = np.random.default_rng(seed + 31 * variant + B)
    return DrafterCase(d_model=D, hidden=H, n_heads=n_heads, head_dim=head_dim, d_ff=d_ff, vocab=V,
                       embed=mh.w, centroids=mh.centroids, pre_proj=nb((H, 2 * D), (2 * D) ** -0.5, (0, 0)),
                       layers=layers, final_norm=one_h.copy(), post_proj=nb((D, H), 0.2, (0, 9)),
                       kv_k=[ks[j] for j in shared_layers], kv_v=[vs[j] for j in shared_layers], length=lens,
                       last_token=rng.integers(0, V, B).astype(np.int32),
                       h_target=nb((B, D), 1.0, (300, B)), seed=philox_seed(k + variant), top_k=top_k)
