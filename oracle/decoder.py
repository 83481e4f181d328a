"""Reference decoder for the full-model verify forward (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The target model is a pre-norm decoder: token embedding, then per layer
RMSNorm -> Q/K/V projections -> rotary position embedding (rotate-half) ->
causal attention over the KV cache plus the new positions -> output
projection -> residual add -> RMSNorm -> SwiGLU feed-forward -> residual add;
then a final RMSNorm and an (untied) LM head.

The verify pass feeds the last accepted token and the gamma drafts as gamma+1
new positions in one forward.  Position i attends to the whole cache and to
new positions 0..i only, so its prediction never sees later drafts
([Infra-ch8] "why one forward pass can verify several tokens").  K and V of
all gamma+1 positions are written into the cache at ``len .. len+gamma``;
the caller then keeps only the accepted ones by setting
``len += n + 1`` ([Self-spec] section 3.3: trim the cache to the accepted
length and check that cache length equals sequence length;
[MTP-drafters] section 4.2 item 3: only the accepted part of the verify
pass's cache stays valid).

Arithmetic: float64 throughout, with bf16 round-to-nearest-even at exactly
the points where the GPU stores bf16 (the GPU's matrix-core inputs):
(i) each RMSNorm output, (ii) K (after RoPE) and V as stored in the cache,
(iii) the attention output fed to the output projection, (iv) SiLU(gate)*up
fed to the down projection, (v) the final-norm output fed to the LM head.
Q, attention scores, softmax and the residual stream stay unrounded.

Pinned by (tests/test_oracle_decoder.py): per-operation closed forms
(RMSNorm of a constant vector, RoPE as a rotation with relative-position
scores, attention over one key / identical keys, SiLU values); verifying
G positions in one pass equals G single-position passes; changing a later
token leaves earlier slots unchanged; greedy speculative decoding reproduces
plain greedy autoregressive decoding token for token; and, with ``exact``, the
end-to-end logits of random small models equal those of the Llama implementation
in the ``transformers`` library run in float64 (tests/test_oracle_decoder_hf.py).
"""
from dataclasses import dataclass, field
from typing import List

import numpy as np

from .bf16 import bf16_to_f64, round_bf16, f64_to_bf16

LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")


@dataclass
class DecoderWeights:
    """bf16 weights (uint16 bit patterns), row-major [out, in] matrices."""
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ff: int
    vocab: int
    rms_eps: float
    rope_theta: float
    embed: np.ndarray                 # [vocab, d]
    layers: List[dict] = field(default_factory=list)   # LAYER_KEYS -> array
    final_norm: np.ndarray = None     # [d]
    lm_head: np.ndarray = None        # [vocab, d]


@dataclass
class KVCache:
    """bf16 cache [n_layers, B, n_heads, max_len, head_dim] and lengths [B]."""
    k: np.ndarray
    v: np.ndarray
    length: np.ndarray


def rmsnorm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def rope(x, pos, theta):
    """Rotary embedding, rotate-half convention.

    ``x``: [..., n_heads, head_dim]; ``pos``: broadcastable to x.shape[:-2].
    Pair (j, j + head_dim/2) is rotated by angle pos * theta^(-2j/head_dim).
    """
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv      # [..., 1, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    """x * sigmoid(x)."""
    return x / (1.0 + np.exp(-x))


def attention(q, k, v):
    """softmax(q k^T / sqrt(head_dim)) v for one query row set.

    ``q``: [nq, hd], ``k``/``v``: [nk, hd]; every query sees every key given.
    """
    s = q @ k.T / np.sqrt(q.shape[-1])
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v


def _w(a):
    return bf16_to_f64(a)


def forward(wts: DecoderWeights, tokens, kv: KVCache, exact: bool = False):
    """Verify forward over ``tokens`` [B, G] (G = gamma + 1 new positions).

    Writes K/V of the G positions into ``kv`` at ``length[b] + i`` and returns
    float64 logits [B, G, vocab].  ``kv.length`` is left unchanged; commit with
    :func:`commit`.

    ``exact``: the same model without the five bf16 rounding points (the new
    positions' K/V enter the attention in float64; the cache still stores them as
    bf16), for comparison with other float64 implementations of the architecture.
    """
    rnd = (lambda a: a) if exact else round_bf16
    tokens = np.asarray(tokens, dtype=np.int64)
    B, G = tokens.shape
    H, hd, d = wts.n_heads, wts.head_dim, wts.d_model
    base = np.asarray(kv.length, dtype=np.int64)
    if np.any(base + G > kv.k.shape[3]):
        raise ValueError("KV cache too short for the verify positions")
    pos = base[:, None] + np.arange(G)[None, :]                       # [B, G]
    x = _w(wts.embed[tokens])                                          # [B, G, d]
    for li, L in enumerate(wts.layers):
        h = rnd(rmsnorm(x, _w(L["attn_norm"]), wts.rms_eps))
        q = (h @ _w(L["wq"]).T).reshape(B, G, H, hd)
        k = (h @ _w(L["wk"]).T).reshape(B, G, H, hd)
        v = (h @ _w(L["wv"]).T).reshape(B, G, H, hd)
        q = rope(q, pos, wts.rope_theta)
        k = rope(k, pos, wts.rope_theta)
        kb, vb = f64_to_bf16(k), f64_to_bf16(v)
        for b in range(B):
            for i in range(G):
                kv.k[li, b, :, pos[b, i], :] = kb[b, i]
                kv.v[li, b, :, pos[b, i], :] = vb[b, i]
        o = np.zeros((B, G, H, hd))
        for b in range(B):
            nk = int(base[b]) + G
            kk = bf16_to_f64(kv.k[li, b, :, :nk, :])                  # [H, nk, hd]
            vv = bf16_to_f64(kv.v[li, b, :, :nk, :])
            if exact:
                kk[:, int(base[b]):nk] = k[b].transpose(1, 0, 2)
                vv[:, int(base[b]):nk] = v[b].transpose(1, 0, 2)
            for i in range(G):
                lim = int(base[b]) + i + 1                             # causal
                for hh in range(H):
                    o[b, i, hh] = attention(q[b, i, hh][None, :], kk[hh, :lim], vv[hh, :lim])[0]
        a = rnd(o.reshape(B, G, H * hd))
        x = x + a @ _w(L["wo"]).T
        h2 = rnd(rmsnorm(x, _w(L["ffn_norm"]), wts.rms_eps))
        f = rnd(silu(h2 @ _w(L["w_gate"]).T) * (h2 @ _w(L["w_up"]).T))
        x = x + f @ _w(L["w_down"]).T
    hf = rnd(rmsnorm(x, _w(wts.final_norm), wts.rms_eps))
    return hf @ _w(wts.lm_head).T


def commit(kv: KVCache, n_accepted):
    """Keep the accepted positions: length += n + 1 (step a8)."""
    kv.length = np.asarray(kv.length, dtype=np.int64) + np.asarray(n_accepted, dtype=np.int64) + 1


def greedy_autoregressive(wts: DecoderWeights, first_token, kv: KVCache, steps):
    """Plain greedy decoding, one position per forward ([Self-spec] 1.1).

    Feeds ``first_token`` [B], appends the argmax, repeats ``steps`` times;
    returns the generated tokens [B, steps].  The argmax is taken over the
    float32-rounded logits (lowest index on ties), as the verify rule does.
    """
    B = len(first_token)
    cur = np.asarray(first_token, dtype=np.int64)[:, None]
    out = []
    for _ in range(steps):
        logits = forward(wts, cur, kv)
        nxt = np.argmax(logits[:, 0, :].astype(np.float32), axis=-1)
        commit(kv, np.zeros(B, dtype=np.int64))
        out.append(nxt)
        cur = nxt[:, None]
    return np.stack(out, axis=1)
