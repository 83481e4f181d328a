"""Parity bounds of the MTP drafter's GPU test, and the float32 model they come from.

The drafter's hidden state passes through bf16 rounding points in every layer (the
RMSNorm outputs, the attention output, SiLU(gate) * up, the final-norm output and the
up-projected state itself) and is fed back at every step.  The GPU accumulates in
float32 and the oracle (oracle/drafter.py) in float64, so a difference of one float32
rounding before a rounding point either vanishes or becomes a whole bf16 step, and
those steps compound with the depth traversed.  The bounds the GPU test applies are
therefore derived, not fitted to the GPU: :func:`float32_drift` runs the same recipe
with float32 arithmetic on the CPU (numpy, the same operations in the same order as the
oracle, bf16 rounding at the same points), following the oracle's own drafted tokens so
both sides see the same inputs, and measures how far its logits and q move from the
oracle's at every step.  tests/test_drafter_drift_cpu.py recomputes that drift at the
full shapes and checks that the bounds below cover it.

Not a test module.  Test infrastructure only; shares no code with the HIP library.
"""
import numpy as np

from oracle import drafter as od
from oracle import rules

# Decision margin of step k: a draft whose two best scores are closer than
# MARGIN * depth_scale(k) / min(1, T) may differ from the oracle's (the scores log q + G
# move by up to twice the logit drift divided by T; T = 0 compares logits).  Cluster
# cuts use the same margin.  q is held to Q_TOL * depth_scale(k) of the row's largest
# q.  The float32 model's logit drift grows about linearly with the layers the hidden
# state has traversed, (k + 1) * n_layers: at the full shapes 0.040, 0.060, 0.083, 0.105
# at steps 0-3 of a four-layer drafter (twelve rows), its q drift up to 0.053; the scale
# 0.4 + 0.15 * layers traversed (1, 1.6, 2.2, 2.8 at four layers) keeps twice the logit
# drift about 25 % below the margin at every step.
MARGIN = 1e-1
Q_TOL = 4e-2


def depth_scale(k, n_layers):
    """Growth of the drift with the depth traversed by step k (0-based) of a drafter of
    n_layers layers (at least 1)."""
    return max(1.0, 0.4 + 0.15 * (k + 1) * n_layers)


def margin(k, n_layers, temperature=1.0):
    t = float(temperature)
    return MARGIN * depth_scale(k, n_layers) / (min(1.0, t) if t > 0 else 1.0)


def q_tol(k, n_layers):
    return Q_TOL * depth_scale(k, n_layers)


# ---------------------------------------------------------------------------
# float32 evaluation of the drafter step

def _f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _round_bf16_f32(x):
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def _rmsnorm32(x, g, eps):
    x = np.asarray(x, dtype=np.float32)
    ss = np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32)
    return x * (np.float32(1.0) / np.sqrt(ss / np.float32(x.shape[-1]) + np.float32(eps))) * g


def _rope32(x, pos, theta):
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-(2.0 * np.arange(half)) / hd)
    ang = np.asarray(pos, dtype=np.float64)[..., None, None] * inv
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _attention32(q, k, v):
    s = (q @ k.T) / np.float32(np.sqrt(q.shape[-1]))
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True, dtype=np.float32)
    return p @ v


def step_hidden_f32(wts, kv, tokens, g32, k):
    """One drafter pass in float32: the new hidden state (bf16 values as float32 [B, D])
    from the current tokens and hidden states, query position len + k."""
    tokens = np.asarray(tokens, dtype=np.int64)
    B = tokens.shape[0]
    nh, hd = wts.n_heads, wts.head_dim
    lens = np.asarray(kv.length, dtype=np.int64)
    ok = od.valid_rows(kv, tokens, wts.vocab)
    e = np.zeros((B, wts.d_model), dtype=np.float32)
    e[ok] = _f32(wts.embed[tokens[ok]])
    x = np.concatenate([e, g32], axis=1) @ _f32(wts.pre_proj).T
    pos = lens + k
    for li, L in enumerate(wts.layers):
        h = _round_bf16_f32(_rmsnorm32(x, _f32(L["attn_norm"]), wts.rms_eps))
        q = _rope32((h @ _f32(L["wq"]).T).reshape(B, nh, hd), pos, wts.rope_theta)
        o = np.zeros((B, nh, hd), dtype=np.float32)
        for b in range(B):
            if not ok[b]:
                continue
            n = int(lens[b])
            kk = _f32(kv.k[li][b, :, :n, :])
            vv = _f32(kv.v[li][b, :, :n, :])
            for hh in range(nh):
                o[b, hh] = _attention32(q[b, hh][None, :], kk[hh], vv[hh])[0]
        a = _round_bf16_f32(o.reshape(B, nh * hd))
        x = x + a @ _f32(L["wo"]).T
        h2 = _round_bf16_f32(_rmsnorm32(x, _f32(L["ffn_norm"]), wts.rms_eps))
        gate = h2 @ _f32(L["w_gate"]).T
        f = _round_bf16_f32(gate / (np.float32(1.0) + np.exp(-gate)) * (h2 @ _f32(L["w_up"]).T))
        x = x + f @ _f32(L["w_down"]).T
    hf = _round_bf16_f32(_rmsnorm32(x, _f32(wts.final_norm), wts.rms_eps))
    g = _round_bf16_f32(hf @ _f32(wts.post_proj).T)
    g[~ok] = 0.0
    return g


def float32_drift(wts, kv, last_token, h_target_bits, gamma, temperature, seed):
    """Largest logit drift and q drift of the float32 model against the oracle, per step.

    The oracle drafts (oracle/drafter.draft); the model follows the oracle's drafted
    tokens, keeps its own float32 hidden state, and is scored on the oracle's scored
    tokens.  Returns (logit_drift [gamma], q_drift [gamma]): per step the largest
    |l_f32 - l_oracle| over rows and scored tokens, and the largest
    max |q_f32 - q_oracle| / max q_oracle over rows (0 at T = 0)."""
    out = od.draft(wts, kv, last_token, h_target_bits, gamma, temperature, seed)
    ok = od.valid_rows(kv, last_token, wts.vocab)
    tokens = np.where(ok, np.asarray(last_token, dtype=np.int64), 0)
    g32 = _f32(h_target_bits)
    dl, dq = np.zeros(gamma), np.zeros(gamma)
    for k in range(gamma):
        g32 = step_hidden_f32(wts, kv, tokens, g32, k)
        ids, l64 = out["logits"][k]
        for b in np.nonzero(ok)[0]:
            l32 = g32[b] @ _f32(wts.embed[ids[b]]).T
            dl[k] = max(dl[k], float(np.abs(l32.astype(np.float64) - l64[b]).max()))
            if float(temperature) > 0:
                q32 = rules.target_probs(l32, temperature).astype(np.float64)
                qo = rules.target_probs(np.asarray(l64[b]).astype(np.float32), temperature).astype(np.float64)
                dq[k] = max(dq[k], float(np.abs(q32 - qo).max() / qo.max()))
        tokens = np.where(ok, out["draft"][:, k], 0)
    return dl, dq

