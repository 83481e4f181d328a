"""HIP-graph capture of the verify step, the full-model verify and a drafter round.

Each entry point is captured once into a graph (torch.cuda.graph on the caller's
stream, after one eager warm-up call), then the graph is replayed several times with
new inputs copied into its buffers, and the same entry point is called eagerly with the
same workspace between replays.  Every replay must give the eager result for its inputs
bit for bit: the fused sampler's launch epoch and the last-workgroup counters live in
the workspace and are advanced or reset on the device, never from the host, and no
entry point records a memset into the graph.  The eager results are those the parity
tests check against the oracle; this file checks only replay against eager."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from tests.gpu_util import dev, dev_bf16, log
from tests.test_gpu_decoder import gpu_model
from tests.test_gpu_drafter import device_drafter

pytestmark = pytest.mark.gpu

REPLAYS = 6


def capture(fn):
    """Warm up ``fn`` once on a side stream, then capture it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def load(static, values):
    for t, v in zip(static, values):
        t.copy_(v)


def same(a, b, label):
    a, b = a.cpu(), b.cpu()
    assert torch.equal(a, b), f"{label}: replay {a.flatten()[:12].tolist()} eager {b.flatten()[:12].tolist()}"


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_lm_head_verify_replays(T):
    """Hidden-state input, V = 65536, d = 1536, B = 2, gamma = 4: the fused one-launch
    step (greedy rule at T = 0 with its last-workgroup counters; the sampling rule at
    T = 1 with its epoch-tagged hand-offs)."""
    B, G = 2, 4
    cases = [workloads.lm_head_case(65536, 1536, B, G, max(T, 1.0), 1.0, 3, variant=21 + i) for i in range(3)]
    w = dev_bf16(cases[0].w)
    model = sv.lm_head_model(w)
    ws = sv.Workspace()
    inputs = [(dev_bf16(c.h), dev(c.draft.astype(np.int32)), dev_bf16(c.q),
               dev(np.arange(B, dtype=np.int64) * 1000 + 17 * i)) for i, c in enumerate(cases)]
    h_s, d_s, q_s, p_s = (x.clone() for x in inputs[0])
    n_s = torch.empty(B, dtype=torch.int32, device="cuda")
    t_s = torch.empty((B, G + 1), dtype=torch.int32, device="cuda")
    seed = cases[0].seed

    def call(h, d, q, p, out=None):
        if T == 0.0:
            return sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, h, B, G, d, out=out, ws=ws)
        return sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, h, B, G, d, q, T, seed, p, out=out, ws=ws)

    ref = [tuple(x.clone() for x in call(*inp)) for inp in inputs]
    torch.cuda.synchronize()
    g = capture(lambda: call(h_s, d_s, q_s, p_s, out=(n_s, t_s)))
    for r in range(REPLAYS):
        i = r % 3
        load((h_s, d_s, q_s, p_s), inputs[i])
        g.replay()
        torch.cuda.synchronize()
        same(n_s, ref[i][0], f"T={T} replay {r} n")
        same(t_s, ref[i][1], f"T={T} replay {r} tokens")
        n_e, t_e = call(*inputs[(i + 1) % 3])        # eager work between replays
        torch.cuda.synchronize()
        same(n_e, ref[(i + 1) % 3][0], f"T={T} eager after replay {r}")
        same(t_e, ref[(i + 1) % 3][1], f"T={T} eager after replay {r}")
    log(f"[graph] lm head T={T}: {REPLAYS} replays equal eager; n per input {[x[0].tolist() for x in ref]}")


def test_full_model_verify_replays():
    """Token input through the small decoder with its KV cache (B = 2, gamma = 3,
    sampling): each replay starts from the same cached lengths (restored before it) and
    must append the same K/V rows, emit the same tokens and advance the lengths alike."""
    c = workloads.small_decoder_case(B=2, gamma=3)
    B, G1 = c.tokens.shape
    G = G1 - 1
    model, kv = gpu_model(c)
    ws = sv.Workspace()
    len0 = kv.length.clone()
    k0, v0 = kv.k.clone(), kv.v.clone()
    rng = np.random.default_rng(5)
    toks = [dev(c.tokens.astype(np.int32))] + [dev(rng.integers(0, c.vocab, (B, G1)).astype(np.int32)) for _ in range(2)]
    q = dev(c.q.astype(np.float32))
    pos = dev(c.length.astype(np.int64))
    tok_s = toks[0].clone()
    n_s = torch.empty(B, dtype=torch.int32, device="cuda")
    t_s = torch.empty((B, G1), dtype=torch.int32, device="cuda")

    def restore():
        kv.length.copy_(len0)
        kv.k.copy_(k0)
        kv.v.copy_(v0)

    def call(tok, out=None):
        return sv.spec_verify_sample(model, sv.SV_IN_TOKENS, tok, B, G, None, q, 1.0, c.seed, pos, kv=kv, out=out,
                                     ws=ws)

    ref = []
    for t in toks:
        restore()
        n, tk = call(t)
        torch.cuda.synchronize()
        ref.append((n.clone(), tk.clone(), kv.length.clone(), kv.k.clone(), kv.v.clone()))
    restore()
    g = capture(lambda: call(tok_s, out=(n_s, t_s)))
    for r in range(REPLAYS):
        i = r % 3
        restore()
        tok_s.copy_(toks[i])
        g.replay()
        torch.cuda.synchronize()
        same(n_s, ref[i][0], f"replay {r} n")
        same(t_s, ref[i][1], f"replay {r} tokens")
        same(kv.length, ref[i][2], f"replay {r} lengths")
        same(kv.k, ref[i][3], f"replay {r} K cache")
        same(kv.v, ref[i][4], f"replay {r} V cache")
    log(f"[graph] full model: {REPLAYS} replays equal eager; n per input {[x[0].tolist() for x in ref]}")


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_drafter_round_replays(T):
    """A gamma = 4 drafter round (V = 8192, D = 512, H = 256, four layers, masked head
    with 32 of 128 clusters kept, B = 2) with new last tokens and target states per
    replay."""
    c = workloads.drafter_case(V=8192, D=512, H=256, n_layers=4, n_heads=4, head_dim=128, d_ff=512, C=128, top_k=32,
                               B=2, length=[100, 1000], variant=3)
    dr, kv = device_drafter(c, True)
    ws = sv.Workspace()
    rng = np.random.default_rng(9)
    inputs = [(dev(c.last_token.astype(np.int32)), dev_bf16(c.h_target))]
    for _ in range(2):
        hb = workloads.to_bf16_bits(rng.standard_normal(c.h_target.shape).astype(np.float32))
        inputs.append((dev(rng.integers(0, c.vocab, c.last_token.shape).astype(np.int32)), dev_bf16(hb)))
    t_s, h_s = (x.clone() for x in inputs[0])
    d_s = torch.empty((2, 4), dtype=torch.int32, device="cuda")
    q_s = torch.empty((2, 4, c.vocab), dtype=torch.float32, device="cuda") if T > 0 else None

    def call(t, h, draft=None, q=None):
        return sv.mtp_draft(dr, kv, t, h, 4, T, c.seed, draft=draft, q=q, ws=ws)

    ref = []
    for inp in inputs:
        d, q = call(*inp)
        torch.cuda.synchronize()
        ref.append((d.clone(), None if q is None else q.clone()))
    g = capture(lambda: call(t_s, h_s, d_s, q_s))
    for r in range(REPLAYS):
        i = r % 3
        load((t_s, h_s), inputs[i])
        g.replay()
        torch.cuda.synchronize()
        same(d_s, ref[i][0], f"T={T} replay {r} drafts")
        if q_s is not None:
            same(q_s, ref[i][1], f"T={T} replay {r} q")
        d_e, _ = call(*inputs[(i + 1) % 3])
        torch.cuda.synchronize()
        same(d_e, ref[(i + 1) % 3][0], f"T={T} eager after replay {r}")
    log(f"[graph] drafter T={T}: {REPLAYS} replays equal eager; drafts {[x[0].tolist() for x in ref]}")
