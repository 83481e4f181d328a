"""spec_verify_sample_noalloc (the allocation-free entry point) against
spec_verify_sample with a caller workspace: the same n_accepted, tokens and logits, bit
for bit, on two calls in a row with the second one smaller (and more calls after, so the
launch epoch kept in the fixed scratch array advances), at the large-vocabulary shape
(one fused launch) and on a small ragged one; an oversized request is refused before
anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from tests.gpu_util import dev, dev_bf16, log

pytestmark = pytest.mark.gpu


def make_case(V, d, B, gamma, T, seed):
    rng = np.random.default_rng(seed)
    w = workloads.to_bf16_bits((rng.standard_normal((V, d)) * 0.05).astype(np.float32))
    h = workloads.to_bf16_bits(rng.standard_normal((B, gamma + 1, d)).astype(np.float32))
    draft = rng.integers(0, V, (B, gamma)).astype(np.int32)
    q = rng.random((B, gamma, V)).astype(np.float32)
    q /= q.sum(-1, keepdims=True)
    return dict(model=sv.lm_head_model(dev_bf16(w)), h=dev_bf16(h), draft=dev(draft),
                q=dev_bf16(workloads.to_bf16_bits(q)), pos0=dev(rng.integers(0, 9000, B).astype(np.int64)),
                B=B, gamma=gamma, V=V, T=T, seed=777 + seed)


def both(c, ws):
    logits_a = torch.empty((c["B"], c["gamma"] + 1, c["V"]), dtype=torch.float32, device="cuda")
    logits_b = torch.empty_like(logits_a)
    args = (c["model"], sv.SV_IN_HIDDEN, c["h"], c["B"], c["gamma"], c["draft"], c["q"], c["T"], c["seed"], c["pos0"])
    na, ta = sv.spec_verify_sample(*args, logits_out=logits_a, ws=ws)
    nb, tb = sv.spec_verify_sample_noalloc(*args, logits_out=logits_b)
    # and without logits_out (the fused step keeps them on chip)
    nc, tc = sv.spec_verify_sample_noalloc(*args)
    torch.cuda.synchronize()
    return (na, ta, logits_a), (nb, tb, logits_b), (nc, tc)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_noalloc_matches_workspace_entry_point(T):
    ws = sv.Workspace()
    big = make_case(262144, 1536, 1, 4, T, 1)
    small = make_case(20011, 256, 3, 3, T, 2)        # the second call is smaller (and ragged)
    for label, c in (("big", big), ("small", small), ("big again", big), ("small again", small)):
        (na, ta, la), (nb, tb, lb), (nc, tc) = both(c, ws)
        log(f"[noalloc] {label} T={T}: n={na.cpu().numpy().tolist()} / {nb.cpu().numpy().tolist()}")
        assert torch.equal(na, nb) and torch.equal(ta, tb), label
        assert torch.equal(na, nc) and torch.equal(ta, tc), label
        assert torch.equal(la.view(torch.int32), lb.view(torch.int32)), label
        assert (na >= 0).all(), label


def test_noalloc_refuses_oversized_requests():
    """M = 576 rows without logits_out needs the unfused path's logits buffer (hundreds of
    MB): refused with SV_ERR_UNSUPPORTED, outputs untouched."""
    c = make_case(65536, 256, 64, 8, 1.0, 3)
    n = torch.full((64,), 123, dtype=torch.int32, device="cuda")
    t = torch.full((64, 9), 123, dtype=torch.int32, device="cuda")
    with pytest.raises(sv.VerifyError) as e:
        sv.spec_verify_sample_noalloc(c["model"], sv.SV_IN_HIDDEN, c["h"], 64, 8, c["draft"], c["q"], 1.0, 5,
                                      c["pos0"], out=(n, t))
    torch.cuda.synchronize()
    assert e.value.status == 6 and b"scratch" in sv.library().sv_last_error()
    assert (n == 123).all() and (t == 123).all()
