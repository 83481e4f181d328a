"""GPU parity of the batch / draft-length sweep (V = 262144, d = 4096, T = 1):
B in {1, 4, 16, 64} x gamma in {2, 4, 8}, through the C ABI against the oracle.

Same bar as the large-vocabulary configuration: decisions bit-exact except on
oracle-flagged sequences, logits within 1e-4 of each row's max |logit|.  The
shapes exercise both product kernels (resident X for small B * (gamma + 1),
K-chunked X and several row groups for the large batches), the fused and the
separate acceptance, and the fused sampler finish.
"""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import rules
from tests.gpu_util import compare_decisions, dev, dev_bf16, log, oracle_logits_bf16, row_rel_err

pytestmark = pytest.mark.gpu

CASES = [(B, g) for B in (1, 4, 16, 64) for g in (2, 4, 8)]


@pytest.fixture(scope="module")
def sweep():
    log("[config4] generating W [262144, 4096]")
    w = workloads.normal_bf16((262144, 4096), 0.02, workloads.input_seed(4), 0)
    return w, sv.lm_head_model(dev_bf16(w))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B", (1, 4, 16, 64))
def test_config4_sweep(sweep, B):
    w, model = sweep
    for g in (2, 4, 8):
        cs = workloads.batch_sweep(B=B, gamma=g, w=w)
        log(f"[config4] B={B} gamma={g}: oracle")
        ref = oracle_logits_bf16(cs.h, w)
        logits = torch.empty((B, g + 1, 262144), dtype=torch.float32, device="cuda")
        n, tok = sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, dev_bf16(cs.h), B, g, dev(cs.draft.astype(np.int32)),
                                       dev_bf16(cs.q), 1.0, cs.seed, dev(cs.pos0), logits_out=logits)
        torch.cuda.synchronize()
        err = row_rel_err(logits.cpu().numpy(), ref).max()
        qf = (cs.q.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
        n0, t0, fl = rules.verify_sample(ref, cs.draft, qf, 1.0, cs.seed, cs.pos0)
        m, f = compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"B={B} gamma={g}")
        log(f"[config4] B={B} gamma={g}: logit rel err {err:.2e}, mean emitted {np.mean(n0 + 1):.2f}, "
            f"mismatched {m} flagged {f}")
        assert err <= 1e-4
        if B == 16 and g == 4:
            ng, tg = sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, dev_bf16(cs.h), B, g,
                                           dev(cs.draft.astype(np.int32)))
            torch.cuda.synchronize()
            n1, t1, f1 = rules.verify_greedy(ref, cs.draft)
            compare_decisions(ng.cpu().numpy(), tg.cpu().numpy(), n1, t1, f1, "greedy B=16")
