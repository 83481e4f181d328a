"""GPU parity of the wide-batch LM-head product (sv_wide.hpp: M-tiles of up to 192 rows
by W tiles of 256 rows, W read once per M-tile) against the oracle, through the C ABI.

Shapes: the three tile sizes (4, 8 and 12 blocks of 16 rows) with partial last tiles,
one to four M-tiles, vocabularies that are not a multiple of the W tile (ragged last
tile, fewer W tiles than XCDs), K = 256 / 1536 / 4096, the product alone
(verify_forward) and with the rules (greedy, sampling; the acceptance launched by the
product's own path when M <= 20; up to 16 rows the streaming product runs), out-of-range
drafts.  Bar: logits within 1e-4 of
each row's largest |logit| (bf16 inputs, float32 accumulation); decisions bit-exact
except on oracle-flagged sequences."""
import numpy as np
import pytest
import torch

import accept_step_amd as sv
import workloads
from oracle import rules
from tests.gpu_util import compare_decisions, dev, dev_bf16, log, oracle_logits_bf16, row_rel_err

pytestmark = pytest.mark.gpu


def table(V, d, seed):
    rng = np.random.default_rng(seed)
    return workloads.to_bf16_bits((rng.standard_normal((V, d)) * (1.0 / np.sqrt(d))).astype(np.float32))


@pytest.mark.parametrize("B,gamma,V,d", [
    (7, 2, 1000, 256),      # M = 21: one 64-row tile, 4 W tiles (fewer than XCDs), ragged last W tile
    (16, 3, 2503, 1536),    # M = 64: exactly one 64-row tile
    (13, 4, 4099, 256),     # M = 65: a 128-row tile, partial
    (40, 4, 3000, 512),     # M = 200: two 192-row tiles (the second partial), L2-shared W
    (289, 1, 1024, 256),    # M = 578: four tiles of 192 rows, the last two rows
])
def test_product_matches_oracle(B, gamma, V, d):
    M = B * (gamma + 1)
    log(f"[wide] product M={M} V={V} d={d}")
    w = table(V, d, M + V + d)
    rng = np.random.default_rng(7 * M)
    h = workloads.to_bf16_bits(rng.standard_normal((B, gamma + 1, d)).astype(np.float32))
    model = sv.lm_head_model(dev_bf16(w))
    logits = torch.full((B, gamma + 1, V), float("nan"), dtype=torch.float32, device="cuda")
    sv.verify_forward(model, sv.SV_IN_HIDDEN, dev_bf16(h), B, gamma, logits=logits)
    torch.cuda.synchronize()
    ref = oracle_logits_bf16(h, w)
    err = row_rel_err(logits.cpu().numpy(), ref)
    log(f"[wide] M={M} V={V} d={d}: max rel err {err.max():.2e}")
    assert np.isfinite(logits.cpu().numpy()).all() and err.max() <= 1e-4


@pytest.mark.parametrize("V,d,B,gamma,T", [
    (20011, 1536, 4, 4, 1.0),    # M = 20 at d = 1536: the fused k-split step
    (20011, 4096, 4, 4, 1.0),    # M = 20 at d = 4096: X no longer fits that step; wide product + acceptance
    (20011, 4096, 3, 3, 0.0),    # M = 12, greedy: the streaming product (X resident), beside the wide one
    (9001, 1536, 40, 4, 1.0),    # M = 200: two tiles, separate acceptance and sampler
    (9001, 1536, 40, 4, 0.0),
    (4999, 256, 100, 2, 0.7),    # M = 300
])
def test_rules_on_wide_product(V, d, B, gamma, T):
    log(f"[wide] rules V={V} d={d} B={B} gamma={gamma} T={T}")
    rng = np.random.default_rng(V + B)
    w = table(V, d, V + d)
    h = workloads.to_bf16_bits(rng.standard_normal((B, gamma + 1, d)).astype(np.float32))
    lt = rules.f32_logits(oracle_logits_bf16(h[:, :gamma], w))
    draft, q = workloads.drafter(lt, rng.standard_normal((B, gamma, V)).astype(np.float32) * 0.7, T, rng)
    bad = rng.random((B, gamma)) < 0.05
    draft = np.where(bad, np.where(rng.random((B, gamma)) < 0.5, -2, V + 1), draft).astype(np.int32)
    pos0 = rng.integers(0, 9999, B).astype(np.int64)
    ref = oracle_logits_bf16(h, w)
    model = sv.lm_head_model(dev_bf16(w))
    logits = torch.empty((B, gamma + 1, V), dtype=torch.float32, device="cuda")
    if T == 0.0:
        n, tok = sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, dev_bf16(h), B, gamma, dev(draft), logits_out=logits)
        n0, t0, fl = rules.verify_greedy(ref, draft)
    else:
        qb = workloads.to_bf16_bits(q)
        qf = workloads.bf16_bits_to_f32(qb).astype(np.float64)
        n, tok = sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, dev_bf16(h), B, gamma, dev(draft), dev_bf16(qb), T,
                                       555, dev(pos0), logits_out=logits)
        n0, t0, fl = rules.verify_sample(ref, draft, qf, T, 555, pos0)
    torch.cuda.synchronize()
    err = row_rel_err(logits.cpu().numpy(), ref).max()
    m, f = compare_decisions(n.cpu().numpy(), tok.cpu().numpy(), n0, t0, fl, f"V={V} d={d} B={B} T={T}")
    log(f"[wide] V={V} d={d} B={B} gamma={gamma} T={T}: rel err {err:.2e}, n={n.cpu().numpy()[:8].tolist()}..., "
        f"mismatched {m} flagged {f}")
    assert err <= 1e-4
    # without logits_out the logits stay in the workspace: same decisions
    if T == 0.0:
        n2, tok2 = sv.spec_verify_greedy(model, sv.SV_IN_HIDDEN, dev_bf16(h), B, gamma, dev(draft))
    else:
        n2, tok2 = sv.spec_verify_sample(model, sv.SV_IN_HIDDEN, dev_bf16(h), B, gamma, dev(draft), dev_bf16(qb), T,
                                         555, dev(pos0))
    torch.cuda.synchronize()
    assert np.array_equal(n2.cpu().numpy(), n.cpu().numpy()) and np.array_equal(tok2.cpu().numpy(), tok.cpu().numpy())


def test_k_not_multiple_of_two_chunks_uses_the_fallback():
    """K = 384 (three chunks of 128): the wide product does not apply; the fallback's
    logits are still right at M = 100."""
    B, gamma, V, d = 20, 4, 3001, 384
    w = table(V, d, 3)
    h = workloads.to_bf16_bits(np.random.default_rng(3).standard_normal((B, gamma + 1, d)).astype(np.float32))
    logits = torch.empty((B, gamma + 1, V), dtype=torch.float32, device="cuda")
    sv.verify_forward(sv.lm_head_model(dev_bf16(w)), sv.SV_IN_HIDDEN, dev_bf16(h), B, gamma, logits=logits)
    torch.cuda.synchronize()
    assert row_rel_err(logits.cpu().numpy(), oracle_logits_bf16(h, w)).max() <= 1e-4
