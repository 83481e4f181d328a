"""The float32 model behind the full-model logit bound (tests/decoder_bounds.py) computes
the oracle's recipe: on narrow decoders, where few bf16 rounding points flip, it agrees
with the float64 oracle (oracle/decoder.forward) to float32 level, so a dropped term, a
wrong operand or a missing rounding point in it would show as a large drift here instead
of loosening the bound."""
import numpy as np
import pytest

import workloads
from oracle import decoder as dec
from tests import decoder_bounds as dbnd


@pytest.mark.parametrize("n_layers,d,H,hd,ff,B,gamma", [(2, 128, 2, 64, 256, 2, 3), (1, 256, 2, 128, 512, 1, 4)])
def test_float32_model_follows_the_oracle(n_layers, d, H, hd, ff, B, gamma):
    c = workloads.small_decoder_case(n_layers=n_layers, d_model=d, n_heads=H, head_dim=hd, d_ff=ff, vocab=300,
                                     cache_len=20, B=B, gamma=gamma, std=0.1)
    wts = dec.DecoderWeights(c.n_layers, c.d_model, c.n_heads, c.head_dim, c.d_ff, c.vocab, c.rms_eps, c.rope_theta,
                             c.embed, c.layers, c.final_norm, c.lm_head)
    kv = dec.KVCache(c.k_cache.copy(), c.v_cache.copy(), c.length.astype(np.int64))
    ref = dec.forward(wts, c.tokens, kv)
    l32 = dbnd.forward_f32(wts, c.tokens, c.k_cache, c.v_cache, c.length)
    drift = dbnd.row_rel(l32, ref)
    assert drift.max() < 1e-2, drift
    assert np.median(drift) < 1e-5, drift          # most rows: no bf16 flip at all
    assert dbnd.logit_bound(l32, ref) == dbnd.BASE_TOL
