"""Pins the oracle's reference decoder end to end: with its bf16 rounding points off
(``exact``), its logits for the gamma + 1 new positions equal those of the Llama
implementation in the ``transformers`` library run in float64 on the CPU, on small
random models with the same weights and KV cache (pre-norm RMSNorm, rotate-half RoPE,
causal attention over the cache plus the new positions, SwiGLU, untied LM head: the
architecture of [Infra-ch8] "why one forward pass can verify several tokens").  The
library keeps its RMSNorm in float32, so the bound is 1e-5 of each row's largest
logit, far below what any dropped term, sign or transposed operand produces."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from oracle import bf16 as obf16
from oracle import decoder as dec

transformers = pytest.importorskip("transformers")


def hf_model(c):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = LlamaConfig(vocab_size=c.vocab, hidden_size=c.d_model, intermediate_size=c.d_ff,
                      num_hidden_layers=c.n_layers, num_attention_heads=c.n_heads, num_key_value_heads=c.n_heads,
                      head_dim=c.head_dim, rms_norm_eps=c.rms_eps, rope_theta=c.rope_theta,
                      tie_word_embeddings=False, max_position_embeddings=8192, attention_bias=False, mlp_bias=False)
    cfg._attn_implementation = "eager"
    m = LlamaForCausalLM(cfg).to(torch.float64).eval()
    f = lambda a: torch.from_numpy(obf16.bf16_to_f64(a))
    with torch.no_grad():
        m.model.embed_tokens.weight.copy_(f(c.embed))
        for li, L in enumerate(c.layers):
            lay = m.model.layers[li]
            lay.input_layernorm.weight.copy_(f(L["attn_norm"]))
            lay.post_attention_layernorm.weight.copy_(f(L["ffn_norm"]))
            lay.self_attn.q_proj.weight.copy_(f(L["wq"]))
            lay.self_attn.k_proj.weight.copy_(f(L["wk"]))
            lay.self_attn.v_proj.weight.copy_(f(L["wv"]))
            lay.self_attn.o_proj.weight.copy_(f(L["wo"]))
            lay.mlp.gate_proj.weight.copy_(f(L["w_gate"]))
            lay.mlp.up_proj.weight.copy_(f(L["w_up"]))
            lay.mlp.down_proj.weight.copy_(f(L["w_down"]))
        m.model.norm.weight.copy_(f(c.final_norm))
        m.lm_head.weight.copy_(f(c.lm_head))
    return m


def hf_logits(c):
    from transformers.cache_utils import DynamicCache
    m = hf_model(c)
    L = int(c.length[0])
    assert np.all(c.length == L), "one cache length for every sequence"
    cache = DynamicCache()
    for li in range(c.n_layers):
        k = torch.from_numpy(obf16.bf16_to_f64(c.k_cache[li, :, :, :L, :]))
        v = torch.from_numpy(obf16.bf16_to_f64(c.v_cache[li, :, :, :L, :]))
        cache.update(k, v, li)
    B, G = c.tokens.shape
    pos = torch.arange(L, L + G, dtype=torch.long).repeat(B, 1)
    with torch.no_grad():
        out = m(input_ids=torch.from_numpy(c.tokens.astype(np.int64)), past_key_values=cache, position_ids=pos,
                cache_position=torch.arange(L, L + G, dtype=torch.long), use_cache=True)
    return out.logits.numpy()


def gains(c, seed):
    """Norm gains around 1 (bf16), so that a misapplied gain changes the logits."""
    rng = np.random.default_rng(seed)
    g = lambda: workloads.to_bf16_bits((1.0 + 0.25 * rng.standard_normal(c.d_model)).astype(np.float32))
    layers = [dict(L, attn_norm=g(), ffn_norm=g()) for L in c.layers]
    return dataclasses.replace(c, layers=layers, final_norm=g())


@pytest.mark.parametrize("hd,nh,ff,B,gamma,cache", [(64, 2, 256, 1, 4, 37), (128, 2, 384, 2, 3, 100),
                                                     (32, 4, 192, 1, 7, 0)])
def test_exact_oracle_equals_llama_reference(hd, nh, ff, B, gamma, cache):
    c = workloads.small_decoder_case(n_layers=2, d_model=nh * hd, n_heads=nh, head_dim=hd, d_ff=ff, vocab=300,
                                     cache_len=cache, B=B, gamma=gamma, std=0.08)
    c = gains(c, hd + ff)
    wts = dec.DecoderWeights(c.n_layers, c.d_model, c.n_heads, c.head_dim, c.d_ff, c.vocab, c.rms_eps, c.rope_theta,
                             c.embed, c.layers, c.final_norm, c.lm_head)
    kv = dec.KVCache(c.k_cache.copy(), c.v_cache.copy(), c.length.astype(np.int64))
    ours = dec.forward(wts, c.tokens, kv, exact=True)
    ref = hf_logits(c)
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    err = (np.abs(ours - ref) / scale).max()
    assert err < 1e-5, err
    # the rounding points of the default oracle move the logits by far more than the bound
    kv2 = dec.KVCache(c.k_cache.copy(), c.v_cache.copy(), c.length.astype(np.int64))
    rounded = dec.forward(wts, c.tokens, kv2)
    assert (np.abs(rounded - ref) / scale).max() > 10 * err
