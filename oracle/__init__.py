"""CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the ``accept_step_amd``
package, its HIP library, or the timed leg of ``bench.py``) may import, call or
execute anything in this package.  The only permitted users are ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``.

The oracle is a plain, slow, obviously correct restatement of what the verify
step computes, written from the pages' statement of the method:

* ``philox``      -- Philox4x64-10 counter-based generator (Salmon et al., SC'11),
                     the random stream keyed by (seed, sequence, position) that the
                     self-speculative decoding page, section 3.3, asks for.
* ``bf16``        -- bfloat16 <-> float conversion (round to nearest even).
* ``rules``       -- LM-head logits, row statistics, the greedy rule, the
                     sampling rule with residual resampling, and the bonus token.
* ``decoder``     -- a float64 reference decoder (RMSNorm, RoPE, causal attention
                     over a KV cache, SwiGLU) for the full-model verify forward.
* ``closed_form`` -- E[tokens per round], the law of the emitted count, and the
                     speedup model.

Every function cites the passage of the pages it follows by page title and
section.  Page titles used in citations:

* [MTP-drafters]  "Accelerating Gemma 4: faster inference with multi-token
                  prediction drafters" (blog).
* [X-thread]      Chinese summary of Google Gemma's X thread on the Gemma 4 drafters.
* [MTP-deep-dive] "Gemma 4 Multi-Token Prediction (MTP) deep dive: architecture,
                  performance limits and deployment".
* [Infra-ch8]     AI-infra book, chapter 8, "Speculative decoding: one forward
                  pass verifies several tokens".
* [Self-spec]     "Self-speculative decoding: layer skip and rejection sampling
                  for LLM inference acceleration".

Pin status of each function is recorded in its docstring ("pinned by ...").
The reference decoder is pinned end to end as well: without its bf16 rounding
points its logits equal those of the Llama implementation in the ``transformers``
library (float64, CPU) on small random models (tests/test_oracle_decoder_hf.py);
the rounding points themselves are the GPU's storage points, pinned by the
per-operation tests.  No published values exist for the random-init full-model
configuration itself.
"""
