/*
 * specverify.h -- C ABI of the speculative-decoding verify step on MI355X (gfx950).
 *
 * The verify step of speculative / multi-token-prediction decoding: the target
 * model takes the last accepted token plus gamma drafted tokens, produces
 * next-token logits at all gamma+1 positions in one pass, and applies the
 * acceptance rule.
 *   - [Infra-ch8] AI-infra book, chapter 8 (speculative decoding), sections
 *     "a concrete example", "why one forward pass can verify several tokens",
 *     "why the output does not change", "where the extra token comes from".
 *   - [MTP-deep-dive] "Gemma 4 Multi-Token Prediction (MTP) deep dive", 2.2.
 *   - [Self-spec] "Self-speculative decoding: layer skip and rejection
 *     sampling", sections 3.1 (greedy), 3.2 (sampling), 3.3 (per-position
 *     randomness, KV trim).
 *   - [MTP-drafters] "Accelerating Gemma 4: faster inference with
 *     multi-token prediction drafters", sections 3.2 and 4.2.
 *
 * Notation.  B sequences, gamma drafts each (1 <= gamma <= 15), G1 = gamma+1
 * positions ("slots"), M = B*G1 rows, V vocabulary entries, d hidden size.
 * Slot i's prediction judges draft i (0-based: draft[b*gamma + i] is the token
 * after input slot i); slot gamma gives the bonus (N+1-th) token.
 *
 * Conventions shared by every entry point.
 *   Memory:   every array argument is a DEVICE pointer allocated and owned by
 *             the caller, row-major and densely packed, unless marked "host".
 *             The library never allocates, frees or retains caller memory.
 *   Workspace: scratch is caller-provided.  Call once with ws == NULL: the
 *             required size is written to *ws_bytes, nothing is launched, and
 *             SV_OK is returned.  Then call with ws != NULL and *ws_bytes >= that
 *             size (256-byte aligned).  A new workspace must be zero-filled
 *             (all of it) once before its first use; the library keeps state in
 *             it between calls (counters through which the workgroups of one
 *             launch hand work to each other, and a launch epoch), so keep using
 *             the same workspace or zero-fill a new one.  Every entry point keeps its
 *             scratch out of the first 4096 bytes (that state), so one workspace
 *             serves all of them.  The sampling step with a
 *             small batch runs as one kernel whose workgroups wait for each other
 *             (bounded; one workgroup per compute unit): if a wait gives up (about a
 *             second, e.g. on a device shared with other work; see
 *             SV_OPT_WAIT_LIMIT), the step reports every sequence invalid (see Data
 *             errors) and the next call on the workspace runs normally.  Only if
 *             some workgroup of such a step had not even run does the step mark the
 *             workspace, and later sampling calls on it report every sequence invalid
 *             until it is zero-filled.
 *   Streams:  stream is a hipStream_t (NULL = the null stream).  All work is
 *             enqueued on it and the call returns before it completes;
 *             outputs are valid once the caller synchronises the stream.
 *             Calls that share a workspace must not overlap in time.
 *   Errors:   a status code; nothing throws or aborts across the ABI.  Argument
 *             errors are detected on the host before anything is launched and
 *             leave the outputs untouched.  sv_last_error() returns a message
 *             for the calling thread.  Device faults surface at the caller's
 *             synchronisation as HIP errors.
 *   Data errors that need device values (out-of-range token or draft ids,
 *             a KV cache too short for the new positions) never read or write
 *             out of bounds: an out-of-range draft is rejected; a sequence
 *             with an out-of-range input token or an overfull cache gets
 *             n_accepted[b] = -1, tokens_out[b][*] = -1, and its cache length
 *             is left unchanged.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
  SV_OK = 0,
  SV_ERR_ARG = 1,          /* null pointer, gamma/B/T out of range, bad struct field */
  SV_ERR_DTYPE = 2,        /* unsupported dtype combination */
  SV_ERR_SHAPE = 3,        /* sizes the kernels do not support (e.g. d % 32 != 0) */
  SV_ERR_WORKSPACE = 4,    /* *ws_bytes smaller than required, or misaligned ws */
  SV_ERR_HIP = 5,          /* a HIP runtime call failed (no device, launch error) */
  SV_ERR_UNSUPPORTED = 6   /* valid request this library does not implement */
} sv_status;

/* The two range markers of each enumeration a caller passes in (sv_dtype,
 * sv_input_kind) make every int32 value a valid value of the type, so that a value the
 * library does not know is an error it reports (SV_ERR_DTYPE / SV_ERR_ARG), not undefined
 * behaviour in the C++ implementation; they also fix the type's size at 32 bits.  They
 * are not values to pass. */
typedef enum sv_dtype {
  SV_F32 = 0, SV_BF16 = 1,
  SV_DTYPE_RANGE_MIN_ = -2147483647 - 1, SV_DTYPE_RANGE_MAX_ = 2147483647
} sv_dtype;

/* What ``input`` holds:
 *   SV_IN_LOGITS  float32 [B, G1, V] target logits (the forward is skipped);
 *   SV_IN_HIDDEN  wdtype  [B, G1, d] final hidden states (LM head only);
 *   SV_IN_TOKENS  int32   [B, G1] token ids, slot 0 = last accepted token,
 *                 slots 1..gamma = the drafts (full decoder forward). */
typedef enum sv_input_kind {
  SV_IN_LOGITS = 0, SV_IN_HIDDEN = 1, SV_IN_TOKENS = 2,
  SV_INPUT_RANGE_MIN_ = -2147483647 - 1, SV_INPUT_RANGE_MAX_ = 2147483647
} sv_input_kind;

/* Target model; all pointers are device pointers except ``layers``.
 * n_layers == 0: LM head only (SV_IN_LOGITS / SV_IN_HIDDEN).
 * n_layers > 0: pre-norm decoder (SV_IN_TOKENS), weights bf16, matrices
 * row-major [out, in]:  per layer, in this order,
 *   attn_norm [d], wq [H*hd, d], wk [H*hd, d], wv [H*hd, d], wo [d, H*hd],
 *   ffn_norm [d], w_gate [d_ff, d], w_up [d_ff, d], w_down [d, d_ff].
 * RMSNorm x / sqrt(mean(x^2) + rms_eps) * g; rotary embedding (rotate-half
 * pairs (j, j + hd/2), angle pos * rope_theta^(-2j/hd)); causal softmax
 * attention with scale 1/sqrt(hd); SwiGLU SiLU(gate) * up. */
typedef struct sv_model {
  int32_t n_layers;
  int32_t d_model;             /* d; multiple of 32 */
  int32_t n_heads;
  int32_t head_dim;            /* 64 or 128 when n_layers > 0 */
  int32_t d_ff;                /* multiple of 32 */
  int32_t vocab;               /* V >= 2 */
  sv_dtype wdtype;             /* SV_BF16, or SV_F32 for an LM-head-only model */
  float rms_eps;
  float rope_theta;
  const void* embed;           /* [V, d] (n_layers > 0) */
  const void* const* layers;   /* HOST array of n_layers * 9 device pointers */
  const void* final_norm;      /* [d] (n_layers > 0) */
  const void* lm_head;         /* [V, d]; not read for SV_IN_LOGITS */
} sv_model;

/* KV cache of the decoder: bf16 [n_layers][B][n_heads][max_len][head_dim]
 * for K (after the rotary embedding) and V.  len: device int32 [B], the
 * number of valid positions per sequence.  The verify pass writes K/V of its
 * G1 new positions at len..len+gamma; see the commit rule of the entry points. */
typedef struct sv_kv_cache {
  void* k;
  void* v;
  int32_t max_len;
  int32_t* len;
} sv_kv_cache;

/* Logits of all G1 slots (steps a1-a3 of the verify pass).
 *   input/kind: as above.  kv: required for SV_IN_TOKENS (K/V of the new
 *   positions are written at len..len+gamma; len itself is NOT changed),
 *   ignored otherwise.  logits: out float32 [B, G1, V].
 * [Infra-ch8] "why one forward pass can verify several tokens": one pass over
 * L inputs yields L next-token predictions; the causal mask keeps slot i from
 * seeing later drafts. */
sv_status verify_forward(const sv_model* m, sv_input_kind kind, const void* input,
                         int32_t B, int32_t gamma, const sv_kv_cache* kv,
                         float* logits, void* ws, size_t* ws_bytes, void* stream);

/* Greedy verify: accept draft i while it equals the argmax of slot i (lowest
 * index on ties), stop at the first mismatch and emit the slot's argmax in its
 * place; if all gamma drafts match, emit slot gamma's argmax as the bonus.
 * [MTP-drafters] 3.2; [Self-spec] 3.1 (compare with the mode, not a
 * probability threshold); [Infra-ch8] "a concrete example".
 *   draft:      int32 [B, gamma]; may be NULL for SV_IN_TOKENS (then the
 *               drafts are input slots 1..gamma).
 *   kv:         SV_IN_TOKENS: required; after the pass len[b] += n_b + 1 on
 *               the device (the accepted drafts and the slot-0 token are now
 *               cached; K/V written beyond the new len are stale and will be
 *               overwritten next round; [Self-spec] 3.3).  Otherwise may be
 *               NULL; if given, only len is advanced.
 *   n_accepted: out int32 [B], accepted drafts 0..gamma (-1: see Data errors).
 *   tokens_out: out int32 [B, G1], emitted tokens: the n_b accepted drafts,
 *               then the correction or bonus token; -1 after those n_b + 1.
 *   logits_out: optional out float32 [B, G1, V] (NULL: kept in workspace).
 *   diag:       optional out float32 [B, G1] (NULL: not computed), how close each
 *               decision came to going the other way ([Self-spec] 3.1: the rule
 *               compares with the mode): diag[b][i] = the largest float32 logit of slot
 *               i minus the second largest (0 when two tokens share the maximum) for the
 *               decided slots i <= n_b; NaN past them and for invalid sequences.
 *               Computed by extra passes over the logits after the step (the step then
 *               keeps its logits in memory: in logits_out, else in the workspace). */
sv_status spec_verify_greedy(const sv_model* m, sv_input_kind kind, const void* input,
                             int32_t B, int32_t gamma, const int32_t* draft,
                             const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                             float* logits_out, float* diag, void* ws, size_t* ws_bytes, void* stream);

/* Speculative sampling verify: p_i = softmax(logits_i / T).  Draft i is
 * accepted iff u_i * q_i(x) < p_i(x), i.e. with probability min(1, p/q); at
 * the first rejection the slot's token is drawn from max(0, p - q) (from p if
 * that is zero everywhere); if all drafts are accepted the bonus is drawn
 * from p_gamma.  The output law equals the target's.
 * [MTP-deep-dive] 2.2; [Infra-ch8] "why the output does not change";
 * [Self-spec] 3.2, 3.3.
 *   q, q_dtype:  draft distributions [B, gamma, V], float32 or bf16, used as
 *                given (not renormalised).
 *   temperature: finite, >= 0; 0 applies the greedy rule exactly.
 *   seed, pos0:  the random stream.  pos0: device int64 [B], absolute position
 *                of slot 0.  Draws are Philox4x64-10 (Salmon et al., SC'11)
 *                with key (seed, 0) and counter (block, position, b, tag):
 *                the acceptance uniform of the token at absolute position P is
 *                word 0 of block 0, tag 0, u = (w >> 40) * 2^-24; the
 *                resampling noise of vocab entry v at position P is word v & 3
 *                of block v >> 2, tag 1, U = ((w >> 41) + 0.5) * 2^-23,
 *                Gumbel G = -log(-log U), token = argmax_v log r_v + G_v.
 *                The result is a pure function of (inputs, seed, pos0).
 *   diag:        optional out float32 [B, G1] (NULL: not computed; [Self-spec] 3.2):
 *                diag[b][i] = |u_i - p_i(x) / q_i(x)| (infinity when q_i(x) = 0) for
 *                the decided acceptance tests i <= min(n_b, gamma - 1), NaN for later
 *                slots; diag[b][gamma] = the gap between the two best scores
 *                log r_v + G_v of the final draw, in the class it took (the residual,
 *                or p); NaN rows for invalid sequences.  T = 0: as for the greedy rule.
 *   Other arguments as for spec_verify_greedy. */
sv_status spec_verify_sample(const sv_model* m, sv_input_kind kind, const void* input,
                             int32_t B, int32_t gamma, const int32_t* draft,
                             const void* q, sv_dtype q_dtype, float temperature,
                             uint64_t seed, const int64_t* pos0,
                             const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                             float* logits_out, float* diag, void* ws, size_t* ws_bytes, void* stream);

/* spec_verify_sample without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops, harnesses that forbid
 * allocation).  The same computation, outputs and bits as spec_verify_sample; its scratch
 * is a fixed array of 4 MiB in the library's device memory, one per device, held until
 * the process ends.  It makes no allocation and no memset: the array's counter block is
 * cleared by a fill kernel on the first call on each device, and every call leaves it
 * cleared.  All calls on one device share that array: calls that overlap in time on one
 * device race (serialise them, e.g. on one stream).  A request whose scratch would
 * exceed 4 MiB returns SV_ERR_UNSUPPORTED before anything is launched (the logits of the
 * unfused path for large batches need more: pass logits_out, or use spec_verify_sample
 * with a workspace; diag without logits_out needs a logits buffer too).  Arguments as for
 * spec_verify_sample. */
sv_status spec_verify_sample_noalloc(const sv_model* m, sv_input_kind kind, const void* input,
                                     int32_t B, int32_t gamma, const int32_t* draft,
                                     const void* q, sv_dtype q_dtype, float temperature,
                                     uint64_t seed, const int64_t* pos0,
                                     const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                                     float* logits_out, float* diag, void* stream);

/* Speculative sampling verify with the drafter's top-k / top-p filters applied alike to
 * the target ([Infra-ch8] "why the output does not change", [MTP-drafters] 5.2: the
 * sampling parameters must be handled by one rule in drafting and verifying;
 * [MTP-drafters] 3.1 for the filters; [MTP-deep-dive] 5.1 deploys with top_k 64,
 * top_p 0.95).  The target distribution of every slot becomes p~: softmax(logits / T)
 * restricted to the top_k largest logits (the lower index first on equal values), then
 * to the smallest prefix of those (in descending order) whose probability, renormalised
 * over the top_k set, reaches top_p, renormalised over the kept tokens (computed in
 * double precision, rounded once to float32).  The rule of spec_verify_sample then runs
 * on p~: accept iff u * q(x) < p~(x) (a filtered-out draft is rejected), the first
 * rejection draws from max(0, p~ - q) (p~ if that is zero), all accepted draws the
 * bonus from p~_gamma, with the same random stream.  The output law is p~.
 *   top_k: 1 .. 64 (SV_ERR_UNSUPPORTED otherwise); the vocabulary may hold at most
 *          4096 * floor(4096 / top_k) entries (262,144 at top_k 64).
 *   top_p: in (0, 1]; 1 keeps the whole top-k set.
 *   temperature: finite, >= 0; 0 applies the greedy rule exactly (the filters keep the
 *          argmax).
 *   q:     the drafter's distributions, filtered by the drafter with the same rule, used
 *          as given.
 *   Other arguments as for spec_verify_sample; logits_out, if given, receives the
 *   unfiltered float32 logits. */
sv_status spec_verify_sample_filtered(const sv_model* m, sv_input_kind kind, const void* input,
                                      int32_t B, int32_t gamma, const int32_t* draft,
                                      const void* q, sv_dtype q_dtype, float temperature,
                                      int32_t top_k, float top_p, uint64_t seed, const int64_t* pos0,
                                      const sv_kv_cache* kv, int32_t* n_accepted, int32_t* tokens_out,
                                      float* logits_out, void* ws, size_t* ws_bytes, void* stream);

/* The drafter's centroid-masked LM head ([X-thread] "Gemma 4's MTP", efficient embedder;
 * [MTP-deep-dive] 3.4 "centroids masking"): token embeddings grouped into clusters of
 * similar tokens, one representative embedding per cluster.  The hidden state scores
 * the clusters, the top_k clusters are kept, and exact token logits are computed only
 * for their member tokens (the pages quote 2048 clusters, 32 kept: about 4K of 262,144
 * tokens scored).  Ordered embeddings: cluster c holds the contiguous tokens
 * [c * cs, (c + 1) * cs), cs = vocab / n_clusters. */
typedef struct sv_masked_head {
  int32_t vocab;               /* V, a positive multiple of n_clusters */
  int32_t d_model;             /* d; multiple of 32 */
  int32_t n_clusters;          /* C, 1 .. 4096 */
  sv_dtype wdtype;             /* SV_BF16 */
  const void* embed;           /* [V, d] token embeddings (the tied LM head), cluster-ordered */
  const void* centroids;       /* [C, d] one representative embedding per cluster */
} sv_masked_head;

/* Masked drafter logits for M hidden states.
 *   hidden:         bf16 [M, d], 1 <= M <= 24.
 *   top_k:          clusters kept per row, 1 <= top_k <= C.
 *   clusters:       out int32 [M, top_k], the kept cluster ids in descending order of
 *                   their float32 cluster score, the lower id first on equal scores.
 *   logits:         out float32 [M, top_k * cs]; block j holds the logits of tokens
 *                   clusters[m, j] * cs + [0, cs).  Every other token is masked (not
 *                   scored).
 *   cluster_logits: optional out float32 [M, C] cluster scores (NULL: kept in the
 *                   workspace).
 * Workspace, streams and errors as above.  The result is a pure function of the
 * inputs. */
sv_status draft_masked_logits(const sv_masked_head* head, const void* hidden, int32_t M, int32_t top_k,
                              int32_t* clusters, float* logits, float* cluster_logits,
                              void* ws, size_t* ws_bytes, void* stream);

/* The MTP drafter: a small decoder attached to the target ([X-thread] "Gemma 4's MTP":
 * target activations, KV cache sharing, efficient embedder; [MTP-deep-dive] 3.1-3.4).
 * Each step joins the embedding of the current token (the target's table, d_model wide)
 * with a d_model-wide hidden state, [embedding, hidden], projects the pair down to
 * `hidden` (pre_proj), runs n_layers pre-norm decoder layers whose attention has query
 * projections only and reads keys and values from the target's cache, applies a final
 * RMSNorm and projects back up to d_model (post_proj).  The result, rounded to bf16, is
 * the next step's hidden state and the input of the LM head tied to the token table:
 * every token is scored, or with centroids given, the centroid-masked head (see
 * draft_masked_logits) scores the members of the top_k_clusters clusters only.
 * All weights bf16, row-major [out, in]. */
typedef struct sv_drafter {
  int32_t n_layers;            /* 1 .. 64 */
  int32_t d_model;             /* D: the target's hidden size; multiple of 32 */
  int32_t hidden;              /* H: the drafter's width; multiple of 32, <= 8192 */
  int32_t n_heads, head_dim;   /* query heads; head_dim 64 or 128 (that of the shared cache) */
  int32_t d_ff;                /* multiple of 32 */
  int32_t vocab;               /* V */
  float rms_eps, rope_theta;
  const void* embed;           /* [V, D] token table shared with the target; the tied LM head */
  const void* pre_proj;        /* [H, 2D] */
  const void* const* layers;   /* host array, 7 device pointers per layer: attn_norm [H],
                                  wq [n_heads*head_dim, H], wo [H, n_heads*head_dim],
                                  ffn_norm [H], w_gate [d_ff, H], w_up [d_ff, H], w_down [H, d_ff] */
  const void* final_norm;      /* [H] */
  const void* post_proj;       /* [D, H] */
  const void* centroids;       /* [n_clusters, D] or NULL (tied head over every token) */
  int32_t n_clusters;          /* V a multiple of it, <= 4096 (masked head) */
  int32_t top_k_clusters;      /* 1 .. 64 (masked head) */
} sv_drafter;

/* The target cache layers the drafter reads: k[l], v[l] (host arrays of n_layers device
 * pointers; layers may share one) each [B, n_heads, max_len, head_dim] bf16 with one
 * key/value head per query head; len: device int32 [B], the cached positions [0, len). */
typedef struct sv_shared_kv {
  const void* const* k;
  const void* const* v;
  int32_t max_len;
  const int32_t* len;
} sv_shared_kv;

/* gamma autoregressive drafter steps for B sequences, all on the device.
 *   last_token: device int32 [B], the last emitted token (position len[b]).
 *   h_target:   device bf16 [B, D], the target's last hidden state (the one that
 *               produced last_token's distribution).
 *   Step k (0-based) processes its token at position len + k (RoPE on the queries;
 *   every cached position [0, len) is visible, the cache is not written) and drafts
 *   the token of position len + k + 1.
 *   temperature > 0: q_k = softmax(logits / T) over the scored tokens (0 elsewhere),
 *     written to q (device [B, gamma, V], q_dtype SV_F32 or SV_BF16); the draft is
 *     argmax over scored v of log q_v + G_v with G_v = -log(-log U_v), U_v from
 *     Philox4x64-10 key (seed, 0), counter (v >> 2, position, b, 2), word v & 3,
 *     U = ((w >> 41) + 0.5) 2^-23 (the verify's sampling stream layout under its own
 *     tag), lower id first on ties.  These q feed spec_verify_sample with pos0 = len.
 *   temperature == 0: the draft is the argmax of the logits (lower id first); q is
 *     not written and may be NULL.
 *   draft: out device int32 [B, gamma].  A sequence whose len is outside [1, max_len]
 *     or whose last_token is no token gets drafts -1 and q rows of zeros.
 * B: 1 .. 24 with the masked head, 1 .. 64 with the tied head.  Workspace, streams and
 * errors as above. */
sv_status mtp_draft(const sv_drafter* dr, const sv_shared_kv* kv, int32_t B, int32_t gamma,
                    const int32_t* last_token, const void* h_target, float temperature, uint64_t seed,
                    int32_t* draft, void* q, sv_dtype q_dtype, void* ws, size_t* ws_bytes, void* stream);

/* Round policies around the verify step ([MTP-drafters] 6: adaptive draft length and
 * several draft candidates; [MTP-deep-dive] 5.1: the heuristic schedule; [Self-spec] 3.3:
 * each sequence keeps what it accepted).  All arrays are device arrays; each call
 * enqueues small kernels on the stream.
 *
 * round_pad_drafts: per-sequence draft length within a batch of G = gamma_max slots.
 *   gamma_b (int32 [B], in/out) is clamped to [1, G]; with tau > 0 it is cut further to
 *   the leading steps whose largest q is >= tau (at least 1; needs q).  Then the slots
 *   i >= gamma_b[b] are padded: draft[b, i] = -1, q[b, i, :] = 0 (q may be NULL for the
 *   greedy rule).  Verifying the padded batch gives each sequence exactly what verifying
 *   it alone with gamma_b drafts gives: the rule rejects at slot gamma_b at the latest
 *   (no id matches -1) and the residual there is max(0, p - 0) = p, the bonus
 *   distribution, drawn at the bonus's position.  ws as elsewhere (B * G floats when
 *   tau > 0, else none). */
sv_status round_pad_drafts(int32_t B, int32_t G, int32_t V, int32_t* gamma_b, int32_t* draft, void* q,
                           sv_dtype q_dtype, float tau, void* ws, size_t* ws_bytes, void* stream);

/* round_update_gamma: the heuristic schedule.  gamma_b[b] (in/out) becomes gamma_b + 2
 * when every draft was accepted (n_accepted[b] >= gamma_b[b]), else gamma_b - 1, kept
 * within [gamma_min, gamma_max]; a sequence with n_accepted < 0 (invalid) keeps it.
 * 1 <= gamma_min <= gamma_max <= 15. */
sv_status round_update_gamma(int32_t B, const int32_t* n_accepted, int32_t* gamma_b, int32_t gamma_min,
                             int32_t gamma_max, void* stream);

/* round_select_candidates: C draft candidates per sequence verified as rows b * C + c
 * of one batch (greedy rule); keeps the one with the most accepted drafts, the lower
 * index on ties: best[b] (may be NULL), n_out[b], tokens_out[b, 0..G1).  Under the
 * greedy rule every candidate's accepted prefix is the target's own argmax chain, so
 * the choice is lossless; under the sampling rule it is not (the best of several
 * independent verifications is biased), and this call is not meant for it. */
sv_status round_select_candidates(int32_t B, int32_t C, int32_t G1, const int32_t* n_accepted,
                                  const int32_t* tokens, int32_t* best, int32_t* n_out, int32_t* tokens_out,
                                  void* stream);

/* Process-wide options (every device, every later call).
 *   SV_OPT_WAIT_LIMIT: polls that each bounded wait between the workgroups of the
 *     fused sampling step makes before it gives up (default 1048576, about a second).
 *     A step whose wait gives up reports every sequence invalid; the workspace stays
 *     usable.  Small values force that path (tests of failure handling); value < 0
 *     restores the default.
 * Returns SV_ERR_ARG for an unknown option. */
typedef enum sv_option { SV_OPT_WAIT_LIMIT = 0 } sv_option;
sv_status sv_set_option(int32_t option, int64_t value);

/* Per-device choice of the fused step's load grouping, for callers that run the same
 * bf16 LM-head shape many times.  The fused verify kernel issues its weight loads in
 * items of 4, 6 or 8 16-byte loads per lane; which item size streams fastest depends on
 * the device (on some MI355X boards items of 6 leave the odd XCDs about 4 us behind,
 * on others items of 4 are 1-2 us slower).  sv_tune_verify times the fused greedy step
 * of this model at B x (gamma + 1) rows with each item size that divides the work
 * (three alternating rounds of eight launches on zero inputs; the timing does not depend
 * on the values) and keeps the faster one for this device and shape, for every later
 * call with that shape (greedy, sampling, noalloc).  The item size changes only the
 * grouping of the loads, not the summation order: logits and decisions are the same
 * bits with any item size.
 *   A setup call: it allocates and frees device memory (inputs, outputs, a workspace),
 *   synchronises the stream and must not be captured into a graph.  Models other than
 *   a bf16 LM head, or shapes without a fused step, are left as they are (SV_OK).
 *   Errors: SV_ERR_ARG / SV_ERR_SHAPE as for spec_verify_greedy; SV_ERR_HIP if an
 *   allocation or launch fails (the previous choice is kept).  Thread-safe.
 * sv_tuned_item returns the item size in use for that model and shape on the current
 * device (0: not tuned; the default order applies). */
sv_status sv_tune_verify(const sv_model* m, int32_t B, int32_t gamma, void* stream);
int32_t sv_tuned_item(const sv_model* m, int32_t B, int32_t gamma);

/* Library version (major * 10000 + minor * 100 + patch). */
int32_t sv_version(void);

/* Static string naming a status code. */
const char* sv_status_string(int32_t status);

/* Message describing the calling thread's most recent error ("" if none). */
const char* sv_last_error(void);

/* Kernel timing with HIP events recorded on the caller's stream around the
 * launches of one kernel class.  Classes: 0 = LM-head product (the dominant
 * kernel of the LM-head configurations; with a small batch it also applies the
 * rule and, for sampling, draws and commits: the whole step in one kernel),
 * 1 = decoder layers, 2 = acceptance tail (separate acceptance kernel,
 * resampler, where the batch is too large for the fused step).  sv_timing_enable(mask) records the
 * classes whose bit is set in mask (0 = off) and clears earlier records;
 * sv_timing_read synchronises on the recorded events and returns the summed
 * milliseconds and launch count of class ``which``.  Off by default; costs two
 * event records per timed launch while on. */
sv_status sv_timing_enable(int32_t mask);
sv_status sv_timing_read(int32_t which, double* total_ms, int64_t* count);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
