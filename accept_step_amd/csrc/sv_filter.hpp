// sv_filter.hpp -- speculative sampling verify with the top-k / top-p filters applied to
// the target distribution exactly as the drafter applied them to q (gfx950).
//
// [Infra-ch8] "why the output does not change" and [MTP-drafters] 5.2 (problem 2): the
// temperature, top-k and top-p handling must be one rule in drafting and verifying;
// [MTP-drafters] 3.1 for the filters; [MTP-deep-dive] 5.1 deploys with top_k 64,
// top_p 0.95.  The filtered target p~ keeps the top_k largest logits (the lower index
// first on equal values), then the smallest prefix of them whose renormalised
// probability reaches top_p, renormalised; the acceptance test, the residual
// max(0, p~ - q) and the bonus draw are those of the plain sampling rule (sv_accept.hpp)
// on p~.  Launches after the logits: the top_k of every 4096-logit chunk of every row,
// the top_k of each row's chunk candidates with the top-p cut (double precision), and
// the rule, one wavefront per sequence (the kept tokens, at most 64, fit its lanes).
#pragma once

#include "sv_accept.hpp"
#include "sv_head.hpp"
#include "sv_masked.hpp"

namespace sv {

constexpr int FILT_CHUNK = MASK_MAX_CLUSTERS;   // logits per chunk of the first stage

struct FiltArgs {
  const float* logits;        // [M, V] float32
  int M, V, G1, gamma, B, top_k, nch;
  double inv_t;               // 1 / temperature
  double top_p;
  unsigned long long* cand;   // [M][nch][top_k] chunk candidates (descending keys, 0 = none)
  int* kept_n;                // [M] tokens kept per row
  int* kept_id;               // [M][top_k] their vocabulary indices, in descending probability
  float* kept_p;              // [M][top_k] their filtered probabilities (float32)
  // the rule
  const int* draft;           // drafted token of (b, i) at draft[b * draft_stride + draft_offset + i]
  int draft_stride, draft_offset;
  const void* q;              // [B, gamma, V]
  int q_bf16;
  const int64_t* pos0;        // [B]
  const int* invalid;         // [B] or null
  int* len;                   // [B] or null
  uint64_t seed;
  int* n_accepted;            // [B]
  int* tokens_out;            // [B, G1]
};

// The float a score-order key was made from (inverse of the order map of cluster_key).
__device__ __forceinline__ float key_score(unsigned long long key) {
  const unsigned o = unsigned(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Stage 1: the top_k keys (logit order, complemented vocabulary index) of chunk
// blockIdx.x of row blockIdx.y.  256 threads.
__global__ __launch_bounds__(256) void k_chunk_topk(FiltArgs a) {
  constexpr int PER = FILT_CHUNK / 256;
  const int ch = blockIdx.x, m = blockIdx.y, t = threadIdx.x;
  unsigned long long key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = ch * FILT_CHUNK + t + 256 * u;
    key[u] = v < a.V ? cluster_key(a.logits[size_t(m) * a.V + v], v) : 0ull;
  }
  const unsigned long long kv = block_top_keys(key, a.top_k);
  if (t < a.top_k) a.cand[(size_t(m) * a.nch + ch) * a.top_k + t] = kv;
}

// Stage 2: row blockIdx.x.  The top_k of its nch * top_k chunk candidates; then, one lane
// per kept token in descending order, e_j = exp((l_j - l_0) / T) and p_j = e_j / sum e
// in double precision, a lane keeps its token while the cumulative probability before
// it is below top_p, and the kept probabilities are renormalised and rounded once to
// float32.  256 threads.
__global__ __launch_bounds__(256) void k_row_filter(FiltArgs a) {
  constexpr int PER = MASK_MAX_CLUSTERS / 256;
  const int m = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const int n = a.nch * a.top_k;
  unsigned long long key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = t + 256 * u;
    key[u] = i < n ? a.cand[size_t(m) * n + i] : 0ull;
  }
  const unsigned long long kv = block_top_keys(key, a.top_k);
  if (t >= 64) return;
  const bool real = lane < a.top_k && kv != 0ull;
  const float l = real ? key_score(kv) : 0.0f;
  const double l0 = double(__int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(l))));
  const double e = real ? exp((double(l) - l0) * a.inv_t) : 0.0;
  double sum = e;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
  const double pk = e / sum;
  double cum = pk;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double v = __shfl_up(cum, o);
    if (lane >= o) cum += v;
  }
  double before = __shfl_up(cum, 1);                 // the predecessors' probability
  if (lane == 0) before = 0.0;
  const bool keep = real && before < a.top_p;
  double mass = keep ? pk : 0.0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mass += __shfl_xor(mass, o);
  const int J = __popcll(__ballot(keep));
  if (lane == 0) a.kept_n[m] = J;
  if (lane < a.top_k) {
    a.kept_id[size_t(m) * a.top_k + lane] = keep ? int(0xffffffffu - unsigned(kv)) : -1;
    a.kept_p[size_t(m) * a.top_k + lane] = keep ? float(pk / mass) : 0.0f;
  }
}

__device__ __forceinline__ float filt_q(const FiltArgs& a, size_t idx) {
  return a.q_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.q)[idx]) : reinterpret_cast<const float*>(a.q)[idx];
}

// Stage 3: sequence blockIdx.x, one wavefront.  Lane i < gamma tests draft i: p~(x) from
// its slot's kept list (0 if x was filtered out), accept iff u * q(x) < p~(x) with the
// acceptance uniform of position pos0 + i + 1; n = the first rejection.  Then lane j
// takes kept token j of slot n: r_j = max(0, p~_j - q_n(id_j)) (p~_j when every draft
// was accepted, or when that is zero for every kept token), score log r_j + G with the
// Gumbel noise of id_j at position pos0 + n + 1, and the largest (score, lower id) wins.
// Commit as the plain rule: n, the tokens, len += n + 1.
__global__ __launch_bounds__(64) void k_filtered_rule(FiltArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int G1 = a.G1, gamma = a.gamma, K = a.top_k;
  const bool bad = a.invalid && a.invalid[b];
  const int64_t p0 = a.pos0[b];
  bool ok = true;
  int x = -1;
  if (lane < gamma) {
    x = a.draft[size_t(b) * a.draft_stride + a.draft_offset + lane];
    const int row = b * G1 + lane;
    float px = 0.0f, qx = 0.0f;
    if (x >= 0 && x < a.V) {
      const int J = a.kept_n[row];
      for (int j = 0; j < J; ++j)
        if (a.kept_id[size_t(row) * K + j] == x) px = a.kept_p[size_t(row) * K + j];
      qx = filt_q(a, (size_t(b) * gamma + lane) * a.V + x);
    }
    const float u = accept_uniform(a.seed, uint64_t(b), uint64_t(p0 + lane + 1));
    ok = double(u) * double(qx) < double(px);
  }
  const unsigned long long rej = __ballot(lane < gamma && !ok);
  const int n = rej ? __ffsll(rej) - 1 : gamma;
  const int rown = b * G1 + n;
  const int J = a.kept_n[rown];
  const bool mine = lane < J;
  const int id = mine ? a.kept_id[size_t(rown) * K + lane] : 0;
  const float pj = mine ? a.kept_p[size_t(rown) * K + lane] : 0.0f;
  float r = pj;
  if (n < gamma && mine) r = fmaxf(pj - filt_q(a, (size_t(b) * gamma + n) * a.V + id), 0.0f);
  if (!__any(mine && r > 0.0f)) r = pj;
  unsigned long long key = 0ull;
  if (mine && r > 0.0f) {
    float G[4];
    gumbel4(a.seed, b, uint64_t(p0 + n + 1), id & ~3, G);
    float g = G[0];
#pragma unroll
    for (int e = 1; e < 4; ++e)
      if ((id & 3) == e) g = G[e];
    key = win_key(false, __logf(r) + g, id);
  }
  key = wave_allmax_u64(key);
  const int tok = key ? win_index(key) : -1;
  const int nn = bad ? -1 : n;
  if (lane < G1) {
    int tv = -1;
    if (nn >= 0 && lane < nn) tv = x;
    else if (nn >= 0 && lane == nn) tv = tok;
    a.tokens_out[size_t(b) * G1 + lane] = tv;
  }
  if (lane == 0) {
    a.n_accepted[b] = nn;
    if (a.len && nn >= 0) a.len[b] += nn + 1;
  }
}

}  // namespace sv
