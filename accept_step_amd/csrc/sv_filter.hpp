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
// on p~.  One launch after the logits: the top_k of every 4096-logit chunk of every row,
// then (last workgroup of a row) the top_k of the row's chunk candidates with the top-p
// cut in double precision, then (last row) the rule, one wavefront per sequence (the
// kept tokens, at most 64, fit its lanes).
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
  int* kept_id;               // [M][top_k] kept tokens' vocabulary indices in descending
                              // probability, -1 past the last kept one
  float* kept_p;              // [M][top_k] their filtered probabilities (float32)
  float* kept_q;              // [M][top_k] q of the row's slot at them (drafted slots)
  float* dpx;                 // [M] p~ at the slot's draft (drafted slots)
  float* dqx;                 // [M] q at the slot's draft
  unsigned* counters;         // the workspace's counter block
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

// The fused launch hands work on through one-shot counters in lines 19-31 of the
// workspace's counter block (zero before first use, left zero): row m counts on word
// FILT_CNT_ROW0 + 32 (c % 12) + c / 12 with c = m % FILT_ROW_COUNTERS (rows sharing a
// counter are merged together), and FILT_CNT_ROWS counts the finished row groups.
constexpr int FILT_CNT_ROWS = 19 * CNT_LINE, FILT_CNT_ROW0 = 20 * CNT_LINE;
constexpr int FILT_ROW_COUNTERS = 12 * CNT_LINE;

__device__ __forceinline__ void store_coherent_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float filt_q(const FiltArgs& a, size_t idx) {
  return a.q_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.q)[idx]) : reinterpret_cast<const float*>(a.q)[idx];
}

// Row m's merge, by one workgroup of 256 threads: the top_k of its nch * top_k chunk
// candidates, then, one lane of wavefront 0 per kept token in descending order,
// e_j = exp((l_j - l_0) / T) and p_j = e_j / sum e in double precision; a lane keeps its
// token while the probability of its predecessors is below top_p, and the kept
// probabilities are renormalised and rounded once to float32.  For a drafted slot
// (i = m mod (gamma+1) < gamma) it also records q at the kept tokens, and p~ and q at
// the draft (p~ = 0 when the draft was filtered out or is no token).
__device__ void filt_row(const FiltArgs& a, SelScratch& sel, int m) {
  constexpr int PER = MASK_MAX_CLUSTERS / 256;
  const int t = threadIdx.x, lane = t & 63;
  const int b = m / a.G1, i = m - b * a.G1;
  const bool drafted = i < a.gamma;
  int x = -1;
  float qx = 0.0f;
  if (drafted && t == 0) {
    x = a.draft[size_t(b) * a.draft_stride + a.draft_offset + i];
    if (x >= 0 && x < a.V) qx = filt_q(a, (size_t(b) * a.gamma + i) * a.V + x);
  }
  const int n = a.nch * a.top_k;
  unsigned long long key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int j = t + 256 * u;
    key[u] = j < n ? a.cand[size_t(m) * n + j] : 0ull;
  }
  const unsigned long long kv = block_top_keys(sel, key, a.top_k);
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
  const int id = keep ? int(0xffffffffu - unsigned(kv)) : -1;
  const float p = keep ? float(pk / mass) : 0.0f;
  if (lane < a.top_k) {
    store_coherent(&a.kept_id[size_t(m) * a.top_k + lane], id);
    store_coherent(&a.kept_p[size_t(m) * a.top_k + lane], p);
  }
  if (drafted) {
    if (lane < a.top_k)
      store_coherent(&a.kept_q[size_t(m) * a.top_k + lane], keep ? filt_q(a, (size_t(b) * a.gamma + i) * a.V + id) : 0.0f);
    const int xd = __builtin_amdgcn_readfirstlane(x);
    const unsigned long long hit = __ballot(xd >= 0 && id == xd);
    const float px = hit ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p), __ffsll(hit) - 1)) : 0.0f;
    if (lane == 0) {
      store_coherent(&a.dpx[m], px);
      store_coherent(&a.dqx[m], qx);
    }
  }
}

// The rule for sequence b, one wavefront, in one round of loads: lane i < gamma takes
// draft i with p~ and q at it; lane j holds kept entry j of every slot (id, p~, q).
// Draft i is accepted iff u * q(x_i) < p~(x_i), with u the acceptance uniform of
// position pos0 + i + 1; n = the first rejection.  Lane j then scores kept token j of
// slot n: r_j = max(0, p~_j - q_n(id_j)) (p~_j when every draft was accepted, or when
// that is zero for every kept token), log r_j + G with the Gumbel noise of id_j at
// position pos0 + n + 1; the largest (score, lower id) wins.  Commit as the plain rule:
// n, the tokens, len += n + 1.
__device__ void filt_rule(const FiltArgs& a, int b) {
  constexpr int GMAX = 16;
  const int lane = threadIdx.x & 63;
  const int G1 = a.G1, gamma = a.gamma, K = a.top_k;
  const size_t rb = size_t(b) * G1;
  int kid[GMAX];
  float kp[GMAX], kq[GMAX - 1];
#pragma unroll
  for (int i = 0; i < GMAX; ++i) {
    kid[i] = -1;
    kp[i] = 0.0f;
    if (i < GMAX - 1) kq[i] = 0.0f;
    if (i < G1 && lane < K) {
      kid[i] = a.kept_id[(rb + i) * K + lane];
      kp[i] = a.kept_p[(rb + i) * K + lane];
      if (i < GMAX - 1 && i < gamma) kq[i] = a.kept_q[(rb + i) * K + lane];
    }
  }
  int x = -1;
  float px = 0.0f, qx = 0.0f;
  if (lane < gamma) {
    x = a.draft[size_t(b) * a.draft_stride + a.draft_offset + lane];
    px = a.dpx[rb + lane];
    qx = a.dqx[rb + lane];
  }
  const int64_t p0 = a.pos0[b];
  bool ok = true;
  if (lane < gamma) {
    const float u = accept_uniform(a.seed, uint64_t(b), uint64_t(p0 + lane + 1));
    ok = double(u) * double(qx) < double(px);
  }
  const unsigned long long rej = __ballot(lane < gamma && !ok);
  const int n = rej ? __ffsll(rej) - 1 : gamma;
  int id = -1;
  float pj = 0.0f, qn = 0.0f;
#pragma unroll
  for (int i = 0; i < GMAX; ++i)
    if (i == n) {
      id = kid[i];
      pj = kp[i];
      if (i < GMAX - 1) qn = kq[i];
    }
  const bool mine = id >= 0;
  float r = pj;
  if (n < gamma && mine) r = fmaxf(pj - qn, 0.0f);
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
  const bool bad = a.invalid && a.invalid[b];
  const int nn = bad ? -1 : n;
  if (lane < G1) {
    int tv = -1;
    if (nn >= 0 && lane < nn) tv = x;
    else if (nn >= 0 && lane == nn) tv = tok;
    a.tokens_out[rb + lane] = tv;
  }
  if (lane == 0) {
    a.n_accepted[b] = nn;
    if (a.len && nn >= 0) a.len[b] += nn + 1;
  }
}

// One launch, grid (nch, M), 256 threads.  Workgroup (ch, m) takes the top_k keys
// (logit order, complemented vocabulary index) of the 4096-logit chunk ch of row m and
// hands them on; the last workgroup of a row group merges its rows (filt_row); the last
// row group runs the rule for every sequence, one wavefront each.
__global__ __launch_bounds__(256) void k_filter_tail(FiltArgs a) {
  constexpr int PER = FILT_CHUNK / 256;
  __shared__ SelScratch sel;
  const int ch = blockIdx.x, m = blockIdx.y, t = threadIdx.x;
  float lv[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = ch * FILT_CHUNK + t + 256 * u;
    lv[u] = v < a.V ? a.logits[size_t(m) * a.V + v] : 0.0f;
  }
  sel_prepare(sel);
  unsigned long long key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = ch * FILT_CHUNK + t + 256 * u;
    key[u] = v < a.V ? cluster_key(lv[u], v) : 0ull;
  }
  const unsigned long long kv = block_top_keys(sel, key, a.top_k);
  if (t < a.top_k) store_coherent_u64(&a.cand[(size_t(m) * a.nch + ch) * a.top_k + t], kv);
  const int c = m % FILT_ROW_COUNTERS;
  const unsigned rows_c = unsigned((a.M - 1 - c) / FILT_ROW_COUNTERS + 1);
  if (!last_workgroup(a.counters + FILT_CNT_ROW0 + CNT_LINE * (c % 12) + c / 12, unsigned(a.nch) * rows_c)) return;
  for (int mm = c; mm < a.M; mm += FILT_ROW_COUNTERS) filt_row(a, sel, mm);
  if (!last_workgroup(a.counters + FILT_CNT_ROWS, unsigned(min(a.M, FILT_ROW_COUNTERS)))) return;
  for (int b = t >> 6; b < a.B; b += 4) filt_rule(a, b);
}

}  // namespace sv
