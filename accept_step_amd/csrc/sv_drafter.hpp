// sv_drafter.hpp -- the MTP drafter's draft step (gfx950): the kernels that the
// decoder's products, RMSNorm and attention kernels do not already cover.
//
// [X-thread] "Gemma 4's MTP" (target activations, KV cache sharing, efficient
// embedder) and [MTP-deep-dive] 3.1-3.4: each step joins the embedding of the current
// token with a hidden state (the target's last one at the first step, the drafter's own
// up-projected one after), projects the pair down to the drafter's width, runs decoder
// layers whose attention has query projections only and reads the target's KV cache,
// projects back up and scores tokens with the tied head (or the centroid-masked head).
// The drafted token and the new hidden state feed the next step.
#pragma once

#include "sv_head.hpp"
#include "sv_masked.hpp"

namespace sv {

// Per call: lenq[b] = len[b] - 1 (the attention kernel's view: keys [0, lenq + 1) =
// the cached positions), invalid[b] when len is outside [1, max_len] or the first
// token is no token, tok[b] = the first token (0 for an invalid row), and the
// attention's split counters cleared.
__global__ __launch_bounds__(256) void k_mtp_prep(const int* __restrict__ len, const int* __restrict__ last_token,
                                                  int* __restrict__ lenq, int* __restrict__ invalid,
                                                  int* __restrict__ tok, unsigned* __restrict__ att_cnt, int ncnt,
                                                  int B, int max_len, int V) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < ncnt) att_cnt[t] = 0u;
  if (t < B) {
    const int L = len[t], x = last_token[t];
    const bool bad = L < 1 || L > max_len || x < 0 || x >= V;
    invalid[t] = bad ? 1 : 0;
    lenq[t] = bad ? 0 : L - 1;
    tok[t] = bad ? 0 : x;
  }
}

// z[b] = [embed[tok[b]], g[b]] in bf16, [B, 2D].  One workgroup per row, 16 bytes
// per thread and step.
__global__ __launch_bounds__(256) void k_mtp_join(const int* __restrict__ tok, const bf16_t* __restrict__ embed,
                                                  const bf16_t* __restrict__ g, bf16_t* __restrict__ z, int D) {
  const int b = blockIdx.x;
  const int n8 = D / 8;
  const u32x4* e = reinterpret_cast<const u32x4*>(embed + size_t(tok[b]) * D);
  const u32x4* h = reinterpret_cast<const u32x4*>(g + size_t(b) * D);
  u32x4* o = reinterpret_cast<u32x4*>(z + size_t(b) * 2 * D);
  for (int i = threadIdx.x; i < n8; i += blockDim.x) {
    o[i] = e[i];
    o[n8 + i] = h[i];
  }
}

// Rotate the queries of step k at position len[b] + k (rotate-half pairs j, j + hd/2;
// angle pos * theta^(-2j / hd) in float64).  grid (B, heads), hd / 2 threads.
__global__ void k_mtp_rope_q(float* __restrict__ q, const int* __restrict__ len, int k, int nh, int hd, float theta) {
  const int b = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
  const int half = hd / 2;
  if (j >= half) return;
  const double pos = double(len[b]) + double(k);
  const double ang = pos * exp(-(2.0 * j / double(hd)) * log(double(theta)));
  const float c = float(cos(ang)), s = float(sin(ang));
  float* r = q + (size_t(b) * nh + h) * hd;
  const float x1 = r[j], x2 = r[j + half];
  r[j] = x1 * c - x2 * s;
  r[j + half] = x2 * c + x1 * s;
}

__global__ __launch_bounds__(256) void k_f32_to_bf16(const float* __restrict__ x, bf16_t* __restrict__ y, int n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) y[t] = f32_to_bf16(x[t]);
}

// Zero fill of n bytes at p (16-byte aligned): 16 bytes per thread and step, then the
// last n % 16 bytes by the first threads.
__global__ __launch_bounds__(256) void k_zero_bytes(unsigned char* __restrict__ p, size_t n) {
  const size_t n16 = n / 16;
  u32x4* p16 = reinterpret_cast<u32x4*>(p);
  const size_t t0 = blockIdx.x * size_t(blockDim.x) + threadIdx.x;
  for (size_t i = t0; i < n16; i += size_t(gridDim.x) * blockDim.x) p16[i] = u32x4{0u, 0u, 0u, 0u};
  if (t0 < n - n16 * 16) p[n16 * 16 + t0] = 0;
}

// Gumbel noise of the drafter's stream (tag 2) for vocab entries vb .. vb+3 at absolute
// position pos of sequence b, laid out as the verify's (block vb / 4, word vb & 3).
__device__ __forceinline__ void draft_gumbel4(uint64_t seed, int b, uint64_t pos, int vb, float (&G)[4]) {
  const Philox4 w = philox4x64_10(uint64_t(vb) >> 2, pos, uint64_t(b), TAG_DRAFT, seed, 0);
#pragma unroll
  for (int e = 0; e < 4; ++e) G[e] = -logf(-logf(gumbel_uniform_from_word(w.w[e])));
}

struct DraftSampleArgs {
  const float* logits;        // [B, n] scored logits
  const int32_t* clusters;    // [B, top_k] kept clusters (masked head) or null (tied head: entry j is token j)
  int n, cs, top_k, V, gamma, k;
  float inv_t;                // 1 / T (T > 0)
  int greedy;                 // T == 0
  uint64_t seed;
  const int* len;             // [B]
  const int* invalid;         // [B]
  int* draft;                 // [B, gamma]
  int* tok;                   // [B] the next step's token
  void* q;                    // [B, gamma, V] or null (greedy)
  int q_bf16;
};

__device__ __forceinline__ int draft_token_id(const DraftSampleArgs& a, int b, int j) {
  if (!a.clusters) return j;
  const int c = j / a.cs;
  return a.clusters[size_t(b) * a.top_k + c] * a.cs + (j - c * a.cs);
}

// One workgroup (256 threads) per sequence over its n scored tokens.  T > 0:
// m = max l, Z = sum exp((l - m) / T), q_j = exp((l_j - m) / T) / Z stored at its token
// id; the draft is the largest (log q_j + G, lower id) with G the Gumbel noise of Philox
// stream tag 2 at position len + k + 1.  T = 0: the largest (l, lower id).
__global__ __launch_bounds__(256) void k_mtp_sample(DraftSampleArgs a) {
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ float s_red[4];
  __shared__ unsigned long long s_key[4];
  const float* l = a.logits + size_t(b) * a.n;
  const bool bad = a.invalid[b] != 0;
  const size_t qrow = (size_t(b) * a.gamma + a.k) * a.V;
  unsigned long long key = 0ull;
  if (a.greedy) {
    for (int j = t; j < a.n; j += 256) key = max_u64(key, win_key(false, l[j], draft_token_id(a, b, j)));
  } else {
    float m = -INFINITY;
    for (int j = t; j < a.n; j += 256) m = fmaxf(m, l[j]);
    m = wave_max_rl(m);
    if (lane == 0) s_red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    __syncthreads();
    float z = 0.0f;
    for (int j = t; j < a.n; j += 256) z += expf((l[j] - m) * a.inv_t);
    z = wave_sum_rl(z);
    if (lane == 0) s_red[wave] = z;
    __syncthreads();
    z = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    const float inv_z = 1.0f / z;
    const uint64_t pos = uint64_t(int64_t(a.len[b]) + a.k + 1);
    for (int j = t; j < a.n; j += 256) {
      const int id = draft_token_id(a, b, j);
      const float qv = bad ? 0.0f : expf((l[j] - m) * a.inv_t) * inv_z;
      if (a.q_bf16) reinterpret_cast<bf16_t*>(a.q)[qrow + id] = f32_to_bf16(qv);
      else reinterpret_cast<float*>(a.q)[qrow + id] = qv;
      if (qv > 0.0f) {
        float G[4];
        draft_gumbel4(a.seed, b, pos, id & ~3, G);
        float gv = G[0];
#pragma unroll
        for (int e = 1; e < 4; ++e)
          if ((id & 3) == e) gv = G[e];
        key = max_u64(key, win_key(false, logf(qv) + gv, id));
      }
    }
  }
  key = wave_allmax_u64(key);
  if (lane == 0) s_key[wave] = key;
  __syncthreads();
  if (t == 0) {
    const unsigned long long kb = max_u64(max_u64(s_key[0], s_key[1]), max_u64(s_key[2], s_key[3]));
    const int x = (bad || !kb) ? -1 : win_index(kb);
    a.draft[size_t(b) * a.gamma + a.k] = x;
    a.tok[b] = x < 0 ? 0 : x;
  }
}

}  // namespace sv
