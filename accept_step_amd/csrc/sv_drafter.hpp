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
// per thread and step.  Also clears the row's residual stream x[b, 0..H) when x is given
// (the down-projection of the joined input then adds into it).
__global__ __launch_bounds__(256) void k_mtp_join(const int* __restrict__ tok, const bf16_t* __restrict__ embed,
                                                  const bf16_t* __restrict__ g, bf16_t* __restrict__ z, int D,
                                                  float* __restrict__ x, int H) {
  const int b = blockIdx.x;
  if (x)
    for (int i = threadIdx.x; i < H; i += blockDim.x) x[size_t(b) * H + i] = 0.0f;
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

// cos/sin of the queries of every step, once per call: tab[(k * B + b) * hd/2 + j] for
// position len[b] + k (angle in float64, as k_mtp_rope_q).  Grid-stride.
__global__ __launch_bounds__(256) void k_mtp_rope_table(const int* __restrict__ len, float2* __restrict__ tab, int B,
                                                        int gamma, int hd, float theta) {
  const int half = hd / 2, n = gamma * B * half;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < n; t += gridDim.x * blockDim.x) {
    const int j = t % half, kb = t / half, b = kb % B, k = kb / B;
    const double ang = (double(len[b]) + double(k)) * exp(-(2.0 * j / double(hd)) * log(double(theta)));
    tab[t] = make_float2(float(cos(ang)), float(sin(ang)));
  }
}

// y = bf16(x) for the new hidden state [B, D]; with z given, also into the hidden half of
// the next step's joined input z[b, D..2D).
__global__ __launch_bounds__(256) void k_f32_to_bf16(const float* __restrict__ x, bf16_t* __restrict__ y, int n,
                                                     bf16_t* __restrict__ z = nullptr, int D = 0) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const bf16_t v = f32_to_bf16(x[t]);
  y[t] = v;
  if (z) z[size_t(t / D) * 2 * D + D + t % D] = v;
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
  // with z given: the next step's joined input gets the drafted token's embedding
  // (z[b, 0..D) = embed[x]) and the residual stream x_res[b, 0..H) is cleared
  bf16_t* z;
  const bf16_t* embed;
  float* x_res;
  int D, H;
};

__device__ __forceinline__ int draft_token_id(const DraftSampleArgs& a, int b, int j) {
  if (!a.clusters) return j;
  const int c = j / a.cs;
  return a.clusters[size_t(b) * a.top_k + c] * a.cs + (j - c * a.cs);
}

// Online (max, sum of exp((l - max) / T)) merge.
__device__ __forceinline__ void softmax_merge(float& m, float& s, float m2, float s2, float inv_t) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;
  s = (m == -INFINITY ? 0.0f : s * expf((m - mm) * inv_t)) + (m2 == -INFINITY ? 0.0f : s2 * expf((m2 - mm) * inv_t));
  m = mm;
}

// Threads of the draw: one group of four scored ids (one Philox block) per thread at
// the masked head's 4096 scored tokens.
constexpr int MTP_SAMPLE_THREADS = 1024;

// One workgroup (MTP_SAMPLE_THREADS threads) per sequence over its n scored tokens, four consecutive
// entries per thread and step (one Philox block per four vocabulary ids when they are
// consecutive and aligned, as the members of a cluster are).  T > 0: one pass for
// m = max l and Z = sum exp((l - m) / T) (online per thread, merged over the block),
// one for q_j = exp((l_j - m) / T) / Z, stored at its token id, and the draft = the
// largest (log q_j + G, lower id) with G the Gumbel noise of Philox stream tag 2 at
// position len + k + 1.  T = 0: the largest (l, lower id).
__global__ __launch_bounds__(MTP_SAMPLE_THREADS) void k_mtp_sample(DraftSampleArgs a) {
  constexpr int NT = MTP_SAMPLE_THREADS, NW = NT / 64;
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __shared__ float s_m[NW], s_s[NW];
  __shared__ unsigned long long s_key[NW];
  const float* l = a.logits + size_t(b) * a.n;
  const bool bad = a.invalid[b] != 0;
  const size_t qrow = (size_t(b) * a.gamma + a.k) * a.V;
  const int ng = (a.n + 3) / 4;
  auto load4 = [&](int g, float (&v)[4]) {
    const int j0 = 4 * g;
    if (j0 + 4 <= a.n && (a.n & 3) == 0) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(l + j0);
      v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = j0 + e < a.n ? l[j0 + e] : -INFINITY;
    }
  };
  unsigned long long key = 0ull;
  if (a.greedy) {
    for (int g = t; g < ng; g += NT) {
      float v[4];
      load4(g, v);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * g + e < a.n) key = max_u64(key, win_key(false, v[e], draft_token_id(a, b, 4 * g + e)));
    }
  } else {
    float m = -INFINITY, sum = 0.0f;
    for (int g = t; g < ng; g += NT) {
      float v[4];
      load4(g, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) softmax_merge(m, sum, v[e], 1.0f, a.inv_t);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sum, o);
      softmax_merge(m, sum, m2, s2, a.inv_t);
    }
    if (lane == 0) { s_m[wave] = m; s_s[wave] = sum; }
    __syncthreads();
    m = s_m[0];
    sum = s_s[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) softmax_merge(m, sum, s_m[w], s_s[w], a.inv_t);
    const float inv_z = 1.0f / sum;
    const uint64_t pos = uint64_t(int64_t(a.len[b]) + a.k + 1);
    for (int g = t; g < ng; g += NT) {
      float v[4];
      load4(g, v);
      int id[4];
      float qv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        id[e] = 4 * g + e < a.n ? draft_token_id(a, b, 4 * g + e) : -1;
        qv[e] = (bad || id[e] < 0) ? 0.0f : expf((v[e] - m) * a.inv_t) * inv_z;
      }
      const bool run = id[3] == id[0] + 3 && ((qrow + size_t(id[0])) & 3) == 0;   // four ids, aligned store
      if (run) {
        if (a.q_bf16) {
          uint2 w;
          w.x = uint32_t(f32_to_bf16(qv[0])) | (uint32_t(f32_to_bf16(qv[1])) << 16);
          w.y = uint32_t(f32_to_bf16(qv[2])) | (uint32_t(f32_to_bf16(qv[3])) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(a.q) + qrow + id[0]) = w;
        } else {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.q) + qrow + id[0]) = f32x4{qv[0], qv[1], qv[2], qv[3]};
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (id[e] < 0) continue;
          if (a.q_bf16) reinterpret_cast<bf16_t*>(a.q)[qrow + id[e]] = f32_to_bf16(qv[e]);
          else reinterpret_cast<float*>(a.q)[qrow + id[e]] = qv[e];
        }
      }
      float G[4];
      int blk = -1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!(qv[e] > 0.0f)) continue;
        if ((id[e] >> 2) != blk) {
          blk = id[e] >> 2;
          draft_gumbel4(a.seed, b, pos, id[e] & ~3, G);
        }
        float gv = G[0];
#pragma unroll
        for (int u = 1; u < 4; ++u)
          if ((id[e] & 3) == u) gv = G[u];
        key = max_u64(key, win_key(false, logf(qv[e]) + gv, id[e]));
      }
    }
  }
  key = wave_allmax_u64(key);
  if (lane == 0) s_key[wave] = key;
  __syncthreads();
  __shared__ int s_x;
  if (t == 0) {
    unsigned long long kb = s_key[0];
    for (int w = 1; w < NW; ++w) kb = max_u64(kb, s_key[w]);
    const int x = (bad || !kb) ? -1 : win_index(kb);
    a.draft[size_t(b) * a.gamma + a.k] = x;
    a.tok[b] = x < 0 ? 0 : x;
    s_x = x < 0 ? 0 : x;
  }
  if (!a.z) return;
  __syncthreads();
  const u32x4* e = reinterpret_cast<const u32x4*>(a.embed + size_t(s_x) * a.D);
  u32x4* o = reinterpret_cast<u32x4*>(a.z + size_t(b) * 2 * a.D);
  for (int i = t; i < a.D / 8; i += NT) o[i] = e[i];
  for (int i = t; i < a.H; i += NT) a.x_res[size_t(b) * a.H + i] = 0.0f;
}

}  // namespace sv
