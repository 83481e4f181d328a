// sv_rounds.hpp -- round policies around the verify step, on the device (gfx950).
//
// [MTP-drafters] 6 (adaptive draft length, several candidates), [MTP-deep-dive] 5.1 (the
// heuristic schedule), [Self-spec] 3.3 (each sequence keeps what it accepted).  A batch
// verifies gamma_max slots; sequence b uses gamma_b of them.  Padding the rest with the
// draft id -1 and q rows of zeros makes the unchanged rule stop at slot gamma_b at the
// latest and draw the bonus there (the residual max(0, p - 0) is p), at the bonus's
// position: each sequence gets exactly what verifying it alone with gamma_b drafts gives.
#pragma once

#include "sv_head.hpp"

namespace sv {

// conf[b, k] = max_v q[b, k, v].  grid (G, B), 256 threads.
__global__ __launch_bounds__(256) void k_round_conf(const void* __restrict__ q, int q_bf16, int G, int V,
                                                    float* __restrict__ conf) {
  const int k = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const size_t row = (size_t(b) * G + k) * V;
  float m = 0.0f;
  if (q_bf16) {
    const bf16_t* r = reinterpret_cast<const bf16_t*>(q) + row;
    for (int v = t; v < V; v += 256) m = fmaxf(m, bf16_to_f32(r[v]));
  } else {
    const float* r = reinterpret_cast<const float*>(q) + row;
    for (int v = t; v < V; v += 256) m = fmaxf(m, r[v]);
  }
  m = wave_max_rl(m);
  __shared__ float s[4];
  if ((t & 63) == 0) s[t >> 6] = m;
  __syncthreads();
  if (t == 0) conf[size_t(b) * G + k] = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
}

// gamma_b[b] = clamp(gamma_b[b], 1, G); with conf given, cut further to the leading
// steps whose conf >= tau (at least 1).  One thread per sequence.
__global__ __launch_bounds__(256) void k_round_cut(int* __restrict__ gamma_b, const float* __restrict__ conf,
                                                   float tau, int B, int G) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int g = min(max(gamma_b[b], 1), G);
  if (conf) {
    int k = 0;
    while (k < g && conf[size_t(b) * G + k] >= tau) ++k;
    g = max(1, k);
  }
  gamma_b[b] = g;
}

// Pad: draft[b, i] = -1 and q[b, i, :] = 0 for i >= gamma_b[b].  grid (G, B, chunks),
// 256 threads; chunk c of a row clears entries [c * 4096, (c + 1) * 4096).
__global__ __launch_bounds__(256) void k_round_pad(const int* __restrict__ gamma_b, int* __restrict__ draft,
                                                   void* __restrict__ q, int q_bf16, int G, int V) {
  const int i = blockIdx.x, b = blockIdx.y, c = blockIdx.z, t = threadIdx.x;
  if (i < gamma_b[b]) return;
  if (c == 0 && t == 0) draft[size_t(b) * G + i] = -1;
  if (!q) return;
  const size_t row = (size_t(b) * G + i) * V;
  const int v0 = c * 4096, v1 = min(V, v0 + 4096);
  if (q_bf16) {
    bf16_t* r = reinterpret_cast<bf16_t*>(q) + row;
    for (int v = v0 + t; v < v1; v += 256) r[v] = 0;
  } else {
    float* r = reinterpret_cast<float*>(q) + row;
    for (int v = v0 + t; v < v1; v += 256) r[v] = 0.0f;
  }
}

// Heuristic schedule: gamma_b += 2 if every draft was accepted (n >= gamma_b), else
// gamma_b -= 1, within [gmin, gmax]; an invalid round (n < 0) keeps gamma_b.
__global__ __launch_bounds__(256) void k_round_schedule(const int* __restrict__ n, int* __restrict__ gamma_b,
                                                        int B, int gmin, int gmax) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int g = gamma_b[b], nb = n[b];
  if (nb < 0) return;
  gamma_b[b] = min(max(nb >= g ? g + 2 : g - 1, gmin), gmax);
}

// The longest accepted of C candidates per sequence (the lower index on ties):
// best[b], n_out[b], tokens_out[b, :].  One thread per sequence.
__global__ __launch_bounds__(256) void k_round_select(const int* __restrict__ n, const int* __restrict__ tokens,
                                                      int B, int C, int G1, int* __restrict__ best,
                                                      int* __restrict__ n_out, int* __restrict__ tokens_out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int bi = 0, bn = n[size_t(b) * C];
  for (int c = 1; c < C; ++c) {
    const int v = n[size_t(b) * C + c];
    if (v > bn) { bn = v; bi = c; }
  }
  if (best) best[b] = bi;
  n_out[b] = bn;
  for (int j = 0; j < G1; ++j) tokens_out[size_t(b) * G1 + j] = tokens[(size_t(b) * C + bi) * G1 + j];
}

}  // namespace sv
