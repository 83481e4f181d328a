// sv_decoder.hpp -- the non-GEMM pieces of the full-model verify forward (gfx950):
// embedding gather, RMSNorm, rotary embedding with K/V append into the cache,
// causal decode attention of the gamma+1 new positions over the cache, SiLU*up.
//
// The gamma+1 positions are processed in one pass: position i attends to the
// cached prefix and to new positions 0..i only, so its prediction cannot see later
// drafts ([Infra-ch8] "why one forward pass can verify several tokens").  K/V of all
// new positions are appended at len..len+gamma; the acceptance kernels later advance
// len by n+1, which discards the K/V of rejected drafts ([Self-spec] 3.3;
// [MTP-drafters] 4.2 item 3).
//
// bf16 values are produced exactly where the matrix cores consume them or the cache
// stores them: RMSNorm outputs, K (after RoPE) and V in the cache, the attention
// output, SiLU(gate)*up.  Everything else stays float32.
#pragma once

#include "sv_device.hpp"

namespace sv {

struct DecArgs {
  int B, G1, d, H, hd, ff, V, max_len, n_layers;
  float eps;
};

// Cache lengths and RoPE table for the G1 new positions of every sequence.
// invalid[b] = 1 when the cache cannot hold the new positions.  One thread per
// (row, frequency) pair; angles in float64 (positions reach thousands of radians).
__global__ __launch_bounds__(256) void k_prep(const int* __restrict__ len, float2* __restrict__ rope_cs,
                                              int* __restrict__ invalid, int B, int G1, int hd, int max_len,
                                              float theta) {
  const int half = hd / 2;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < B) invalid[t] = (len[t] < 0 || len[t] > max_len - G1) ? 1 : 0;
  if (t >= B * G1 * half) return;
  const int m = t / half, j = t - m * half;
  const int b = m / G1, i = m - b * G1;
  const double pos = double(len[b]) + double(i);
  const double inv = exp(-(2.0 * j / double(hd)) * log(double(theta)));
  const double ang = pos * inv;
  rope_cs[t] = make_float2(float(cos(ang)), float(sin(ang)));
}

// x[m, :] = embed[tokens[m], :] (float32 residual stream).  Out-of-range ids give
// a zero row and mark the sequence invalid.
__global__ __launch_bounds__(256) void k_embed(const int* __restrict__ tokens, const bf16_t* __restrict__ embed,
                                               float* __restrict__ x, int* __restrict__ invalid, int G1, int V,
                                               int d) {
  const int m = blockIdx.x;
  const int tok = tokens[m];
  const bool ok = tok >= 0 && tok < V;
  if (!ok && threadIdx.x == 0) invalid[m / G1] = 1;
  for (int k = threadIdx.x; k < d; k += blockDim.x)
    x[size_t(m) * d + k] = ok ? bf16_to_f32(embed[size_t(tok) * d + k]) : 0.0f;
}

// Residual add and RMSNorm: x[m, :] += add[m, :] (if add is given), then
// h[m, :] = bf16(x / sqrt(mean(x^2) + eps) * g).  One workgroup per row.
__global__ __launch_bounds__(256) void k_add_rmsnorm(float* __restrict__ x, const float* __restrict__ add,
                                                     const bf16_t* __restrict__ g, bf16_t* __restrict__ h, int d,
                                                     float eps) {
  const int m = blockIdx.x;
  float* xr = x + size_t(m) * d;
  float ss = 0.0f;
  for (int k = threadIdx.x; k < d; k += blockDim.x) {
    float v = xr[k];
    if (add) {
      v += add[size_t(m) * d + k];
      xr[k] = v;
    }
    ss = fmaf(v, v, ss);
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float scale = 1.0f / sqrtf(tot / float(d) + eps);
  for (int k = threadIdx.x; k < d; k += blockDim.x)
    h[size_t(m) * d + k] = f32_to_bf16(xr[k] * scale * bf16_to_f32(g[k]));
}

__device__ __forceinline__ size_t cache_index(const DecArgs& a, int layer, int b, int h, int pos, int j) {
  return ((((size_t(layer) * a.B + b) * a.H + h) * size_t(a.max_len) + pos) * a.hd) + j;
}

// Rotate q and k of the new positions (rotate-half pairs j, j + hd/2), then append
// bf16 K and V into the cache at len[b] + i.  grid (M, H), hd/2 threads.
__global__ void k_rope_append(float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
                              const float2* __restrict__ rope_cs, bf16_t* __restrict__ kc, bf16_t* __restrict__ vc,
                              const int* __restrict__ len, const int* __restrict__ invalid, DecArgs a, int layer) {
  const int m = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
  const int half = a.hd / 2;
  if (j >= half) return;
  const int b = m / a.G1, i = m - b * a.G1;
  const float2 cs = rope_cs[m * half + j];
  const size_t base = size_t(m) * a.H * a.hd + size_t(h) * a.hd;
  const float q1 = q[base + j], q2 = q[base + j + half];
  q[base + j] = q1 * cs.x - q2 * cs.y;
  q[base + j + half] = q2 * cs.x + q1 * cs.y;
  if (invalid[b]) return;
  const float k1 = k[base + j], k2 = k[base + j + half];
  const int pos = len[b] + i;
  kc[cache_index(a, layer, b, h, pos, j)] = f32_to_bf16(k1 * cs.x - k2 * cs.y);
  kc[cache_index(a, layer, b, h, pos, j + half)] = f32_to_bf16(k2 * cs.x + k1 * cs.y);
  vc[cache_index(a, layer, b, h, pos, j)] = f32_to_bf16(v[base + j]);
  vc[cache_index(a, layer, b, h, pos, j + half)] = f32_to_bf16(v[base + j + half]);
}

constexpr int ATT_MAXQ = 16;   // gamma + 1 <= 16

// Split-K decode attention.  grid (S, H, B), 256 threads; split s covers a range of
// the len[b] + G1 keys, processed in tiles of 64 keys per wavefront.  Scores: lane =
// key, dot with the G1 queries from LDS.  Values: lane = dimension pair.  Online
// softmax per query; the four wavefronts are merged in LDS and one partial
// (max, sum, unnormalised output) per (b, h, s, query) is written.
template <int HD>
__global__ __launch_bounds__(256) void k_attn(const float* __restrict__ q, const bf16_t* __restrict__ kc,
                                              const bf16_t* __restrict__ vc, const int* __restrict__ len,
                                              const int* __restrict__ invalid, float* __restrict__ part, DecArgs a,
                                              int layer, int S, float scale) {
  constexpr int DPL = HD / 64;                 // dimensions per lane in the value phase
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G1 = a.G1;
  __shared__ float sq[ATT_MAXQ][HD];
  __shared__ float sp[4][ATT_MAXQ][64];
  __shared__ float sm[4][ATT_MAXQ], sl[4][ATT_MAXQ];
  __shared__ float so[4][ATT_MAXQ][HD];
  const size_t psz = size_t(HD + 2);
  float* out = part + ((((size_t(b) * a.H + h) * S + s) * G1) * psz);
  if (invalid[b]) {
    for (int t = threadIdx.x; t < G1 * int(psz); t += blockDim.x) out[t] = (t % psz == 0) ? -INFINITY : 0.0f;
    return;
  }
  for (int t = threadIdx.x; t < G1 * HD; t += blockDim.x) {
    const int i = t / HD, j = t - i * HD;
    sq[i][j] = q[(size_t(b) * G1 + i) * a.H * HD + size_t(h) * HD + j] * scale;
  }
  __syncthreads();
  const int L = len[b];
  const int nk = L + G1;
  const int per = (nk + S - 1) / S;
  const int k_beg = s * per, k_end = min(nk, k_beg + per);
  float mi[ATT_MAXQ], li[ATT_MAXQ], oi[ATT_MAXQ][DPL];
#pragma unroll
  for (int i = 0; i < ATT_MAXQ; ++i) {
    mi[i] = -INFINITY; li[i] = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) oi[i][e] = 0.0f;
  }
  const bf16_t* kbase = kc + cache_index(a, layer, b, h, 0, 0);
  const bf16_t* vbase = vc + cache_index(a, layer, b, h, 0, 0);
  for (int t0 = k_beg + wave * 64; t0 < k_end; t0 += 4 * 64) {
    const int key = t0 + lane;
    float sc[ATT_MAXQ];
#pragma unroll
    for (int i = 0; i < ATT_MAXQ; ++i) sc[i] = 0.0f;
    if (key < k_end) {
      const bf16_t* kr = kbase + size_t(key) * HD;
      for (int j0 = 0; j0 < HD; j0 += 8) {
        const u32x4 w = load16(kr + j0);
        float kf[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kf[2 * e] = __uint_as_float(w[e] << 16);
          kf[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < ATT_MAXQ; ++i) {
          if (i < G1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sc[i] = fmaf(sq[i][j0 + e], kf[e], sc[i]);
          }
        }
      }
    }
    // causal mask: query i sees keys <= L + i
#pragma unroll
    for (int i = 0; i < ATT_MAXQ; ++i) {
      if (i >= G1) break;
      const float sv_ = (key < k_end && key <= L + i) ? sc[i] : -INFINITY;
      float tmax = sv_;
      for (int o = 32; o > 0; o >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o));
      const float mnew = fmaxf(mi[i], tmax);
      float p = 0.0f, corr = 1.0f;
      if (mnew != -INFINITY) {
        p = (sv_ == -INFINITY) ? 0.0f : expf(sv_ - mnew);
        corr = (mi[i] == -INFINITY) ? 0.0f : expf(mi[i] - mnew);
      }
      float psum = p;
      for (int o = 32; o > 0; o >>= 1) psum += __shfl_xor(psum, o);
      li[i] = li[i] * corr + psum;
      mi[i] = mnew;
#pragma unroll
      for (int e = 0; e < DPL; ++e) oi[i][e] *= corr;
      sp[wave][i][lane] = p;
    }
    __builtin_amdgcn_wave_barrier();
    const int nkt = min(64, k_end - t0);
    for (int kk = 0; kk < nkt; ++kk) {
      const bf16_t* vr = vbase + size_t(t0 + kk) * HD + lane * DPL;
      float vf[DPL];
      if (DPL == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(vr);
        vf[0] = __uint_as_float(w << 16);
        vf[DPL - 1] = __uint_as_float(w & 0xffff0000u);
      } else {
        vf[0] = bf16_to_f32(vr[0]);
      }
#pragma unroll
      for (int i = 0; i < ATT_MAXQ; ++i) {
        if (i < G1) {
          const float p = sp[wave][i][kk];
#pragma unroll
          for (int e = 0; e < DPL; ++e) oi[i][e] = fmaf(p, vf[e], oi[i][e]);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  // merge the four wavefronts
#pragma unroll
  for (int i = 0; i < ATT_MAXQ; ++i) {
    if (i < G1) {
      if (lane == 0) { sm[wave][i] = mi[i]; sl[wave][i] = li[i]; }
#pragma unroll
      for (int e = 0; e < DPL; ++e) so[wave][i][lane * DPL + e] = oi[i][e];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < G1 * HD; t += blockDim.x) {
    const int i = t / HD, j = t - i * HD;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][i]);
    float l = 0.0f, o = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        if (sm[w][i] == -INFINITY) continue;
        const float f = expf(sm[w][i] - M);
        l += sl[w][i] * f;
        o += so[w][i][j] * f;
      }
    }
    float* po = out + size_t(i) * psz;
    if (j == 0) { po[0] = M; po[1] = l; }
    po[2 + j] = o;
  }
}

// Merge the S partials of every (row, head) and store bf16 attention output
// [M, H*hd].  grid (M, H), hd threads.
__global__ void k_attn_merge(const float* __restrict__ part, bf16_t* __restrict__ out, DecArgs a, int S) {
  const int m = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
  if (j >= a.hd) return;
  const int b = m / a.G1, i = m - b * a.G1;
  const size_t psz = size_t(a.hd + 2);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, part[((((size_t(b) * a.H + h) * S + s) * a.G1) + i) * psz]);
  float l = 0.0f, o = 0.0f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float* p = part + ((((size_t(b) * a.H + h) * S + s) * a.G1) + i) * psz;
      if (p[0] == -INFINITY) continue;
      const float f = expf(p[0] - M);
      l += p[1] * f;
      o += p[2 + j] * f;
    }
  }
  out[size_t(m) * a.H * a.hd + size_t(h) * a.hd + j] = f32_to_bf16(l > 0.0f ? o / l : 0.0f);
}

// f[m, j] = bf16(SiLU(gate) * up).
__global__ __launch_bounds__(256) void k_silu_mul(const float* __restrict__ gate, const float* __restrict__ up,
                                                  bf16_t* __restrict__ f, int n) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  const float gv = gate[t];
  f[t] = f32_to_bf16(gv / (1.0f + expf(-gv)) * up[t]);
}

}  // namespace sv
