// sv_diag.hpp -- the optional per-slot margins of a verify step (gfx950).
//
// How close each decision of the step came to going the other way, so that a caller
// can count near ties on the device ([Self-spec] 3.1: the greedy rule compares each
// draft with the target's mode; 3.2: the sampling rule accepts with probability
// min(1, p/q) and draws the correction from max(0, p - q)):
//   greedy:   diag[b, i] = the gap between the largest and second-largest float32 logit
//             of slot i (0 when two tokens share the maximum), for the decided slots
//             i <= n_b;
//   sampling: diag[b, i] = |u_i - p_i(x) / q_i(x)| (infinity when q_i(x) = 0) for the
//             decided acceptance tests i <= min(n_b, gamma - 1), and diag[b, gamma] = the
//             gap between the two best scores log r_v + G_v of the final draw, in the
//             class the draw took (the residual max(0, p - q), or p when the residual is
//             empty or every draft was accepted);
//   NaN elsewhere (slots past the decision, invalid sequences).
// Computed after the step from the float32 logits in memory, in three launches: per
// (row, chunk) the top two logits and the softmax partial; per (sequence, chunk) the two
// best draw scores of each class; per sequence the merge.  The step's own kernels are
// untouched, so asking for no diagnostics costs nothing.
#pragma once

#include "sv_accept.hpp"
#include "sv_device.hpp"

namespace sv {

constexpr int DIAG_CHUNK = 4096;

struct DiagRow {        // one (row, chunk): top two logits, argmax, sum of exp2((l - m1) * c)
  float m1, m2, s;
  int i1;
};
struct DiagDraw {       // one (sequence, chunk): the two best scores per class
  float r1, r2, p1, p2;
  int any_r;
  int pad[3];
};

struct DiagArgs {
  const float* logits;    // [M, V]
  const int* draft;
  int draft_stride, draft_offset;
  const void* q;          // [B, gamma, V] (sampling)
  int q_bf16;
  const int64_t* pos0;    // [B] (sampling)
  const int* n_accepted;  // [B], the step's output (-1: invalid)
  float* diag;            // [B, gamma + 1]
  DiagRow* rows;          // [M, nch]
  DiagDraw* draws;        // [B, nch]
  uint64_t seed;
  int B, gamma, V, nch;
  float c;                // log2(e) / T; 0 for the greedy rule
};

// (m1, i1, m2) merge: the larger maximum wins; the second is the larger of the other
// side's maximum and the winner's second; equal maxima (different indices) tie, second =
// maximum, lower index first.
__device__ __forceinline__ void top2_merge(float& m1, int& i1, float& m2, float bm1, int bi1, float bm2) {
  if (bm1 > m1 || (bm1 == m1 && bi1 < i1)) {
    m2 = fmaxf(bm2, m1);
    m1 = bm1;
    i1 = bi1;
  } else {
    m2 = fmaxf(m2, bm1);
  }
}

__device__ __forceinline__ void best2_merge(float& a1, float& a2, float b1, float b2) {
  const float hi = fmaxf(a1, b1), lo = fminf(a1, b1);
  a1 = hi;
  a2 = fmaxf(lo, fmaxf(a2, b2));
}

// grid (nch, M): top two logits and the softmax partial of one chunk of one row
__global__ __launch_bounds__(256) void k_diag_rows(DiagArgs a) {
  const int ch = blockIdx.x, row = blockIdx.y;
  const float* l = a.logits + size_t(row) * a.V;
  const int v0 = ch * DIAG_CHUNK, v1 = min(a.V, v0 + DIAG_CHUNK);
  float m1 = -INFINITY, m2 = -INFINITY;
  int i1 = 0x7fffffff;
  for (int v = v0 + int(threadIdx.x); v < v1; v += blockDim.x) {
    const float x = l[v];
    if (x > m1) { m2 = m1; m1 = x; i1 = v; }   // ascending v per thread: the first maximum kept
    else m2 = fmaxf(m2, x);
  }
  __shared__ float s_m1[256], s_m2[256];
  __shared__ int s_i1[256];
  s_m1[threadIdx.x] = m1; s_m2[threadIdx.x] = m2; s_i1[threadIdx.x] = i1;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (int(threadIdx.x) < o) {
      float am1 = s_m1[threadIdx.x], am2 = s_m2[threadIdx.x];
      int ai1 = s_i1[threadIdx.x];
      top2_merge(am1, ai1, am2, s_m1[threadIdx.x + o], s_i1[threadIdx.x + o], s_m2[threadIdx.x + o]);
      s_m1[threadIdx.x] = am1; s_m2[threadIdx.x] = am2; s_i1[threadIdx.x] = ai1;
    }
    __syncthreads();
  }
  const float cm = s_m1[0];
  float s = 0.0f;
  if (a.c != 0.0f)
    for (int v = v0 + int(threadIdx.x); v < v1; v += blockDim.x) s += exp2f((l[v] - cm) * a.c);
  s = wave_allsum(s);
  __shared__ float s_s[4];
  if ((threadIdx.x & 63) == 0) s_s[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    DiagRow r;
    r.m1 = cm; r.m2 = s_m2[0]; r.i1 = s_i1[0];
    r.s = ((s_s[0] + s_s[1]) + s_s[2]) + s_s[3];
    a.rows[size_t(row) * a.nch + ch] = r;
  }
}

// Max and softmax sum of row ``row`` from its chunk partials (every thread of the block
// gets the same values).
__device__ __forceinline__ void diag_row_stats(const DiagArgs& a, int row, float& m, float& z) {
  __shared__ float s_m[256], s_z[256];
  float lm = -INFINITY, lz = 0.0f;
  for (int ch = threadIdx.x; ch < a.nch; ch += blockDim.x) {
    const DiagRow r = a.rows[size_t(row) * a.nch + ch];
    if (r.m1 > lm) { lz = (lz != 0.0f ? lz * exp2f((lm - r.m1) * a.c) : 0.0f) + r.s; lm = r.m1; }
    else if (r.s != 0.0f) lz += r.s * exp2f((r.m1 - lm) * a.c);
  }
  s_m[threadIdx.x] = lm;
  s_z[threadIdx.x] = lz;
  __syncthreads();
  if (threadIdx.x == 0) {
    float gm = -INFINITY, gz = 0.0f;
    for (int t = 0; t < int(blockDim.x); ++t) {
      const float tm = s_m[t], tz = s_z[t];
      if (tz == 0.0f) continue;
      if (tm > gm) { gz = (gz != 0.0f ? gz * exp2f((gm - tm) * a.c) : 0.0f) + tz; gm = tm; }
      else gz += tz * exp2f((tm - gm) * a.c);
    }
    s_m[0] = gm;
    s_z[0] = gz;
  }
  __syncthreads();
  m = s_m[0];
  z = s_z[0];
  __syncthreads();
}

// grid (nch, B), sampling only: the two best scores log r + G of each class over one
// chunk of row n_b, the row the step drew its last token from.
__global__ __launch_bounds__(256) void k_diag_draw(DiagArgs a) {
  const int ch = blockIdx.x, b = blockIdx.y;
  const int n = a.n_accepted[b];
  DiagDraw out;
  out.r1 = out.r2 = out.p1 = out.p2 = -INFINITY;
  out.any_r = 0;
  out.pad[0] = out.pad[1] = out.pad[2] = 0;
  if (n < 0) {
    if (threadIdx.x == 0) a.draws[size_t(b) * a.nch + ch] = out;
    return;
  }
  const int G1 = a.gamma + 1;
  float m, z;
  diag_row_stats(a, b * G1 + n, m, z);
  const bool resid = n < a.gamma;
  const float* l = a.logits + size_t(b * G1 + n) * a.V;
  const size_t qrow = (size_t(b) * a.gamma + (resid ? n : 0)) * a.V;
  const uint64_t pos = uint64_t(a.pos0[b] + n + 1);
  const int v0 = ch * DIAG_CHUNK, v1 = min(a.V, v0 + DIAG_CHUNK);
  float r1 = -INFINITY, r2 = -INFINITY, p1 = -INFINITY, p2 = -INFINITY;
  int any_r = 0;
  for (int vb = v0 + 4 * int(threadIdx.x); vb < v1; vb += 4 * int(blockDim.x)) {
    const Philox4 w = philox4x64_10(uint64_t(vb) >> 2, pos, uint64_t(b), TAG_GUMBEL, a.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = vb + e;
      if (v >= v1) break;
      const float G = -logf(-logf(gumbel_uniform_from_word(w.w[e])));
      const float p = exp2f((l[v] - m) * a.c) / z;
      if (p > 0.0f) best2_merge(p1, p2, logf(p) + G, -INFINITY);
      if (resid) {
        const float qv = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.q)[qrow + v])
                                  : reinterpret_cast<const float*>(a.q)[qrow + v];
        const float r = fmaxf(p - qv, 0.0f);
        if (r > 0.0f) {
          any_r = 1;
          best2_merge(r1, r2, logf(r) + G, -INFINITY);
        }
      }
    }
  }
  __shared__ float s_v[4][256];
  __shared__ int s_any;
  if (threadIdx.x == 0) s_any = 0;
  s_v[0][threadIdx.x] = r1; s_v[1][threadIdx.x] = r2; s_v[2][threadIdx.x] = p1; s_v[3][threadIdx.x] = p2;
  __syncthreads();
  if (any_r) s_any = 1;
  for (int o = 128; o > 0; o >>= 1) {
    if (int(threadIdx.x) < o) {
      float a1 = s_v[0][threadIdx.x], a2 = s_v[1][threadIdx.x];
      best2_merge(a1, a2, s_v[0][threadIdx.x + o], s_v[1][threadIdx.x + o]);
      s_v[0][threadIdx.x] = a1; s_v[1][threadIdx.x] = a2;
      float c1 = s_v[2][threadIdx.x], c2 = s_v[3][threadIdx.x];
      best2_merge(c1, c2, s_v[2][threadIdx.x + o], s_v[3][threadIdx.x + o]);
      s_v[2][threadIdx.x] = c1; s_v[3][threadIdx.x] = c2;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out.r1 = s_v[0][0]; out.r2 = s_v[1][0]; out.p1 = s_v[2][0]; out.p2 = s_v[3][0]; out.any_r = s_any;
    a.draws[size_t(b) * a.nch + ch] = out;
  }
}

// grid B: the margins of sequence b.
__global__ __launch_bounds__(256) void k_diag_finish(DiagArgs a) {
  const int b = blockIdx.x, G1 = a.gamma + 1;
  const int n = a.n_accepted[b];
  float* out = a.diag + size_t(b) * G1;
  if (n < 0) {
    for (int i = threadIdx.x; i < G1; i += blockDim.x) out[i] = NAN;
    return;
  }
  if (a.c == 0.0f) {
    // greedy: the top-two gap of every decided slot
    for (int i = 0; i < G1; ++i) {
      __shared__ float s_m1[256], s_m2[256];
      __shared__ int s_i1[256];
      float m1 = -INFINITY, m2 = -INFINITY;
      int i1 = 0x7fffffff;
      if (i <= n)
        for (int ch = threadIdx.x; ch < a.nch; ch += blockDim.x) {
          const DiagRow r = a.rows[size_t(b * G1 + i) * a.nch + ch];
          top2_merge(m1, i1, m2, r.m1, r.i1, r.m2);
        }
      s_m1[threadIdx.x] = m1; s_m2[threadIdx.x] = m2; s_i1[threadIdx.x] = i1;
      __syncthreads();
      if (threadIdx.x == 0) {
        for (int t = 1; t < int(blockDim.x); ++t) top2_merge(m1, i1, m2, s_m1[t], s_i1[t], s_m2[t]);
        out[i] = i <= n ? m1 - m2 : NAN;
      }
      __syncthreads();
    }
    return;
  }
  // sampling: the acceptance margin of every decided slot
  for (int i = 0; i < a.gamma; ++i) {
    if (i > n) {
      if (threadIdx.x == 0) out[i] = NAN;
      continue;
    }
    float m, z;
    diag_row_stats(a, b * G1 + i, m, z);
    if (threadIdx.x == 0) {
      const int x = a.draft[size_t(b) * a.draft_stride + a.draft_offset + i];
      float margin = INFINITY;
      if (x >= 0 && x < a.V) {
        const float qx = a.q_bf16 ? bf16_to_f32(reinterpret_cast<const bf16_t*>(a.q)[(size_t(b) * a.gamma + i) * a.V + x])
                                  : reinterpret_cast<const float*>(a.q)[(size_t(b) * a.gamma + i) * a.V + x];
        const float px = exp2f((a.logits[size_t(b * G1 + i) * a.V + x] - m) * a.c) / z;
        const float u = accept_uniform(a.seed, uint64_t(b), uint64_t(a.pos0[b] + i + 1));
        if (qx > 0.0f) margin = fabsf(u - px / qx);
      }
      out[i] = margin;
    }
  }
  // and the gap of the final draw, in the class it took
  if (threadIdx.x == 0) {
    bool any_r = false;
    for (int ch = 0; ch < a.nch; ++ch) any_r |= a.draws[size_t(b) * a.nch + ch].any_r != 0;
    const bool use_r = n < a.gamma && any_r;
    float s1 = -INFINITY, s2 = -INFINITY;
    for (int ch = 0; ch < a.nch; ++ch) {
      const DiagDraw d = a.draws[size_t(b) * a.nch + ch];
      if (use_r) best2_merge(s1, s2, d.r1, d.r2);
      else best2_merge(s1, s2, d.p1, d.p2);
    }
    out[a.gamma] = s2 == -INFINITY ? INFINITY : s1 - s2;
  }
}

}  // namespace sv
