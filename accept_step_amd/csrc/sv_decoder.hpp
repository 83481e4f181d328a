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

#include "sv_accept.hpp"
#include "sv_device.hpp"

namespace sv {

struct DecArgs {
  int B, G1, d, H, hd, ff, V, max_len, n_layers;
  float eps;
};

// Cache lengths and RoPE table for the G1 new positions of every sequence.
// invalid[b] = 1 when the cache cannot hold the new positions.  One thread per
// (row, frequency) pair; angles in float64 (positions reach thousands of radians).
// Also zeroes the attention's split counters (their place in the workspace depends
// on the shapes of the call, so it may hold anything from an earlier call).
__global__ __launch_bounds__(256) void k_prep(const int* __restrict__ len, float2* __restrict__ rope_cs,
                                              int* __restrict__ invalid, unsigned* __restrict__ att_cnt, int ncnt,
                                              int B, int G1, int hd, int max_len, float theta) {
  const int half = hd / 2;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < ncnt) att_cnt[t] = 0;
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
// Also stores the row's sum of squares in ss_out[m] (if given) for the RMSNorm that the
// next product applies while staging the row.
__global__ __launch_bounds__(256) void k_embed(const int* __restrict__ tokens, const bf16_t* __restrict__ embed,
                                               float* __restrict__ x, int* __restrict__ invalid,
                                               float* __restrict__ ss_out, int G1, int V, int d) {
  const int m = blockIdx.x;
  const int tok = tokens[m];
  const bool ok = tok >= 0 && tok < V;
  if (!ok && threadIdx.x == 0) invalid[m / G1] = 1;
  float ss = 0.0f;
  for (int k = threadIdx.x; k < d; k += blockDim.x) {
    const float v = ok ? bf16_to_f32(embed[size_t(tok) * d + k]) : 0.0f;
    x[size_t(m) * d + k] = v;
    ss = fmaf(v, v, ss);
  }
  if (!ss_out) return;
  ss = wave_allsum(ss);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) ss_out[m] = red[0] + red[1] + red[2] + red[3];
}

// Residual add and RMSNorm: x[m, :] += add[m, :] (if add is given), then
// h[m, :] = bf16(x / sqrt(mean(x^2) + eps) * g).  One workgroup per row; each thread
// keeps its float4 groups of the row in registers (d <= 256 * 4 * RMS_VEC).
constexpr int RMS_VEC = 8;

__global__ __launch_bounds__(256) void k_add_rmsnorm(float* __restrict__ x, const float* __restrict__ add,
                                                     const bf16_t* __restrict__ g, bf16_t* __restrict__ h, int d,
                                                     float eps) {
  const int m = blockIdx.x;
  float* xr = x + size_t(m) * d;
  const int n4 = d / 4;                                 // d % 32 == 0
  f32x4 v[RMS_VEC], ad[RMS_VEC];
#pragma unroll
  for (int u = 0; u < RMS_VEC; ++u) {
    const int k4 = threadIdx.x + u * blockDim.x;
    v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    ad[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (k4 < n4) {
      v[u] = reinterpret_cast<const f32x4*>(xr)[k4];
      if (add) ad[u] = reinterpret_cast<const f32x4*>(add + size_t(m) * d)[k4];
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int u = 0; u < RMS_VEC; ++u) {
    const int k4 = threadIdx.x + u * blockDim.x;
    if (k4 < n4) {
      if (add) {
        v[u] += ad[u];
        reinterpret_cast<f32x4*>(xr)[k4] = v[u];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) ss = fmaf(v[u][e], v[u][e], ss);
    }
  }
  ss += dpp<DPP_XOR1>(ss);
  ss += dpp<DPP_XOR2>(ss);
  ss += dpp<DPP_HALF_MIRROR>(ss);
  ss += dpp<DPP_MIRROR>(ss);
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float scale = 1.0f / sqrtf(tot / float(d) + eps);
#pragma unroll
  for (int u = 0; u < RMS_VEC; ++u) {
    const int k4 = threadIdx.x + u * blockDim.x;
    if (k4 < n4) {
      const uint2 gw = reinterpret_cast<const uint2*>(g)[k4];
      const float g0 = __uint_as_float(gw.x << 16), g1 = __uint_as_float(gw.x & 0xffff0000u);
      const float g2 = __uint_as_float(gw.y << 16), g3 = __uint_as_float(gw.y & 0xffff0000u);
      uint2 o;
      o.x = uint32_t(f32_to_bf16(v[u][0] * scale * g0)) | (uint32_t(f32_to_bf16(v[u][1] * scale * g1)) << 16);
      o.y = uint32_t(f32_to_bf16(v[u][2] * scale * g2)) | (uint32_t(f32_to_bf16(v[u][3] * scale * g3)) << 16);
      reinterpret_cast<uint2*>(h + size_t(m) * d)[k4] = o;
    }
  }
}

__device__ __forceinline__ size_t cache_index(const DecArgs& a, int layer, int b, int h, int pos, int j) {
  return ((((size_t(layer) * a.B + b) * a.H + h) * size_t(a.max_len) + pos) * a.hd) + j;
}

constexpr int ATT_KEYS = 256;   // keys per workgroup and pass (64 per wavefront)
constexpr int ATT_SPLITS_CAP = 16;   // key splits per head at most
constexpr int ATT_QMAX = 8;     // query slots per workgroup; more new positions use several query groups

// float32 -> (hi, lo) bf16 pair with hi + lo = x to about 16 significant bits.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  const bf16_t h = f32_to_bf16(x);
  hi = h;
  lo = f32_to_bf16(x - bf16_to_f32(h));
}

// Split-K decode attention of the new positions, with the merge of the splits.
// grid (H, B * NQ, S), the split outermost so that the workgroups dispatched first
// hold the most keys (split s takes blocks s, s + S, ...; a grid larger than the chip
// then doubles up the light ones on a CU, not two full ones), and a head's splits sit
// on one XCD (workgroup id % 8 = head % 8 when H is a multiple of 8).
// Workgroup (s, h, b, g) handles query slots [g*QG, g*QG + QG)
// (those below G1) of head h and the keys [256 s, 256 s + 256), then every 256 S
// further, of the len[b] + G1 keys; wavefront w takes 64 keys from 64 w of each such
// block.  Scores in base-2 units (the queries carry scale * log2 e):
//   * Q K^T on the matrix cores, 16x16x32 bf16 tiles.  The key rows are the B operand,
//     read straight from the cache (16 keys x 64 contiguous bytes per load); each
//     query is split into bf16 hi + lo parts, two products per tile, so the scores
//     keep about 16 significant bits of the float32 query.  A lane ends with the
//     scores of query rows 4 (l/16) + e, e < 4, for key l % 16 of each 16-key block.
//   * online softmax per query row with DPP reductions inside rows of 16 lanes;
//   * P V on the vector ALU: the value rows are read fully coalesced (a lane holds 8
//     dimensions of one key per load) and each lane accumulates its 8 dimensions over
//     its keys for every query; the weights and rescale factors go through LDS.
// With ``rope`` given ([row][HD/2] cos/sin of each query row's position), the queries
// are rotated as they are staged.  All loads of a block are issued before the first
// product.  The four wavefronts are
// merged in LDS and the workgroup's partial (max, sum, unnormalised output) per query
// is stored for the other workgroups of the head; the last of the S workgroups to
// finish combines them and writes the bf16 attention output.  cnt[(b*H + h)*NQ + g]
// counts the finished workgroups and is reset by the last one.  kc and vc are not
// __restrict__: a launch that appends writes cache rows its own workgroup then loads.
template <int HD, int QG>
__global__ __launch_bounds__(256) void k_attn(const float* __restrict__ q, const bf16_t* kc,
                                              const bf16_t* vc, const int* __restrict__ len,
                                              const int* __restrict__ invalid, float* __restrict__ part,
                                              bf16_t* __restrict__ out, unsigned* __restrict__ cnt, DecArgs a,
                                              int layer, int S, int NQ, float qscale,
                                              const float2* __restrict__ rope = nullptr,
                                              const float* __restrict__ knew = nullptr,
                                              const float* __restrict__ vnew = nullptr) {
  static_assert(HD == 64 || HD == 128, "head_dim 64 or 128");
  static_assert(QG >= 1 && QG <= ATT_QMAX, "query slots per workgroup");
  constexpr int KC = HD / 32;          // 32-dimension chunks of a score product
  constexpr int LPK = HD / 8;          // lanes per value row in the coalesced value loads
  constexpr int KPI = 64 / LPK;        // value rows per load
  constexpr int NV = HD / 8;           // value loads per 64 keys
  const int s = blockIdx.z, h = blockIdx.x;
  const int b = blockIdx.y / NQ, qg = blockIdx.y - b * NQ;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G1 = a.G1;
  const int q0 = qg * QG;
  const int nq = min(QG, G1 - q0);
  __shared__ u32x4 sqa[KC][2][64];                           // query hi / lo in A-operand order
  __shared__ __attribute__((aligned(16))) float sp[4][QG][64];  // weights, [r][c] order per query
  __shared__ __attribute__((aligned(16))) float scorr[4][ATT_QMAX];
  __shared__ float sm[4][QG], sl[4][QG];
  __shared__ float so[4][QG][HD];
  const size_t psz = size_t(HD + 2);
  bf16_t* outp = out + (size_t(b) * G1 + q0) * a.H * HD + size_t(h) * HD;
  const int L = len[b];
  const int nk = L + G1;
  const int g = lane >> 4, col = lane & 15;        // score layout: query rows 4g + e, key col
  const int r = lane / LPK, j = lane % LPK;        // value layout: key r of each load, dims 8j..8j+7
  const bf16_t* kbase = kc + cache_index(a, layer, b, h, 0, 0);
  const bf16_t* vbase = vc + cache_index(a, layer, b, h, 0, 0);
  // Rows past the last key are clamped to it (loaded, then masked); the clamp also
  // keeps a sequence whose new positions do not fit the cache inside it (its result
  // is discarded below).
  const int klast = max(0, min(nk, a.max_len) - 1);
  u32x4 kb[4][KC], vb[NV];
  auto load_block = [&](int k0) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
      for (int c = 0; c < KC; ++c)
        kb[blk][c] = load16(kbase + size_t(min(k0 + 16 * blk + col, klast)) * HD + 32 * c + 8 * g);
#pragma unroll
    for (int c = 0; c < NV; ++c) vb[c] = load16(vbase + size_t(min(k0 + KPI * c + r, klast)) * HD + 8 * j);
  };
  // The query loads go out first (staged below), then the first block's keys and
  // values, unconditionally (a wave without keys loads the last row), so that the
  // waits before the staging and the scores count only the loads they need.
  const int tq = threadIdx.x;                       // KC * 64 <= 256 staging threads
  const int qkc = tq >> 6, ql = tq & 63, qm = ql & 15;
  const int qd0 = 32 * qkc + 8 * (ql >> 4);
  f32x4 x0 = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, x1 = x0;
  if (tq < KC * 64) {
    const int qrow = int(b) * G1 + q0 + min(qm, nq - 1);
    const float* qr = q + size_t(qrow) * a.H * HD + size_t(h) * HD + qd0;
    x0 = *reinterpret_cast<const f32x4*>(qr);
    x1 = *reinterpret_cast<const f32x4*>(qr + 4);
    if (rope) {
      // RoPE on the query (rotate-half: dimension j pairs with j + HD/2), from the
      // cos/sin table of the row's position: the lane's 8 dimensions and their partners.
      constexpr int HALF = HD / 2;
      const bool lo_half = qd0 < HALF;
      const float* pr = qr + (lo_half ? HALF : -HALF);
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(pr), p1 = *reinterpret_cast<const f32x4*>(pr + 4);
      const float2* cs = rope + size_t(qrow) * HALF + (lo_half ? qd0 : qd0 - HALF);
      const float sg = lo_half ? -1.0f : 1.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float2 c0 = cs[e], c1 = cs[4 + e];
        x0[e] = x0[e] * c0.x + sg * (p0[e] * c0.y);
        x1[e] = x1[e] * c1.x + sg * (p1[e] * c1.y);
      }
    }
  }
  // With knew / vnew given (float32 [B * G1, H * HD], the projections of the new
  // positions) the launch also appends them: the workgroup whose key blocks hold new
  // position L + i rotates that key (RoPE from the same table as the queries), writes
  // bf16 K and V at L + i of the cache, and only then loads its keys (the barrier
  // makes its own stores visible to its loads).  Other workgroups never read them.
  bool appends = false;
  if (knew && rope && !invalid[b])
    for (int i = 0; i < G1; ++i) appends |= ((L + i) / ATT_KEYS) % S == s && L + i < a.max_len;
  if (appends) {
    constexpr int HALF = HD / 2;
    for (int t = threadIdx.x; t < G1 * HALF; t += blockDim.x) {
      const int i = t / HALF, jd = t - i * HALF, pos = L + i;
      if (((pos / ATT_KEYS) % S) != s || pos >= a.max_len) continue;
      const size_t row = (size_t(b) * G1 + i) * a.H * HD + size_t(h) * HD;
      const float2 cs = rope[(size_t(b) * G1 + i) * HALF + jd];
      const float k1 = knew[row + jd], k2 = knew[row + jd + HALF];
      bf16_t* kd = const_cast<bf16_t*>(kbase) + size_t(pos) * HD;
      bf16_t* vd = const_cast<bf16_t*>(vbase) + size_t(pos) * HD;
      kd[jd] = f32_to_bf16(k1 * cs.x - k2 * cs.y);
      kd[jd + HALF] = f32_to_bf16(k2 * cs.x + k1 * cs.y);
      vd[jd] = f32_to_bf16(vnew[row + jd]);
      vd[jd + HALF] = f32_to_bf16(vnew[row + jd + HALF]);
    }
    __syncthreads();
  }
  int k0 = s * ATT_KEYS + wave * 64;
  load_block(k0);
  __builtin_amdgcn_sched_barrier(0);
  if (invalid[b]) {   // same for every workgroup of the sequence: no counting, zero output
    if (s == 0)
      for (int t = threadIdx.x; t < nq * HD; t += blockDim.x) outp[size_t(t / HD) * a.H * HD + t % HD] = 0;
    return;
  }
  if (tq < KC * 64) {
    const float f = qm < nq ? qscale : 0.0f;
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      split_bf16(x0[e] * f, hi[e], lo[e]);
      split_bf16(x1[e] * f, hi[4 + e], lo[4 + e]);
    }
    u32x4 vh, vl;
#pragma unroll
    for (int w = 0; w < 4; ++w) { vh[w] = hi[2 * w] | (hi[2 * w + 1] << 16); vl[w] = lo[2 * w] | (lo[2 * w + 1] << 16); }
    sqa[qkc][0][ql] = vh;
    sqa[qkc][1][ql] = vl;
  }
  __syncthreads();
  float mi[4], li[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { mi[e] = -INFINITY; li[e] = 0.0f; }
  float o[QG][8];
#pragma unroll
  for (int i = 0; i < QG; ++i)
#pragma unroll
    for (int d = 0; d < 8; ++d) o[i][d] = 0.0f;
  auto process = [&](int k0) {
    f32x4 sc[4];
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) sc[blk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 ah = sqa[c][0][lane], al = sqa[c][1][lane];
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        sc[blk] = mfma16x16x32(ah, kb[blk][c], sc[blk]);
        sc[blk] = mfma16x16x32(al, kb[blk][c], sc[blk]);
      }
    }
    // online softmax; query row 4g + e sees keys <= L + q0 + 4g + e
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int qi = 4 * g + e;
      float sv[4], mloc = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const int key = k0 + 16 * blk + col;
        sv[blk] = (key < nk && key <= L + q0 + qi) ? sc[blk][e] : -INFINITY;
        mloc = fmaxf(mloc, sv[blk]);
      }
      const float mnew = fmaxf(mi[e], row16_max(mloc));
      const float corr = mi[e] == -INFINITY ? 0.0f : exp2f(mi[e] - mnew);
      float psum = 0.0f;
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) {
        const float p = sv[blk] == -INFINITY ? 0.0f : exp2f(sv[blk] - mnew);
        psum += p;
        const int kl = 16 * blk + col;
        if (qi < QG) sp[wave][qi < QG ? qi : 0][(kl % KPI) * NV + kl / KPI] = p;
      }
      li[e] = li[e] * corr + row16_sum(psum);
      mi[e] = mnew;
      if (col == 0 && qi < QG) scorr[wave][qi] = corr;
    }
    __builtin_amdgcn_wave_barrier();
    // weighted values: lane (r, j) takes key KPI c + r of load c, dimensions 8j..8j+7
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      const float cf = scorr[wave][i];
#pragma unroll
      for (int d = 0; d < 8; ++d) o[i][d] *= cf;
    }
#pragma unroll
    for (int c4 = 0; c4 < NV; c4 += 4) {
      f32x4 pw[QG];
#pragma unroll
      for (int i = 0; i < QG; ++i) pw[i] = *reinterpret_cast<const f32x4*>(&sp[wave][i][r * NV + c4]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float v[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          v[2 * w] = __uint_as_float(vb[c4 + u][w] << 16);
          v[2 * w + 1] = __uint_as_float(vb[c4 + u][w] & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < QG; ++i)
#pragma unroll
          for (int d = 0; d < 8; ++d) o[i][d] = fmaf(pw[i][u], v[d], o[i][d]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };
  // first block (loaded above), then the rest with each block's loads issued together
  if (k0 < nk) process(k0);
  for (k0 += S * ATT_KEYS; k0 < nk; k0 += S * ATT_KEYS) {
    load_block(k0);
    __builtin_amdgcn_sched_barrier(0);
    process(k0);
  }
  // sum the KPI key lanes of each dimension group, then merge the four wavefronts
#pragma unroll
  for (int x = LPK; x < 64; x <<= 1)
#pragma unroll
    for (int i = 0; i < QG; ++i)
#pragma unroll
      for (int d = 0; d < 8; ++d) o[i][d] += __shfl_xor(o[i][d], x);
  if (lane < LPK) {
#pragma unroll
    for (int i = 0; i < QG; ++i)
#pragma unroll
      for (int d = 0; d < 8; ++d) so[wave][i][8 * lane + d] = o[i][d];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int qi = 4 * g + e;
    if (col == 0 && qi < QG) { sm[wave][qi] = mi[e]; sl[wave][qi] = li[e]; }
  }
  __syncthreads();
  float* pout = part + (((size_t(b) * a.H + h) * S + s) * G1 + q0) * psz;
  for (int t = threadIdx.x; t < nq * HD; t += blockDim.x) {
    const int i = t / HD, d = t - i * HD;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm[w][i]);
    float l = 0.0f, ov = 0.0f;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        if (sm[w][i] == -INFINITY) continue;
        const float f = exp2f(sm[w][i] - M);
        l += sl[w][i] * f;
        ov += so[w][i][d] * f;
      }
    }
    float* po = pout + size_t(i) * psz;
    if (d == 0) { store_coherent(po, M); store_coherent(po + 1, l); }
    store_coherent(po + 2 + d, ov);
  }
  if (!last_workgroup(cnt + (size_t(b) * a.H + h) * NQ + qg, unsigned(S))) return;
  // last workgroup of the head: combine the S partials of every query.  The split
  // weights f_u = 2^(m_u - M) and the total l of a query are the same for all of its
  // dimensions: one thread per query computes them into LDS.  Every thread issues the
  // value loads of all its outputs first (they do not depend on the weights), so the
  // merge waits for one round of loads, then sums in split order.
  const float* pb = part + ((size_t(b) * a.H + h) * S * G1 + q0) * psz;
  __shared__ float s_f[ATT_SPLITS_CAP][ATT_QMAX], s_l[ATT_QMAX];
  constexpr int EPT = (ATT_QMAX * HD + 255) / 256;   // outputs per thread at most (256 threads)
  float pv[EPT][ATT_SPLITS_CAP];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int t = min(int(threadIdx.x) + e * int(blockDim.x), nq * HD - 1);
    const int i = t / HD, d = t - i * HD;
#pragma unroll
    for (int u = 0; u < ATT_SPLITS_CAP; ++u) pv[e][u] = pb[(size_t(min(u, S - 1)) * G1 + i) * psz + 2 + d];
  }
  if (threadIdx.x < nq) {
    const int i = threadIdx.x;
    float pm[ATT_SPLITS_CAP], pl[ATT_SPLITS_CAP];
#pragma unroll
    for (int u = 0; u < ATT_SPLITS_CAP; ++u) {
      const float* pp = pb + (size_t(min(u, S - 1)) * G1 + i) * psz;
      pm[u] = pp[0];
      pl[u] = pp[1];
    }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < ATT_SPLITS_CAP; ++u) M = fmaxf(M, pm[u]);
    float l = 0.0f;
#pragma unroll
    for (int u = 0; u < ATT_SPLITS_CAP; ++u) {
      const float f = (u >= S || M == -INFINITY || pm[u] == -INFINITY) ? 0.0f : exp2f(pm[u] - M);
      l += pl[u] * f;
      s_f[u][i] = f;
    }
    s_l[i] = l;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int t = int(threadIdx.x) + e * int(blockDim.x);
    if (t >= nq * HD) continue;
    const int i = t / HD, d = t - i * HD;
    float ov = 0.0f;
#pragma unroll
    for (int u = 0; u < ATT_SPLITS_CAP; ++u) ov += pv[e][u] * s_f[u][i];
    const float l = s_l[i];
    outp[size_t(i) * a.H * HD + d] = f32_to_bf16(l > 0.0f ? ov / l : 0.0f);
  }
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
