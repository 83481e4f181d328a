// sv_gemm.hpp -- weight-streaming skinny products out[m, v] = sum_k X[m, k] W[v, k]
// for the LM head and the decoder's linear layers (gfx950).
//
// The verify pass multiplies a few rows (M = B * (gamma + 1) positions) by a large
// weight matrix: arithmetic intensity is about M FLOP per weight byte, far below
// the ridge of the matrix cores, so the kernel is bound by streaming W from HBM
// once ([Self-spec] section 1.1-1.2 and [Infra-ch8] introduction: a decode-sized
// step reads all weights and barely computes; [MTP-deep-dive] 2.1).
//
// Layout of the work.  A wavefront owns a tile of 16 consecutive W rows and all
// M rows of X (in blocks of 16).  It multiplies them with
// v_mfma_f32_16x16x32_bf16: operand A = 16 W rows x 32 k, operand B = 32 k x
// 16 X rows.  The contraction order over k is free, so the k-slots of each MFMA are
// assigned to make every lane's loads contiguous: lane l (row l % 16, k-quarter
// g = l / 16) streams the contiguous quarter [g*kc/4, (g+1)*kc/4) of its W row in
// 16-byte pieces, and MFMA j takes piece j of every lane.  X is staged once per
// k-chunk in LDS with the same layout (row stride padded by 16 bytes so the 16
// lanes of a quarter hit distinct banks) and feeds operand B.
//
// Epilogue: logits are written as float32 (4 consecutive v per lane); optionally
// the running row statistics (max, sum of exp((l - max)/T), lowest-index argmax)
// are folded over the tiles a workgroup visits and written as one partial per
// (workgroup, row): the vocab-wide softmax/argmax reduction needs only a small
// merge afterwards.
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int GEMM_GRP = 8;          // 16-byte loads in flight per lane per stage

// Up to three weight matrices sharing X and K (e.g. the Q/K/V or gate/up projections)
// run as one launch: W tiles are numbered across the segments.
constexpr int MAX_SEG = 3;

struct GemmArgs {
  const bf16_t* W[MAX_SEG];   // [N_s, K] row-major (N_0 = V for the LM head)
  float* out[MAX_SEG];        // [M, N_s] row-major
  int N[MAX_SEG];
  int tile_end[MAX_SEG];      // cumulative 16-row tile counts
  int nseg;
  const bf16_t* X;       // [M, K] row-major
  RowPart* part;         // [gridDim.x, M] row-statistics partials (stats only; segment 0)
  int M, K, KC;          // KC: k-chunk staged in LDS (multiple of 32; the last chunk may be shorter)
  float c_stat;          // log2(e) / T for the sum of exponentials; 0 = argmax/max only
  int want_stats;
  int accumulate;        // out += result instead of out = result
};

// Stage X[m_base .. m_base+rows) [k0, k0+kc) into LDS rows of stride ``ld`` elements.
__device__ __forceinline__ void stage_x(const GemmArgs& a, bf16_t* sX, int ld, int m_base, int rows, int k0, int kc) {
  const int pieces = kc / 8;                  // 16-byte pieces per row
  for (int t = threadIdx.x; t < rows * pieces; t += blockDim.x) {
    int r = t / pieces, c = t - r * pieces;
    *reinterpret_cast<u32x4*>(sX + r * ld + c * 8) =
        load16(a.X + size_t(m_base + r) * a.K + k0 + c * 8);
  }
}

template <int MB>
__device__ __forceinline__ void mfma_piece(const u32x4& w, const bf16_t* sX, int ld, int rows, int r, int kofs,
                                           f32x4 (&acc)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = mb * 16 + r;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < rows) x = *reinterpret_cast<const u32x4*>(sX + row * ld + kofs);
    acc[mb] = mfma16x16x32(w, x, acc[mb]);
  }
}

// One k-chunk of one 16-row W tile: ``nsteps`` MFMA steps, loads pipelined GEMM_GRP deep.
template <int MB>
__device__ __forceinline__ void tile_chunk(const bf16_t* wq, const bf16_t* sX, int ld, int rows, int r, int xq,
                                           int nsteps, f32x4 (&acc)[MB]) {
  u32x4 bufA[GEMM_GRP], bufB[GEMM_GRP];
#pragma unroll
  for (int j = 0; j < GEMM_GRP; ++j)
    if (j < nsteps) bufA[j] = load_stream16(wq + 8 * j);
  for (int s0 = 0; s0 < nsteps; s0 += 2 * GEMM_GRP) {
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + GEMM_GRP + j < nsteps) bufB[j] = load_stream16(wq + 8 * (s0 + GEMM_GRP + j));
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + j < nsteps) mfma_piece<MB>(bufA[j], sX, ld, rows, r, xq + 8 * (s0 + j), acc);
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + 2 * GEMM_GRP + j < nsteps) bufA[j] = load_stream16(wq + 8 * (s0 + 2 * GEMM_GRP + j));
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + GEMM_GRP + j < nsteps) mfma_piece<MB>(bufB[j], sX, ld, rows, r, xq + 8 * (s0 + GEMM_GRP + j), acc);
  }
}

// grid.x: workgroups striding over W tiles; grid.y: blocks of 16*MB rows of X.
// Dynamic LDS: min(16*MB, M - m_base) rows x (KC + 8) bf16, at least the statistics
// scratch (WAVES * 16 * MB * 12 bytes).
template <int MB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_bf16(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sX = reinterpret_cast<bf16_t*>(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m_base = blockIdx.y * MB * 16;
  const int rows = min(MB * 16, a.M - m_base);
  const int ld = a.KC + 8;
  const int ntiles = a.tile_end[a.nseg - 1];
  const int nblk = (ntiles + WAVES - 1) / WAVES;
  const bool one_chunk = a.KC >= a.K;

  float rm[MB], rs[MB];
  int ra[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) { rm[mb] = -INFINITY; rs[mb] = 0.0f; ra[mb] = 0x7fffffff; }

  if (one_chunk) {
    stage_x(a, sX, ld, m_base, rows, 0, a.K);
    __syncthreads();
  }
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int tile = blk * WAVES + wave;
    const bool live = tile < ntiles;
    int seg = 0;
#pragma unroll
    for (int q = 0; q < MAX_SEG - 1; ++q) seg += (q + 1 < a.nseg && tile >= a.tile_end[q]) ? 1 : 0;
    const int N = a.N[seg];
    const int v0 = (tile - (seg ? a.tile_end[seg - 1] : 0)) * 16;
    const bf16_t* Wseg = a.W[seg];
    float* outseg = a.out[seg];
    const int vrow = min(v0 + r, N - 1);
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < a.K; k0 += a.KC) {
      const int kc = min(a.KC, a.K - k0);
      if (!one_chunk) {
        __syncthreads();
        stage_x(a, sX, ld, m_base, rows, k0, kc);
        __syncthreads();
      }
      if (live) {
        const int xq = g * (kc / 4);
        tile_chunk<MB>(Wseg + size_t(vrow) * a.K + k0 + xq, sX, ld, rows, r, xq, kc / 32, acc);
      }
    }
    if (!live) continue;
    // lane holds out[m = m_base + mb*16 + r][v = v0 + 4g + e], e = 0..3
    const int vb = v0 + 4 * g;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m_base + mb * 16 + r;
      if (mb * 16 + r >= rows) continue;
      float* o = outseg + size_t(m) * N + vb;
      float val[4] = {acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]};
      if (vb + 3 < N && (N & 3) == 0) {
        f32x4 v4 = acc[mb];
        if (a.accumulate) {
          f32x4 old = *reinterpret_cast<const f32x4*>(o);
          v4 += old;
        }
        *reinterpret_cast<f32x4*>(o) = v4;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (vb + e < N) o[e] = a.accumulate ? o[e] + val[e] : val[e];
      }
      if (a.want_stats) {
        float tm = -INFINITY;
        int ta = 0x7fffffff;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (vb + e < N && val[e] > tm) { tm = val[e]; ta = vb + e; }
        float ts = 0.0f;
        if (a.c_stat != 0.0f) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (vb + e < N) ts += exp2f((val[e] - tm) * a.c_stat);
        }
        if (ta != 0x7fffffff) merge_stat(rm[mb], rs[mb], ra[mb], tm, ts, ta, a.c_stat);
      }
    }
  }
  if (!a.want_stats) return;
  // reduce over the four k-quarter lane groups, then over the waves
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    for (int o = 16; o < 64; o <<= 1) {
      float m2 = __shfl_xor(rm[mb], o), s2 = __shfl_xor(rs[mb], o);
      int a2 = __shfl_xor(ra[mb], o);
      merge_stat(rm[mb], rs[mb], ra[mb], m2, s2, a2, a.c_stat);
    }
  }
  __syncthreads();   // LDS reuse
  float* sm = reinterpret_cast<float*>(smem);
  float* ss = sm + WAVES * 16 * MB;
  int* sa = reinterpret_cast<int*>(ss + WAVES * 16 * MB);
  if (g == 0) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int idx = wave * 16 * MB + mb * 16 + r;
      sm[idx] = rm[mb]; ss[idx] = rs[mb]; sa[idx] = ra[mb];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < rows; t += blockDim.x) {
    float m = -INFINITY, s = 0.0f;
    int am = 0x7fffffff;
    for (int w = 0; w < WAVES; ++w) {
      const int idx = w * 16 * MB + t;
      merge_stat(m, s, am, sm[idx], ss[idx], sa[idx], a.c_stat);
    }
    RowPart p;
    p.m = m; p.s = s; p.a = am; p.pad = 0;
    a.part[size_t(blockIdx.x) * a.M + m_base + t] = p;
  }
}

// float32 LM head (small tables only): one thread per W row, X in LDS.
// grid.x = ceil(N / 256); dynamic LDS = M * K floats.
__global__ __launch_bounds__(256) void k_gemm_f32(const float* __restrict__ W, const float* __restrict__ X,
                                                  float* __restrict__ out, RowPart* __restrict__ part,
                                                  int M, int N, int K, float c_stat, int want_stats) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sX = reinterpret_cast<float*>(smem);
  for (int t = threadIdx.x; t < M * K; t += blockDim.x) sX[t] = X[t];
  __syncthreads();
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __shared__ float sm[4], ss[4];
  __shared__ int sa[4];
  for (int m = 0; m < M; ++m) {
    float acc = 0.0f;
    if (v < N) {
      const float* w = W + size_t(v) * K;
      const float* x = sX + m * K;
      for (int k = 0; k < K; ++k) acc = fmaf(x[k], w[k], acc);
      out[size_t(m) * N + v] = acc;
    }
    if (!want_stats) continue;
    float rm = v < N ? acc : -INFINITY, rs = v < N && c_stat != 0.0f ? 1.0f : 0.0f;
    int ra = v < N ? v : 0x7fffffff;
    wave_merge_stat(rm, rs, ra, c_stat);
    __syncthreads();
    if (lane == 0) { sm[wave] = rm; ss[wave] = rs; sa[wave] = ra; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float M0 = -INFINITY, S0 = 0.0f;
      int A0 = 0x7fffffff;
      for (int w = 0; w < 4; ++w) merge_stat(M0, S0, A0, sm[w], ss[w], sa[w], c_stat);
      RowPart p;
      p.m = M0; p.s = S0; p.a = A0; p.pad = 0;
      part[size_t(blockIdx.x) * M + m] = p;
    }
  }
}

}  // namespace sv
