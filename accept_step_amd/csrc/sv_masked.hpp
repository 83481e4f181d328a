// sv_masked.hpp -- the drafter's centroid-masked LM head (gfx950).
//
// [MTP-drafters] "efficient embedder", [MTP-deep-dive] 3.4: the hidden state scores
// clusters of tokens through a table of one representative embedding per cluster; the
// top_k clusters are kept and exact logits are computed only for their member tokens.
// With ordered embeddings cluster c is the contiguous token block [c * cs, (c+1) * cs).
// Three launches: the cluster scores on the k-split product kernel (sv_head.hpp), the
// selection below (one workgroup per row), and the gathered product of the kept
// clusters' rows below.
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int MASK_MAX_CLUSTERS = 4096;   // bitonic sort of the cluster keys in LDS
constexpr int MASK_ROWS_PER_WG = 32;      // gathered token rows per workgroup (8 per wavefront)

// Orderable key of a cluster score: the float mapped to an unsigned order (-0 as +0)
// in the high word, the complemented cluster id in the low word, so that the larger
// key is the higher score, then the lower id.  Real scores never map to zero.
__device__ __forceinline__ unsigned long long cluster_key(float v, int c) {
  const unsigned u = __float_as_uint(v + 0.0f);
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(o) << 32) | (0xffffffffu - unsigned(c));
}

// Kept clusters of row blockIdx.x: the C cluster scores become keys in LDS (zeros pad
// to P, a power of two), a bitonic network sorts them in descending order, and the
// first top_k ids are written to clusters[m, 0..top_k).  256 threads.
__global__ __launch_bounds__(256) void k_select_clusters(const float* __restrict__ cl, int C, int P, int top_k,
                                                         int32_t* __restrict__ clusters) {
  __shared__ unsigned long long key[MASK_MAX_CLUSTERS];
  const int m = blockIdx.x;
  for (int i = threadIdx.x; i < P; i += blockDim.x) key[i] = i < C ? cluster_key(cl[size_t(m) * C + i], i) : 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P; i += blockDim.x) {
        const int j = i ^ stride;
        if (j > i) {
          const unsigned long long a = key[i], b = key[j];
          const bool desc = (i & size) == 0;   // this run ends up descending (all of it when size == P)
          if (desc ? a < b : a > b) { key[i] = b; key[j] = a; }
        }
      }
      __syncthreads();
    }
  }
  for (int j = threadIdx.x; j < top_k; j += blockDim.x)
    clusters[size_t(m) * top_k + j] = int32_t(0xffffffffu - unsigned(key[j]));
}

// Token logits of the kept clusters: workgroup (j, chunk, m) computes rows
// chunk * 32 .. chunk * 32 + 31 of cluster clusters[m, j] (row r = token c * cs + r):
// out[m, j * cs + r] = W[c * cs + r] . h[m].  Each group of 16 lanes takes one row, 16
// bytes per lane per step (256 contiguous bytes of the row), accumulates in float32
// and sums its 16 lanes with DPP; a wavefront takes two groups of four rows.  h is
// staged in LDS as float32.  Rows past cs read the last row and are not stored.
__global__ __launch_bounds__(256) void k_gather_logits(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                       const int32_t* __restrict__ clusters, int d, int cs, int top_k,
                                                       float* __restrict__ out) {
  extern __shared__ float sh[];
  const int j = blockIdx.x, chunk = blockIdx.y, m = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int c = __builtin_amdgcn_readfirstlane(clusters[size_t(m) * top_k + j]);
  for (int i = threadIdx.x; i < d; i += blockDim.x) sh[i] = bf16_to_f32(h[size_t(m) * d + i]);
  __syncthreads();
  const int steps = (d + 127) / 128;
#pragma unroll
  for (int grp = 0; grp < 2; ++grp) {
    const int r = chunk * MASK_ROWS_PER_WG + wave * 8 + grp * 4 + g;
    const bf16_t* wr = W + (size_t(c) * cs + min(r, cs - 1)) * d;
    float acc = 0.0f;
#pragma unroll 4
    for (int s = 0; s < steps; ++s) {
      const int k0 = s * 128 + l16 * 8;
      if (k0 < d) {
        const u32x4 v = load16(wr + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc = fmaf(__uint_as_float(v[e] << 16), sh[k0 + 2 * e], acc);
          acc = fmaf(__uint_as_float(v[e] & 0xffff0000u), sh[k0 + 2 * e + 1], acc);
        }
      }
    }
    acc = row16_sum(acc);
    if (l16 == 0 && r < cs) out[(size_t(m) * top_k + j) * cs + r] = acc;
  }
}

}  // namespace sv
