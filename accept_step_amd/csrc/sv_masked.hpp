// sv_masked.hpp -- the drafter's centroid-masked LM head (gfx950).
//
// [X-thread] "Gemma 4's MTP", efficient embedder, [MTP-deep-dive] 3.4: the hidden state scores
// clusters of tokens through a table of one representative embedding per cluster; the
// top_k clusters are kept and exact logits are computed only for their member tokens.
// With ordered embeddings cluster c is the contiguous token block [c * cs, (c+1) * cs).
// Three launches: the cluster scores on the k-split product kernel (sv_head.hpp), the
// selection below (one workgroup per row), and the gathered product of the kept
// clusters' rows below.
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int MASK_MAX_CLUSTERS = 4096;   // cluster keys of one row held in LDS / registers
constexpr int MASK_FAST_K = 64;           // top_k up to this: radix selection (else a full bitonic sort)
constexpr int MASK_ROWS_PER_WG = 16;      // gathered token rows per workgroup (4 per wavefront)

// Orderable key of a cluster score: the float mapped to an unsigned order (-0 as +0)
// in the high word, the complemented cluster id in the low word, so that the larger
// key is the higher score, then the lower id.  Real scores never map to zero.
__device__ __forceinline__ unsigned long long cluster_key(float v, int c) {
  const unsigned u = __float_as_uint(v + 0.0f);
  const unsigned o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(o) << 32) | (0xffffffffu - unsigned(c));
}

// Kept clusters of row blockIdx.x for top_k > MASK_FAST_K: the C cluster scores become
// keys in LDS (zeros pad to P, a power of two), a bitonic network sorts them in
// descending order, and the first top_k ids are written to clusters[m, 0..top_k).
// 256 threads.
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

// The k (<= MASK_FAST_K) largest of up to MASK_MAX_CLUSTERS distinct 64-bit keys held by
// a workgroup of 256 threads (thread t: key[u] of entry t + 256 u; 0 = no entry, smaller
// than every real key), left in descending order in wavefront 0's lanes (lane j: the
// j-th largest, 0 past the number of real keys).  (1) An LDS histogram of the top 12
// bits of the keys (for a float score: sign, exponent and three mantissa bits, which
// spread typical scores over many bins), scanned from the top by the four wavefronts (a
// quarter of the bins each), gives the bin B that holds the k-th largest key and the
// number ``need`` of keys still to take from it.  (2) Every key in a bin above B is
// kept; the keys of bin B are gathered in LDS and each ranks itself by counting the
// larger ones (few keys in practice; all of them in the worst case), and the ``need``
// largest are kept.  (3) Wavefront 0 sorts the kept keys with a bitonic network across
// its lanes.  Every thread of the workgroup must call it.
__device__ unsigned long long block_top_keys(const unsigned long long (&key)[MASK_MAX_CLUSTERS / 256], int k) {
  constexpr int PER = MASK_MAX_CLUSTERS / 256;
  constexpr int NBINS = 4096, SHIFT = 52, BPL = NBINS / 256;   // bins per lane in the scan
  __shared__ unsigned hist[NBINS];
  __shared__ unsigned s_bin, s_need, s_cnt, s_nb, s_nreal, s_wt[4];
  __shared__ unsigned long long s_sel[MASK_FAST_K];
  __shared__ unsigned long long s_cand[MASK_MAX_CLUSTERS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  for (int b = t; b < NBINS; b += 256) hist[b] = 0u;
  if (t == 0) { s_cnt = 0u; s_nb = 0u; s_nreal = 0u; }
  if (t < MASK_FAST_K) s_sel[t] = 0ull;
  __syncthreads();
  unsigned nreal = 0u;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (key[u]) { atomicAdd(&hist[unsigned(key[u] >> SHIFT)], 1u); ++nreal; }
  atomicAdd(&s_nreal, nreal);
  __syncthreads();
  const unsigned kk = min(unsigned(k), s_nreal);
  // wavefront w scans bins NBINS - 1 - w * NBINS / 4 downwards; lane l takes BPL of them
  const int top = NBINS - 1 - wave * (NBINS / 4) - lane * BPL;
  unsigned tot = 0u;
#pragma unroll
  for (int j = 0; j < BPL; ++j) tot += hist[top - j];
  unsigned incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned v = unsigned(__shfl_up(int(incl), off));
    if (lane >= off) incl += v;
  }
  if (lane == 63) s_wt[wave] = incl;
  __syncthreads();
  unsigned base = 0u;
  for (int w = 0; w < wave; ++w) base += s_wt[w];
  unsigned above = base + incl - tot;
  if (kk > 0u && above < kk && kk <= base + incl) {
#pragma unroll
    for (int j = 0; j < BPL; ++j) {
      const unsigned cj = hist[top - j];
      if (above < kk && kk <= above + cj) { s_bin = unsigned(top - j); s_need = kk - above; }
      above += cj;
    }
  }
  __syncthreads();
  if (kk > 0u) {
    const unsigned bin = s_bin, need = s_need, n_above = kk - need;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (!key[u]) continue;
      const unsigned kb = unsigned(key[u] >> SHIFT);
      if (kb > bin) s_sel[atomicAdd(&s_cnt, 1u)] = key[u];
      else if (kb == bin) s_cand[atomicAdd(&s_nb, 1u)] = key[u];
    }
    __syncthreads();
    const unsigned nb = s_nb;
    for (unsigned i = t; i < nb; i += 256) {
      const unsigned long long x = s_cand[i];
      unsigned rank = 0u;
      for (unsigned j = 0; j < nb; ++j) rank += s_cand[j] > x ? 1u : 0u;
      if (rank < need) s_sel[n_above + rank] = x;
    }
  }
  __syncthreads();
  unsigned long long kv = 0ull;
  if (wave == 0) {
    kv = lane < int(kk) ? s_sel[lane] : 0ull;
    for (int size = 2; size <= 64; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const unsigned lo = unsigned(__shfl_xor(int(unsigned(kv)), stride));
        const unsigned hi = unsigned(__shfl_xor(int(unsigned(kv >> 32)), stride));
        const unsigned long long other = (static_cast<unsigned long long>(hi) << 32) | lo;
        const bool desc = (lane & size) == 0;          // all of it at size 64
        const bool keep_max = ((lane & stride) == 0) == desc;
        kv = keep_max ? (other > kv ? other : kv) : (other < kv ? other : kv);
      }
    }
  }
  return kv;
}

// Kept clusters of row blockIdx.x for top_k <= MASK_FAST_K (256 threads): the keys of the
// C cluster scores through block_top_keys; wavefront 0 writes the ids.
__global__ __launch_bounds__(256) void k_select_topk(const float* __restrict__ cl, int C, int top_k,
                                                     int32_t* __restrict__ clusters) {
  constexpr int PER = MASK_MAX_CLUSTERS / 256;
  const int m = blockIdx.x, t = threadIdx.x;
  unsigned long long key[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int c = t + 256 * u;
    key[u] = c < C ? cluster_key(cl[size_t(m) * C + c], c) : 0ull;
  }
  const unsigned long long kv = block_top_keys(key, top_k);
  if (t < top_k) clusters[size_t(m) * top_k + t] = int32_t(0xffffffffu - unsigned(kv));
}

// Token logits of the kept clusters: workgroup (j, chunk, m) computes rows
// chunk * 16 .. chunk * 16 + 15 of cluster clusters[m, j] (row r = token c * cs + r):
// out[m, j * cs + r] = W[c * cs + r] . h[m].  Each group of 16 lanes takes one row, 16
// bytes per lane per step (256 contiguous bytes of the row), accumulates in float32
// and sums its 16 lanes with DPP; a wavefront takes four rows.  h is staged in LDS as
// float32.  Rows past cs read the last row and are not stored.
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
  {
    const int r = chunk * MASK_ROWS_PER_WG + wave * 4 + g;
    const bf16_t* wr = W + (size_t(c) * cs + min(r, cs - 1)) * d;
    float acc = 0.0f;
#pragma unroll 12
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
