// sv_masked.hpp -- the drafter's centroid-masked LM head (gfx950).
//
// [X-thread] "Gemma 4's MTP", efficient embedder, [MTP-deep-dive] 3.4: the hidden state scores
// clusters of tokens through a table of one representative embedding per cluster; the
// top_k clusters are kept and exact logits are computed only for their member tokens.
// With ordered embeddings cluster c is the contiguous token block [c * cs, (c+1) * cs).
// Two launches: the cluster scores on the k-split product kernel (sv_head.hpp), then
// the gathered product of the kept clusters' rows below, whose workgroups each select
// their row's kept clusters first (a separate selection launch, one workgroup per row,
// above MASK_FAST_K kept clusters).
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

// LDS of block_top_keys, declared __shared__ by the calling kernel.  Between calls the
// histogram and the candidate slots are zero and nc is 0; sel_prepare establishes that
// at kernel start (no barrier needed: the selection begins with one).
constexpr int SEL_RANK_MAX = 128;                            // bin keys ranked directly
constexpr int SEL_CAND = MASK_FAST_K + SEL_RANK_MAX;         // gathered candidates, at most
struct SelScratch {
  alignas(16) unsigned hist[4096];
  alignas(16) unsigned long long cand[SEL_CAND];
  unsigned long long out[MASK_FAST_K];
  unsigned wt[4], bin, need, nb, nc;
};

__device__ __forceinline__ void sel_prepare(SelScratch& S) {
  const int t = threadIdx.x;
  reinterpret_cast<uint4*>(S.hist)[t * 4 + 0] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4*>(S.hist)[t * 4 + 1] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4*>(S.hist)[t * 4 + 2] = make_uint4(0u, 0u, 0u, 0u);
  reinterpret_cast<uint4*>(S.hist)[t * 4 + 3] = make_uint4(0u, 0u, 0u, 0u);
  if (t < SEL_CAND) S.cand[t] = 0ull;
  if (t == 0) S.nc = 0u;
}

// The k (<= MASK_FAST_K) largest of up to 256 * PER (at most MASK_MAX_CLUSTERS) distinct
// 64-bit keys held by a workgroup of 256 threads (PER per thread, in any order; 0 = no
// entry, smaller than every real key), returned in descending order in wavefront 0's
// lanes (lane j: the j-th largest, 0 past the number of real keys).  Every thread must
// call it.
//   (1) Radix refinement from the top: an LDS histogram of 12 key bits (bits 52..63
//       first: for a float score the sign, exponent and three mantissa bits) over the
//       keys that share the prefix fixed so far; a block scan from the top bin finds the
//       bin holding the k-th largest key and how many keys are still needed from it.
//       The bin joins the prefix and the next 12 bits are examined while the bin holds
//       more than SEL_RANK_MAX keys (keys are distinct, so five passes always suffice).
//       Each thread owns 16 bins of the scan and clears them once it has read them.
//   (2) Every key at or above the final prefix (at most k - 1 above it plus the bin's
//       keys) is gathered in LDS (one LDS atomic per wavefront) and ranks itself by
//       counting the larger ones in 32-key blocks; the key of rank r < k is stored at
//       position r, which leaves them sorted.
template <int PER>
__device__ unsigned long long block_top_keys(SelScratch& S, const unsigned long long (&key)[PER], int k) {
  static_assert(PER * 256 <= MASK_MAX_CLUSTERS, "more keys than the selection's candidate bound assumes");
  constexpr int NBINS = 4096, BPT = NBINS / 256;   // bins per thread in the scan
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  uint4* h4 = reinterpret_cast<uint4*>(S.hist + NBINS - BPT * (t + 1));   // bins NBINS-16(t+1) .. NBINS-16t-1
  unsigned long long prefix = 0ull, pmask = 0ull;
  unsigned need = 0u, kk = 0u;
  __syncthreads();                                   // the scratch is clear, the keys are loaded
  for (int shift = 52;; shift -= 12) {
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (key[u] && (key[u] & pmask) == prefix) atomicAdd(&S.hist[unsigned(key[u] >> shift) & 0xfffu], 1u);
    __syncthreads();
    unsigned c[BPT];
#pragma unroll
    for (int j = 0; j < BPT / 4; ++j) {
      const uint4 v = h4[j];
      c[4 * j] = v.x; c[4 * j + 1] = v.y; c[4 * j + 2] = v.z; c[4 * j + 3] = v.w;
      h4[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    unsigned tot = 0u;
#pragma unroll
    for (int j = 0; j < BPT; ++j) tot += c[j];
    unsigned incl = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned v = unsigned(__shfl_up(int(incl), off));
      if (lane >= off) incl += v;
    }
    if (lane == 63) S.wt[wave] = incl;
    __syncthreads();
    unsigned above = incl - tot;
    for (int w = 0; w < wave; ++w) above += S.wt[w];
    if (shift == 52) {
      kk = min(unsigned(k), S.wt[0] + S.wt[1] + S.wt[2] + S.wt[3]);
      need = kk;
    }
    if (kk == 0u) break;
    if (above < need && need <= above + tot) {      // exactly one thread
#pragma unroll
      for (int j = BPT - 1; j >= 0; --j) {           // c[BPT-1] is this thread's top bin
        if (above < need && need <= above + c[j]) {
          S.bin = unsigned(NBINS - BPT * (t + 1) + j);
          S.need = need - above;
          S.nb = c[j];
        }
        above += c[j];
      }
    }
    __syncthreads();
    prefix |= static_cast<unsigned long long>(S.bin) << shift;
    pmask |= 0xfffull << shift;
    need = S.need;
    if (S.nb <= unsigned(SEL_RANK_MAX) || shift == 4) break;
  }
  if (kk > 0u) {
    unsigned off[PER], pos = 0u;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const bool in = key[u] && (key[u] & pmask) >= prefix;
      const unsigned long long bal = __ballot(in);
      off[u] = pos + __builtin_amdgcn_mbcnt_hi(unsigned(bal >> 32), __builtin_amdgcn_mbcnt_lo(unsigned(bal), 0u));
      pos += unsigned(__popcll(bal));
    }
    unsigned base = 0u;
    if (pos && lane == 0) base = atomicAdd(&S.nc, pos);
    base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (key[u] && (key[u] & pmask) >= prefix) S.cand[base + off[u]] = key[u];
    __syncthreads();
    const unsigned nc = S.nc;
    if (unsigned(t) < nc) {
      const unsigned long long x = S.cand[t];
      unsigned rank = 0u;
#pragma unroll
      for (int blk = 0; blk < SEL_CAND / 32; ++blk) {
        if (unsigned(blk * 32) < nc) {
#pragma unroll
          for (int j = 0; j < 32; j += 2) {
            const ulonglong2 v = *reinterpret_cast<const ulonglong2*>(&S.cand[blk * 32 + j]);
            rank += (v.x > x ? 1u : 0u) + (v.y > x ? 1u : 0u);
          }
        }
      }
      if (rank < kk) S.out[rank] = x;
    }
  }
  __syncthreads();
  const unsigned long long r = (wave == 0 && unsigned(lane) < kk) ? S.out[lane] : 0ull;
  if (t < SEL_CAND) S.cand[t] = 0ull;               // clear for the next call (its first barrier orders this)
  if (t == 0) S.nc = 0u;
  return r;
}

// Token logits of the kept clusters: workgroup (j, chunk, m) computes rows
// chunk * 16 .. chunk * 16 + 15 of cluster clusters[m, j] (row r = token c * cs + r):
// out[m, j * cs + r] = W[c * cs + r] . h[m].  Each group of 16 lanes takes one row, 16
// bytes per lane per step (256 contiguous bytes of the row), accumulates in float32
// and sums its 16 lanes with DPP; a wavefront takes four rows.  h is staged in LDS as
// float32.  Rows past cs read the last row and are not stored.
// SELECT (top_k <= MASK_FAST_K): every workgroup selects row m's top_k clusters itself
// from the C cluster scores cl[m, 0..C) (block_top_keys: the same inputs and code in
// every workgroup, so the same ranking) and takes the j-th; workgroup (0, 0, m) also
// stores the ranking in clusters[m, 0..top_k).  This replaces a selection launch of
// its own: the saved launch outweighs the selection repeated per workgroup.  SP: cluster
// scores per thread in the selection (C <= 256 * SP; 8 for the pages' 2048 clusters,
// half the work per pass of 16).
template <bool SELECT = false, int SP = MASK_MAX_CLUSTERS / 256>
__global__ __launch_bounds__(256) void k_gather_logits(const bf16_t* __restrict__ W, const bf16_t* __restrict__ h,
                                                       int32_t* __restrict__ clusters, int d, int cs, int top_k,
                                                       float* __restrict__ out, const float* __restrict__ cl = nullptr,
                                                       int C = 0) {
  extern __shared__ float sh[];
  const int j = blockIdx.x, chunk = blockIdx.y, m = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  for (int i = threadIdx.x; i < d; i += blockDim.x) sh[i] = bf16_to_f32(h[size_t(m) * d + i]);
  int c;
  if constexpr (SELECT) {
    constexpr int PER = SP;
    __shared__ SelScratch sel;
    __shared__ int s_c;
    const int t = threadIdx.x;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int cc = t + 256 * u;
      v[u] = cc < C ? cl[size_t(m) * C + cc] : 0.0f;
    }
    sel_prepare(sel);
    unsigned long long key[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int cc = t + 256 * u;
      key[u] = cc < C ? cluster_key(v[u], cc) : 0ull;
    }
    const unsigned long long kv = block_top_keys(sel, key, top_k);   // thread t < 64: the t-th largest
    const int id = int(0xffffffffu - unsigned(kv));
    if (t == j) s_c = id;
    if (j == 0 && chunk == 0 && t < top_k) clusters[size_t(m) * top_k + t] = id;
    __syncthreads();
    c = __builtin_amdgcn_readfirstlane(s_c);
  } else {
    c = __builtin_amdgcn_readfirstlane(clusters[size_t(m) * top_k + j]);
    __syncthreads();
  }
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
