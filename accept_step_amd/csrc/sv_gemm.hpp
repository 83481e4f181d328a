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
// 16 X rows.  Lane l holds row l % 16 and k-group g = l / 16 (8 values).  The
// contraction order over k is free, so the k-slots of MFMA step j are assigned to
// make the loads of one step contiguous per row: lane (r, g) takes the 16-byte piece
// 4j + g of its row, so the four lanes of a row read 64 consecutive bytes and two
// steps cover a 128-byte line.  X is staged once per k-chunk in LDS (row stride
// padded by 16 bytes so the 16 lanes of a k-group hit distinct banks) and feeds
// operand B with the same piece assignment.
//
// Epilogue: logits are written as float32 (4 consecutive v per lane); optionally
// the running row statistics (max, sum of exp((l - max)/T), lowest-index argmax)
// are folded over the tiles a workgroup visits and written as one partial per
// (workgroup, row): the vocab-wide softmax/argmax reduction needs only a small
// merge afterwards.
#pragma once

#include "sv_accept.hpp"
#include "sv_device.hpp"

namespace sv {

constexpr int GEMM_GRP = 8;          // 16-byte loads in flight per lane per stage

// Up to three weight matrices sharing X and K (e.g. the Q/K/V or gate/up projections)
// run as one launch: W tiles are numbered across the segments.
constexpr int MAX_SEG = 3;

struct GemmArgs;
__device__ __forceinline__ int seg_of(const GemmArgs& a, int tile);

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
  unsigned* counter;     // non-null: the last workgroup to finish runs the acceptance
  AcceptArgs acc;        // ... for all acc.B sequences (acc.B * (gamma + 1) <= ACC_MAX_ROWS)
  float* xlogit;         // non-null: logit of each row's draft token (row m = b*(gamma+1)+i, i < gamma)
};

// Draft token judged by row m (slot i of sequence b), -1 for the bonus slot.
__device__ __forceinline__ int row_draft(const GemmArgs& a, int m) {
  if (!a.xlogit || m >= a.M) return -1;
  const int G1 = a.acc.gamma + 1;
  const int b = m / G1, i = m - b * G1;
  if (i >= a.acc.gamma) return -1;
  return a.acc.draft[size_t(b) * a.acc.draft_stride + a.acc.draft_offset + i];
}

// Segment of a tile and its fields, selected without indexing the argument arrays by
// a runtime value (which would turn into memory loads and waits in the hot loop).
__device__ __forceinline__ int seg_of(const GemmArgs& a, int tile) {
  return (a.nseg > 1 && tile >= a.tile_end[0]) ? ((a.nseg > 2 && tile >= a.tile_end[1]) ? 2 : 1) : 0;
}
template <class T>
__device__ __forceinline__ T pick(int seg, T x0, T x1, T x2) { return seg == 0 ? x0 : (seg == 1 ? x1 : x2); }

struct TileRef {
  const bf16_t* W;
  float* out;
  int N, v0;
};

__device__ __forceinline__ TileRef tile_ref(const GemmArgs& a, int tile) {
  const int seg = seg_of(a, tile);
  TileRef t;
  t.W = pick(seg, a.W[0], a.W[1], a.W[2]);
  t.out = pick(seg, a.out[0], a.out[1], a.out[2]);
  t.N = pick(seg, a.N[0], a.N[1], a.N[2]);
  t.v0 = (tile - pick(seg, 0, a.tile_end[0], a.tile_end[1])) * 16;
  return t;
}

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
// ``wq`` points at piece g of the lane's row within the chunk, ``xq`` = 8 * g; step j
// reads 32 * j elements further.
template <int MB>
__device__ __forceinline__ void tile_chunk(const bf16_t* wq, const bf16_t* sX, int ld, int rows, int r, int xq,
                                           int nsteps, f32x4 (&acc)[MB]) {
  u32x4 bufA[GEMM_GRP], bufB[GEMM_GRP];
#pragma unroll
  for (int j = 0; j < GEMM_GRP; ++j)
    if (j < nsteps) bufA[j] = load16(wq + 32 * j);
  for (int s0 = 0; s0 < nsteps; s0 += 2 * GEMM_GRP) {
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + GEMM_GRP + j < nsteps) bufB[j] = load16(wq + 32 * (s0 + GEMM_GRP + j));
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + j < nsteps) mfma_piece<MB>(bufA[j], sX, ld, rows, r, xq + 32 * (s0 + j), acc);
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + 2 * GEMM_GRP + j < nsteps) bufA[j] = load16(wq + 32 * (s0 + 2 * GEMM_GRP + j));
#pragma unroll
    for (int j = 0; j < GEMM_GRP; ++j)
      if (s0 + GEMM_GRP + j < nsteps) mfma_piece<MB>(bufB[j], sX, ld, rows, r, xq + 32 * (s0 + GEMM_GRP + j), acc);
  }
}

// Store one finished 16-row tile (4 consecutive outputs per lane) and fold it into
// the lane's running row statistics.
template <int MB>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& a, const f32x4 (&acc)[MB], float* outseg, int N, int v0,
                                              int m_base, int rows, int r, int g, float (&rm)[MB], float (&rs)[MB],
                                              int (&ra)[MB], const int (&xd)[MB]) {
  // lane holds out[m = m_base + mb*16 + r][v = v0 + 4g + e], e = 0..3
  const int vb = v0 + 4 * g;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = m_base + mb * 16 + r;
    if (mb * 16 + r >= rows) continue;
    float* o = outseg + size_t(m) * N + vb;
    float val[4] = {acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]};
    if (vb + 3 < N && (N & 3) == 0) {
      *reinterpret_cast<f32x4*>(o) = acc[mb];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (vb + e < N) o[e] = val[e];
    }
    if (xd[mb] >= vb && xd[mb] < vb + 4 && xd[mb] < N) store_coherent(a.xlogit + m, val[xd[mb] - vb]);
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

// Reduce the running statistics over the four k-group lanes and the wavefronts and
// write one partial per (workgroup, row).  LDS is reused (a barrier comes first).
template <int MB, int WAVES>
__device__ __forceinline__ void stats_tail(const GemmArgs& a, unsigned char* smem, int m_base, int rows, int g, int r,
                                           int wave, float (&rm)[MB], float (&rs)[MB], int (&ra)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    for (int o = 16; o < 64; o <<= 1) {
      float m2 = __shfl_xor(rm[mb], o), s2 = __shfl_xor(rs[mb], o);
      int a2 = __shfl_xor(ra[mb], o);
      merge_stat(rm[mb], rs[mb], ra[mb], m2, s2, a2, a.c_stat);
    }
  }
  __syncthreads();
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
    store_part(a.part + size_t(blockIdx.x) * a.M + m_base + t, m, s, am);
  }
}

// General path (any K % 32 == 0, X staged chunk by chunk).
// grid.x: workgroups striding over W tiles; grid.y: blocks of 16*MB rows of X.
// Dynamic LDS: min(16*MB, M - m_base) rows x (KC + 8) bf16, at least the statistics
// scratch (WAVES * 16 * MB * 12 bytes).
template <int MB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_chunked(GemmArgs a) {
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
  int ra[MB], xd[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    rm[mb] = -INFINITY; rs[mb] = 0.0f; ra[mb] = 0x7fffffff;
    xd[mb] = row_draft(a, m_base + mb * 16 + r);
  }

  if (one_chunk) {
    stage_x(a, sX, ld, m_base, rows, 0, a.K);
    __syncthreads();
  }
  for (int blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int tile = blk * WAVES + wave;
    const bool live = tile < ntiles;
    const TileRef tr = tile_ref(a, min(tile, ntiles - 1));
    const int N = tr.N, v0 = tr.v0;
    const bf16_t* Wseg = tr.W;
    float* outseg = tr.out;
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
      if (live) tile_chunk<MB>(Wseg + size_t(vrow) * a.K + k0 + 8 * g, sX, ld, rows, r, 8 * g, kc / 32, acc);
    }
    if (!live) continue;
    tile_epilogue<MB>(a, acc, outseg, N, v0, m_base, rows, r, g, rm, rs, ra, xd);
  }
  if (a.want_stats) stats_tail<MB, WAVES>(a, smem, m_base, rows, g, r, wave, rm, rs, ra);
  if (a.counter && last_workgroup(a.counter, gridDim.x * gridDim.y)) accept_block(a.acc, 0, a.acc.B);
}


// Streaming path: K % (32 * GEMM_GRP) == 0 and all of X (its 16*MB-row block) in LDS.
// Each wavefront walks a flat stream of work items (tile, group of GEMM_GRP k-steps)
// over its tiles; the loads of item k+1 are issued before item k is multiplied, across
// tile boundaries, so the load pipeline never drains and no per-step guard breaks the
// compiler's load counting.  No load is issued that is not consumed.
struct StreamCtx {
  int gpt;       // work items per tile
  int first;     // first tile of this wavefront
  int tstride;   // tile stride between its work items' tiles
};

__device__ __forceinline__ const bf16_t* stream_item_ptr(const GemmArgs& a, const StreamCtx& c, int k, int r, int g) {
  const int i = k / c.gpt, gg = k - i * c.gpt;
  const TileRef tr = tile_ref(a, c.first + i * c.tstride);
  const int vrow = min(tr.v0 + r, tr.N - 1);
  return tr.W + size_t(vrow) * a.K + 8 * g + gg * (GEMM_GRP * 32);
}

__device__ __forceinline__ void stream_load(const bf16_t* p, u32x4 (&buf)[GEMM_GRP]) {
#pragma unroll
  for (int j = 0; j < GEMM_GRP; ++j) buf[j] = load16(p + 32 * j);
}

template <int MB>
__device__ __forceinline__ void stream_compute(const GemmArgs& a, const StreamCtx& c, int k, const u32x4 (&buf)[GEMM_GRP],
                                               const bf16_t* sX, int ld, int rows, int r, int g, int m_base,
                                               f32x4 (&acc)[MB], float (&rm)[MB], float (&rs)[MB], int (&ra)[MB],
                                               const int (&xd)[MB]) {
  const int i = k / c.gpt, gg = k - i * c.gpt;
  const int kofs = 8 * g + gg * (GEMM_GRP * 32);
#pragma unroll
  for (int j = 0; j < GEMM_GRP; ++j) mfma_piece<MB>(buf[j], sX, ld, rows, r, kofs + 32 * j, acc);
  if (gg == c.gpt - 1) {
    const TileRef tr = tile_ref(a, c.first + i * c.tstride);
    tile_epilogue<MB>(a, acc, tr.out, tr.N, tr.v0, m_base, rows, r, g, rm, rs, ra, xd);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int MB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_gemm_stream(GemmArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sX = reinterpret_cast<bf16_t*>(smem);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m_base = blockIdx.y * MB * 16;
  const int rows = min(MB * 16, a.M - m_base);
  const int ld = a.K + 8;
  const int ntiles = a.tile_end[a.nseg - 1];

  float rm[MB], rs[MB];
  int ra[MB], xd[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    rm[mb] = -INFINITY; rs[mb] = 0.0f; ra[mb] = 0x7fffffff;
    xd[mb] = row_draft(a, m_base + mb * 16 + r);
  }

  stage_x(a, sX, ld, m_base, rows, 0, a.K);
  __syncthreads();

  // this wave's tiles: (blockIdx.x + i * gridDim.x) * WAVES + wave, i = 0 .. n_my - 1
  StreamCtx c;
  c.gpt = a.K / (32 * GEMM_GRP);
  c.first = blockIdx.x * WAVES + wave;
  c.tstride = gridDim.x * WAVES;
  const int n_my = c.first < ntiles ? (ntiles - 1 - c.first) / c.tstride + 1 : 0;
  const int items = n_my * c.gpt;
  if (items > 0) {
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 bufA[GEMM_GRP], bufB[GEMM_GRP];
    // steady state over pairs while a third item exists, then one or two peeled items
    stream_load(stream_item_ptr(a, c, 0, r, g), bufA);
    int k = 0;
    for (; k + 2 < items; k += 2) {
      stream_load(stream_item_ptr(a, c, k + 1, r, g), bufB);
      stream_compute<MB>(a, c, k, bufA, sX, ld, rows, r, g, m_base, acc, rm, rs, ra, xd);
      stream_load(stream_item_ptr(a, c, k + 2, r, g), bufA);
      stream_compute<MB>(a, c, k + 1, bufB, sX, ld, rows, r, g, m_base, acc, rm, rs, ra, xd);
    }
    if (k + 1 < items) {
      stream_load(stream_item_ptr(a, c, k + 1, r, g), bufB);
      stream_compute<MB>(a, c, k, bufA, sX, ld, rows, r, g, m_base, acc, rm, rs, ra, xd);
      stream_compute<MB>(a, c, k + 1, bufB, sX, ld, rows, r, g, m_base, acc, rm, rs, ra, xd);
    } else {
      stream_compute<MB>(a, c, k, bufA, sX, ld, rows, r, g, m_base, acc, rm, rs, ra, xd);
    }
  }
  if (a.want_stats) stats_tail<MB, WAVES>(a, smem, m_base, rows, g, r, wave, rm, rs, ra);
  if (a.counter && last_workgroup(a.counter, gridDim.x * gridDim.y)) accept_block(a.acc, 0, a.acc.B);
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
      store_part(part + size_t(blockIdx.x) * M + m, M0, S0, A0);
    }
  }
}

}  // namespace sv
