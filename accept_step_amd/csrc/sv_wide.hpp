// sv_wide.hpp -- the LM-head product of wide verify batches (gfx950):
// out[m, v] = sum_k X[m, k] W[v, k] for M = B * (gamma + 1) up to several hundred rows.
//
// Batching many sequences into one verify step raises the arithmetic intensity of the
// head from a few FLOP per weight byte towards the matrix cores' ridge ([Self-spec]
// 1.2: the roofline argument; 4.3: the gain of speculation shrinks as the batch
// grows).  Below the ridge (about 300 rows here) the step is bound by reading W once;
// above it by the matrix cores.  So W must be read from HBM once whatever M is, and
// the MFMA work must keep its operands in registers and LDS, not in HBM.
//
// Tiling.  A workgroup (four wavefronts) computes a tile of 16 * MB rows of X (MB = 4,
// 8 or 12: up to 192 rows) by 256 rows of W over all of K.  Wavefront w owns W rows
// [64 w, 64 w + 64) of the tile (four MFMA blocks of 16 rows) and streams them chunk by
// chunk (128 k), the next chunk's loads in flight while the current one is multiplied.
// The X chunk [16 MB x 128] is shared by the four wavefronts through LDS (double-
// buffered: the next chunk is loaded into registers during the multiplication and
// stored to the other buffer after it, one barrier per chunk).  Per MFMA step (32 k) a
// wavefront reads MB X fragments from LDS and multiplies each with its four W
// fragments, so the X traffic per MFMA is a quarter fragment.
//
// W loads.  The 192-row tile loads its W fragments straight into registers in the
// operand layout: one load instruction covers 64 bytes of each of 16 rows.  The 64- and
// 128-row tiles (bound by HBM) load W in runs of 256 contiguous bytes of 4 rows per
// instruction and pass it through a wavefront-private LDS area (WL below): 477 against
// 527 us at 20 rows of the 4096-wide head, 487 against 548 at 48.  The 192-row tile
// has no LDS left for it.  (The template keeps BLK, the W blocks per wavefront, as a
// parameter: one or two blocks with longer chunks measured slower.)
//
// MFMA v_mfma_f32_16x16x32_bf16: operand A = 16 W rows x 32 k, operand B = 32 k x 16
// X rows; lane (r, g) = (lane % 16, lane / 16) holds row r and k-group g.  The k-slots
// of step j are assigned so a step's loads are contiguous per row: lane (r, g) takes
// the 16-byte piece 4 j + g of the chunk, the four lanes of a row read 64 consecutive
// bytes, two steps a 128-byte line; X in LDS uses the same assignment (row stride
// padded by 16 bytes).  The output lane (r, g) holds out[m = r][v = 4 g + e], e < 4.
//
// Batches above 192 rows take several M-tiles per W tile.  Their workgroups are
// numbered so that the M-tiles of one W tile are dispatched one after the other on
// the same XCD (workgroup b runs on XCD b mod 8): they stream the same W chunks at
// about the same time, the first from HBM and the others from that XCD's L2 (plain
// loads there; with a single M-tile the weights are read with non-temporal loads).
//
// Epilogue: the logits are stored (non-temporal: only the rows the sampler draws from
// are read again), each row's draft-token logit is stored for the acceptance rule,
// and one row-statistics partial (max, sum of exp2((l - max) c), lowest-index argmax)
// per (W tile, row) goes to part[n_tile][m].
#pragma once

#include "sv_accept.hpp"
#include "sv_device.hpp"

namespace sv {

constexpr int WIDE_MB_MAX = 12;         // 16-row blocks of X per workgroup tile (192 rows)

// A wavefront owns BLK blocks of 16 W rows (the workgroup 64 BLK rows) and takes
// 16 / BLK MFMA steps of 32 k per chunk: the same 16 loads per lane per chunk in
// flight whatever the shape, and runs of 1024 / BLK bytes of each W row per chunk.
__host__ __device__ constexpr int wide_kch(int BLK) { return 32 * (16 / BLK); }

struct WideArgs {
  const bf16_t* W;        // [N, K] row-major
  const bf16_t* X;        // [M, K] row-major
  float* out;             // [M, N] row-major, or null (statistics only)
  RowPart* part;          // [n_tiles, M] or null
  float* xlogit;          // [M] or null: logit of each row's draft token
  const int* draft;       // row m = b * (gamma + 1) + i judges draft[b * draft_stride + draft_offset + i], i < gamma
  int draft_stride, draft_offset, gamma;
  int M, N, K;
  int m_tiles, n_tiles;   // M-tiles of 16 * MB rows, W tiles of 64 * BLK rows (MB, BLK: the instantiation's)
  float c_stat;           // log2(e) / T for the sums; 0: max and argmax only
};

// The W pieces of one chunk: lane (r, g), block blk, step j: piece 4 j + g of the chunk.
template <int BLK, bool NT>
__device__ __forceinline__ void wide_load_w(const bf16_t* const (&wp)[BLK], int k0, u32x4 (&w)[BLK][16 / BLK]) {
#pragma unroll
  for (int blk = 0; blk < BLK; ++blk)
#pragma unroll
    for (int j = 0; j < 16 / BLK; ++j)
      w[blk][j] = NT ? load_stream16(wp[blk] + k0 + 32 * j) : load16(wp[blk] + k0 + 32 * j);
}

// The X chunk at k0: 16 MB rows x KCH columns in 16-byte pieces, NX per thread; piece
// u of the thread is p = tid + 256 u, row p / (KCH / 8), column group p % (KCH / 8).
// xo[u]: element offset of the piece's row (rows past the tile: a clamped row, zeroed
// when stored) and column group.
template <int MB, int BLK>
struct WideX {
  static constexpr int KCH = wide_kch(BLK), LD = KCH + 8, PPR = KCH / 8, NX = MB * KCH / 128;
};

template <int MB, int BLK>
__device__ __forceinline__ void wide_load_x(const bf16_t* X, const int (&xo)[WideX<MB, BLK>::NX], int k0,
                                            u32x4 (&xr)[WideX<MB, BLK>::NX]) {
#pragma unroll
  for (int u = 0; u < WideX<MB, BLK>::NX; ++u) xr[u] = load16(X + xo[u] + k0);
}

template <int MB, int BLK>
__device__ __forceinline__ void wide_store_x(int rows, const u32x4 (&xr)[WideX<MB, BLK>::NX], bf16_t* sx) {
  using XC = WideX<MB, BLK>;
#pragma unroll
  for (int u = 0; u < XC::NX; ++u) {
    const int p = int(threadIdx.x) + 256 * u, row = p / XC::PPR, c = p - row * XC::PPR;
    *reinterpret_cast<u32x4*>(sx + row * XC::LD + 8 * c) = row < rows ? xr[u] : u32x4{0u, 0u, 0u, 0u};
  }
}

// One chunk: 16 / BLK MFMA steps over the MB X fragments.  Fragments are read from LDS
// two (step, block) groups ahead of the BLK MFMAs that use them, and a scheduling
// barrier closes each group: left to itself the compiler hoists all of the chunk's LDS
// reads ahead of the MFMAs and runs out of registers.  xb = sx + r * LD + 8 g; fragment
// (j, mb) lies a constant offset away.
template <int MB, int BLK>
__device__ __forceinline__ u32x4 wide_xfrag(const bf16_t* xb, int q) {
  const int j = q / MB, mb = q - (q / MB) * MB;          // group q = j * MB + mb
  return *reinterpret_cast<const u32x4*>(xb + mb * 16 * WideX<MB, BLK>::LD + 32 * j);
}

template <int MB, int BLK>
__device__ __forceinline__ void wide_chunk(const u32x4 (&w)[BLK][16 / BLK], const bf16_t* xb,
                                           f32x4 (&acc)[BLK][MB]) {
  constexpr int NQ = (16 / BLK) * MB;
  u32x4 x0 = wide_xfrag<MB, BLK>(xb, 0), x1 = wide_xfrag<MB, BLK>(xb, 1 < NQ ? 1 : 0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int j = q / MB, mb = q % MB;
    u32x4 x2 = x1;
    if (q + 2 < NQ) x2 = wide_xfrag<MB, BLK>(xb, q + 2);
#pragma unroll
    for (int blk = 0; blk < BLK; ++blk) acc[blk][mb] = mfma16x16x32(w[blk][j], x0, acc[blk][mb]);
    x0 = x1;
    x1 = x2;
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- W through LDS (WL): the 64-row, four-block shape with W loaded in long runs.
// A load instruction of the register path covers 64 bytes of each of 16 rows (the MFMA
// operand layout); here instruction u of a chunk covers 256 contiguous bytes of each of
// 4 rows (lane l: row 4 u + l / 16, piece l % 16), the wavefront writes the chunk to its
// own LDS area [64 rows][WIDE_WLD] and reads the A fragments back in the operand layout.
constexpr int WIDE_WLD = 128 + 8;       // row stride of a wavefront's W chunk in LDS (elements)

template <bool NT>
__device__ __forceinline__ void wide_load_wl(const bf16_t* W, const int (&wro)[16], int k0, u32x4 (&w)[16]) {
#pragma unroll
  for (int u = 0; u < 16; ++u) w[u] = NT ? load_stream16(W + size_t(wro[u]) + k0) : load16(W + size_t(wro[u]) + k0);
}

__device__ __forceinline__ void wide_store_wl(const u32x4 (&w)[16], bf16_t* wl) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < 16; ++u)
    *reinterpret_cast<u32x4*>(wl + (4 * u + (lane >> 4)) * WIDE_WLD + 8 * (lane & 15)) = w[u];
}

// One chunk from LDS: step j's four A fragments (blocks 0-3; ab = wl + r * WIDE_WLD + 8 g)
// are read during step j - 1; X fragments two groups ahead as in wide_chunk.
template <int MB>
__device__ __forceinline__ void wide_chunk_wl(const bf16_t* ab, const bf16_t* xb, f32x4 (&acc)[4][MB]) {
  constexpr int NQ = 4 * MB;
  u32x4 ac[4], an[4];
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) ac[blk] = *reinterpret_cast<const u32x4*>(ab + 16 * blk * WIDE_WLD);
  u32x4 x0 = wide_xfrag<MB, 4>(xb, 0), x1 = wide_xfrag<MB, 4>(xb, 1 < NQ ? 1 : 0);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int j = q / MB, mb = q % MB;
    u32x4 x2 = x1;
    if (q + 2 < NQ) x2 = wide_xfrag<MB, 4>(xb, q + 2);
    if (mb == 0 && j + 1 < 4) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk)
        an[blk] = *reinterpret_cast<const u32x4*>(ab + 16 * blk * WIDE_WLD + 32 * (j + 1));
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) acc[blk][mb] = mfma16x16x32(ac[blk], x0, acc[blk][mb]);
    x0 = x1;
    x1 = x2;
    if (mb == MB - 1 && j + 1 < 4) {
#pragma unroll
      for (int blk = 0; blk < 4; ++blk) ac[blk] = an[blk];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// grid: ceil(n_tiles / 8) * 8 * m_tiles workgroups of 256 threads; M-tiles of 16 * MB
// rows, W tiles of 64 * BLK rows; dynamic LDS 2 * 16 * MB * (KCH + 8) * 2 bytes.
template <int MB, int BLK, bool NT, bool WL = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_wide(WideArgs a) {
  static_assert(!WL || BLK == 4, "W through LDS: the four-block shape");
  using XC = WideX<MB, BLK>;
  constexpr int STEPS = 16 / BLK;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  // workgroup -> (W tile, M-tile): the M-tiles of a W tile are consecutive on one XCD
  const int xcd = blockIdx.x & 7, j8 = blockIdx.x >> 3;
  const int nl = j8 / a.m_tiles, mt = j8 - nl * a.m_tiles;
  const int n_tile = nl * 8 + xcd;
  if (n_tile >= a.n_tiles) return;
  const int K = a.K, N = a.N;
  const int m0 = mt * 16 * MB;
  const int rows = min(16 * MB, a.M - m0);
  if (rows <= 0) return;
  const int vw = n_tile * 64 * BLK + wave * 16 * BLK;     // the wavefront's first W row
  const bf16_t* wp[BLK];
#pragma unroll
  for (int blk = 0; blk < BLK; ++blk) wp[blk] = a.W + size_t(min(vw + 16 * blk + r, N - 1)) * K + 8 * g;
  int xo[XC::NX];
#pragma unroll
  for (int u = 0; u < XC::NX; ++u) {
    const int p = int(threadIdx.x) + 256 * u, row = p / XC::PPR, c = p - row * XC::PPR;
    xo[u] = (m0 + min(row, rows - 1)) * K + 8 * c;
  }
  bf16_t* sx0 = reinterpret_cast<bf16_t*>(smem);
  bf16_t* sx1 = sx0 + 16 * MB * XC::LD;
  const bf16_t* xb0 = sx0 + r * XC::LD + 8 * g;
  const bf16_t* xb1 = sx1 + r * XC::LD + 8 * g;
  const int nch = K / XC::KCH;
  // WL: the wavefront's LDS area after the two X buffers, and the element offsets of its
  // 16 load rows (4 u + lane / 16, clamped) and piece (lane % 16)
  bf16_t* wl = sx1 + 16 * MB * XC::LD + wave * 64 * WIDE_WLD;
  const bf16_t* ab = wl + r * WIDE_WLD + 8 * g;
  int wro[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) wro[u] = min(vw + 4 * u + (lane >> 4), N - 1) * K + 8 * (lane & 15);

  f32x4 acc[BLK][MB];
#pragma unroll
  for (int blk = 0; blk < BLK; ++blk)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[blk][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 wa[BLK][STEPS], wb[BLK][STEPS], xr[XC::NX];
  u32x4 (&wla)[16] = reinterpret_cast<u32x4 (&)[16]>(wa);    // WL: the same registers, load-run order
  u32x4 (&wlb)[16] = reinterpret_cast<u32x4 (&)[16]>(wb);

  // chunk 0; then two chunks per iteration (K is a multiple of two chunks), the next
  // one's loads (the last iteration's clamped to the last chunk, so every load is
  // unconditional and the compiler's load counting stays exact) issued before the
  // current one is multiplied: X first, then W.  Loads complete in issue order, so the
  // store of the next X chunk waits for those X loads only and the next W chunk stays
  // in flight across the barrier (issued the other way round, every chunk's W had to
  // arrive before the next chunk's loads went out).  No exit in the middle of the
  // body: two exits would give the accumulators two sets of registers and copies
  // between them.
  wide_load_x<MB, BLK>(a.X, xo, 0, xr);
  if constexpr (WL) wide_load_wl<NT>(a.W, wro, 0, wla);
  else wide_load_w<BLK, NT>(wp, 0, wa);
  wide_store_x<MB, BLK>(rows, xr, sx0);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    const int k1 = (c + 1) * XC::KCH;
    wide_load_x<MB, BLK>(a.X, xo, k1, xr);
    if constexpr (WL) {
      wide_load_wl<NT>(a.W, wro, k1, wlb);
      wide_store_wl(wla, wl);                  // this wavefront's area: no barrier needed
      wide_chunk_wl<MB>(ab, xb0, reinterpret_cast<f32x4 (&)[4][MB]>(acc));
    } else {
      wide_load_w<BLK, NT>(wp, k1, wb);
      wide_chunk<MB, BLK>(wa, xb0, acc);
    }
    wide_store_x<MB, BLK>(rows, xr, sx1);
    __syncthreads();
    const int k2 = min(c + 2, nch - 1) * XC::KCH;
    wide_load_x<MB, BLK>(a.X, xo, k2, xr);
    if constexpr (WL) {
      wide_load_wl<NT>(a.W, wro, k2, wla);
      wide_store_wl(wlb, wl);
      wide_chunk_wl<MB>(ab, xb1, reinterpret_cast<f32x4 (&)[4][MB]>(acc));
    } else {
      wide_load_w<BLK, NT>(wp, k2, wa);
      wide_chunk<MB, BLK>(wb, xb1, acc);
    }
    wide_store_x<MB, BLK>(rows, xr, sx0);
    __syncthreads();
  }

  // ---- epilogue: logits, draft logits, row statistics over the tile's 64 BLK columns
  const bool stats = a.part != nullptr;
  const float c = a.c_stat;
  const int G1 = a.gamma + 1;
  float rm[MB], rs[MB];
  int ra[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    rm[mb] = -INFINITY; rs[mb] = 0.0f; ra[mb] = 0x7fffffff;
    const int ml = mb * 16 + r, m = m0 + ml;
    if (ml >= rows) continue;
    int xd = -1;
    if (a.xlogit) {
      const int b = m / G1, i = m - b * G1;
      if (i < a.gamma) xd = a.draft[size_t(b) * a.draft_stride + a.draft_offset + i];
    }
#pragma unroll
    for (int blk = 0; blk < BLK; ++blk) {
      const int v = vw + blk * 16 + 4 * g;
      const f32x4 val = acc[blk][mb];
      if (v >= N) continue;
      if (a.out) {
        float* o = a.out + size_t(m) * N + v;
        if (v + 3 < N && (N & 3) == 0) {
          __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(o));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < N) o[e] = val[e];
        }
      }
      if (xd >= v && xd < v + 4 && xd < N) store_coherent(a.xlogit + m, val[xd - v]);
      if (stats) {
        float tm = -INFINITY;
        int ta = 0x7fffffff;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (v + e < N && val[e] > tm) { tm = val[e]; ta = v + e; }
        float ts = 0.0f;
        if (c != 0.0f) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (v + e < N) ts += exp2f((val[e] - tm) * c);
        }
        if (ta != 0x7fffffff) merge_stat(rm[mb], rs[mb], ra[mb], tm, ts, ta, c);
      }
    }
  }
  if (!stats) return;
  // the four k-group lanes of a row, then the four wavefronts (fixed order)
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    xor_merge_stat(rm[mb], rs[mb], ra[mb], c, 16);
    xor_merge_stat(rm[mb], rs[mb], ra[mb], c, 32);
  }
  float* sm = reinterpret_cast<float*>(smem);             // the X buffers are no longer read
  float* ss = sm + 4 * 16 * MB;
  int* sa = reinterpret_cast<int*>(ss + 4 * 16 * MB);
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
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int idx = w * 16 * MB + t;
      merge_stat(m, s, am, sm[idx], ss[idx], sa[idx], c);
    }
    store_part(a.part + size_t(n_tile) * a.M + m0 + t, m, s, am);
  }
}

}  // namespace sv
